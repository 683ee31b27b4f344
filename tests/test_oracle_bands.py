"""Pins of the oracle's rounding-decision bands (CPU only).

A bf16-storage layer rounds every stored activation to bfloat16.  Two correct
float32-accumulating implementations may sum in different orders, land on
opposite sides of a rounding midpoint and store values one bf16 spacing apart;
the oracle's ``rounding_bands`` bounds that per element.  These tests pin the
bands to things other than the oracle: torch's own bfloat16 conversion, the
float32 products of numpy and torch in several summation orders, and a whole
float32 evaluation of the layer (tests/standin.py, at the same rounding
points) that must land inside the bands element by element.  The bands are
capped at two bf16 spacings, so they stay tight where the first-order bound
would grow; the float32 evaluation landing inside them shows the cap holds.
"""
import numpy as np
import pytest
import torch

from moe_workloads import MoEConfig, make_inputs
from oracle import moe_oracle as O
from tests.standin import float32_layer


def _bf16(a):
    """Round to bfloat16 with torch's conversion (round to nearest even)."""
    return torch.as_tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def test_bf16_flip_covers_every_input_in_the_interval():
    rng = np.random.default_rng(1)
    pre = rng.standard_normal(4000) * np.exp2(rng.integers(-10, 10, 4000))
    rounded = _bf16(pre)
    spacing = np.abs(rounded) * 2.0 ** -7
    sigma = spacing * rng.uniform(0.0, 0.8, 4000)
    band = O.bf16_flip(pre, rounded, sigma)
    for t in np.linspace(-1.0, 1.0, 33):
        dev = np.abs(_bf16(pre + t * sigma) - rounded)
        assert np.all(dev <= band), "a rounding inside the interval leaves the band"
        # where the band is zero, every input in the interval rounds alike
        assert np.all(dev[band == 0] == 0)
    # the band is not vacuous: most intervals do not reach a midpoint
    assert 0.2 < np.mean(band == 0) < 0.98


@pytest.mark.parametrize("n", [1, 7, 128, 1000])
def test_gemm_sigma_bounds_float32_sums_in_any_order(n):
    rng = np.random.default_rng(n)
    a = _bf16(rng.standard_normal((16, n)))
    b = _bf16(rng.standard_normal((n, 24)) / np.sqrt(n))
    exact = a @ b
    sig = O.gemm_sigma(a, b)
    prods = (a[:, :, None] * b[None, :, :]).astype(np.float32)     # exact: bf16 x bf16 fits float32
    orders = [np.arange(n), np.arange(n)[::-1], rng.permutation(n)]
    for o in orders:
        acc = np.zeros((16, 24), np.float32)
        for k in o:
            acc = acc + prods[:, k, :]
        assert np.all(np.abs(acc.astype(np.float64) - exact) <= sig)
    t32 = (torch.tensor(a, dtype=torch.float32) @ torch.tensor(b, dtype=torch.float32)).double().numpy()
    assert np.all(np.abs(t32 - exact) <= sig)


@pytest.mark.parametrize("cfg", [MoEConfig("b_small", N=160, H=128, F=128, E=5, K=2, dtype="bf16"),
                                 MoEConfig("b_bias", N=96, H=256, F=128, E=8, K=3, dtype="bf16",
                                           zipf_s=1.2, zipf_tau=1.25)], ids=lambda c: c.name)
def test_rounding_bands_cover_a_float32_evaluation(cfg):
    inp = {k: (None if v is None else O.as_f64(v)) for k, v in make_inputs(cfg, 3, with_dy=True).items()}
    fwd = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.K, bias=inp["bias"],
                    store="bf16")
    bwd = O.backward(fwd, inp["dy"])
    band = O.rounding_bands(fwd, bwd, inp["dy"], cap=False)
    capped = O.rounding_bands(fwd, bwd, inp["dy"])
    alt = float32_layer(inp, fwd, cfg.K)
    ref = dict(fwd)
    ref.update(bwd)
    flips = 0
    assert set(band) == set(capped) == {"G", "U", "A", "ys", "y", "dys", "dG", "dU", "dxs", "dx"}
    for k in band:
        a = alt[k]
        r = np.asarray(ref[k], dtype=np.float64).reshape(a.shape)
        dev = np.abs(a - r)
        # the first-order bound alone covers every deviation ...
        b = np.asarray(band[k]).reshape(a.shape)
        bad = dev > b
        assert not bad.any(), f"{k}: {int(bad.sum())} elements leave the band, worst {float((dev - b).max()):.3g}"
        # ... and so does the capped band with the 2e-2 absolute tolerance, as the parity checks use it
        c = np.asarray(capped[k]).reshape(a.shape)
        assert np.all(c <= b) and np.all(dev <= 2e-2 + c), k
        flips += int(np.sum(dev > 0))
    # the float32 evaluation does differ from the oracle, so the check has teeth
    assert flips > 0
