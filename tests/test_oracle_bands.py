"""Pins of the oracle's rounding-decision bands (CPU only).

A bf16-storage layer rounds every stored activation to bfloat16.  Two correct
float32-accumulating implementations may sum in different orders, land on
opposite sides of a rounding midpoint and store values one bf16 spacing apart;
the oracle's ``rounding_bands`` bounds that per element.  These tests pin the
bands to things other than the oracle: torch's own bfloat16 conversion, the
float32 products of numpy and torch in several summation orders, and a whole
float32 evaluation of the layer (written here, at the same rounding points)
that must land inside the bands element by element.
"""
import numpy as np
import pytest
import torch

from moe_workloads import MoEConfig, make_inputs
from oracle import moe_oracle as O


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


def _float32_layer(inp, fwd, K):
    """The layer in float32 at the oracle's rounding points, given the
    oracle's assignment (torch float32 matmuls: another summation order)."""
    f = lambda a: torch.tensor(np.asarray(a), dtype=torch.float32)
    rb = lambda t: t.to(torch.bfloat16).to(torch.float32)
    x, w_r = f(inp["x"]), f(inp["w_r"])
    wg, wu, wd, dy = f(inp["w_gate"]), f(inp["w_up"]), f(inp["w_down"]), f(inp["dy"])
    N, H = x.shape
    E = w_r.shape[1]
    sf = torch.tensor(fwd["sorted_flat"], dtype=torch.int64)
    inv = torch.tensor(fwd["inv"], dtype=torch.int64).view(N, K)
    off = [int(v) for v in fwd["offsets"]]
    gates = f(fwd["gates"])
    tok = sf // K
    xs = x[tok]
    NK, F = N * K, wg.shape[2]
    G, U, A, ys = (torch.zeros(NK, F), torch.zeros(NK, F), torch.zeros(NK, F), torch.zeros(NK, H))
    for e in range(E):
        s = slice(off[e], off[e + 1])
        G[s] = rb(xs[s] @ wg[e])
        U[s] = rb(xs[s] @ wu[e])
        A[s] = rb(torch.nn.functional.silu(G[s]) * U[s])
        ys[s] = rb(A[s] @ wd[e])
    y = rb(sum(gates[:, k:k + 1] * ys[inv[:, k]] for k in range(K)))
    grow = gates.reshape(-1)[sf][:, None]
    dys = rb(grow * dy[tok])
    dgates = torch.stack([(dy * ys[inv[:, k]]).sum(1) for k in range(K)], 1)
    dG, dU, dxs = torch.zeros(NK, F), torch.zeros(NK, F), torch.zeros(NK, H)
    dwg, dwu, dwd = torch.zeros_like(wg), torch.zeros_like(wu), torch.zeros_like(wd)
    for e in range(E):
        s = slice(off[e], off[e + 1])
        dA = dys[s] @ wd[e].T
        sg = torch.sigmoid(G[s])
        dG[s] = rb(dA * U[s] * sg * (1 + G[s] * (1 - sg)))
        dU[s] = rb(dA * G[s] * sg)
        dxs[s] = rb(dG[s] @ wg[e].T + dU[s] @ wu[e].T)
        dwg[e] = xs[s].T @ dG[s]
        dwu[e] = xs[s].T @ dU[s]
        dwd[e] = A[s].T @ dys[s]
    dl_sel = gates * (dgates - (gates * dgates).sum(1, keepdim=True))
    dlogits = torch.zeros(N, E).scatter_(1, torch.tensor(fwd["topk"], dtype=torch.int64), dl_sel)
    dw_r = x.T @ dlogits
    dx = rb(sum(dxs[inv[:, k]] for k in range(K)) + dlogits @ w_r.T)
    out = dict(G=G, U=U, A=A, ys=ys, y=y, dys=dys, dgates=dgates, dG=dG, dU=dU, dxs=dxs, dw_gate=dwg, dw_up=dwu,
               dw_down=dwd, dlogits=dlogits, dw_r=dw_r, dx=dx)
    return {k: v.double().numpy() for k, v in out.items()}


@pytest.mark.parametrize("cfg", [MoEConfig("b_small", N=160, H=128, F=128, E=5, K=2, dtype="bf16"),
                                 MoEConfig("b_bias", N=96, H=256, F=128, E=8, K=3, dtype="bf16",
                                           zipf_s=1.2, zipf_tau=1.25)], ids=lambda c: c.name)
def test_rounding_bands_cover_a_float32_evaluation(cfg):
    inp = {k: (None if v is None else O.as_f64(v)) for k, v in make_inputs(cfg, 3, with_dy=True).items()}
    fwd = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.K, bias=inp["bias"],
                    store="bf16")
    bwd = O.backward(fwd, inp["dy"])
    band = O.rounding_bands(fwd, bwd, inp["dy"])
    alt = _float32_layer(inp, fwd, cfg.K)
    ref = dict(fwd)
    ref.update(bwd)
    flips = 0
    for k, a in alt.items():
        r = np.asarray(ref[k], dtype=np.float64).reshape(a.shape)
        b = np.asarray(band[k]).reshape(a.shape)
        dev = np.abs(a - r)
        bad = dev > b
        assert not bad.any(), f"{k}: {int(bad.sum())} elements leave the band, worst {float((dev - b).max()):.3g}"
        flips += int(np.sum(dev > 0))
    # the float32 evaluation does differ from the oracle, so the check has teeth
    assert flips > 0
