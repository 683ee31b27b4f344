"""Pins of the oracle's token-dropping capacity variant (CPU only).

Expert capacity C ("MoE computation principle and execution process",
section 3.4): each expert processes at most C of its rows, the overflow is
dropped.  Reading: the kept rows of an expert are its first C in the stable
expert-grouped order (lowest flat index n*K + k first); a dropped slot adds
nothing to y and its gate is not renormalised away.

Pinned by: a brute-force keep rule that counts earlier slots of the same
expert and evaluates each token on its own; metadata invariants; the special
cases C >= max count (the dropless layer) and C = 0 (nothing computed);
torch autograd of an independent dense formulation with the keep mask fixed;
and a planted mistake (keeping the last C rows) that the pins must catch.
"""
import numpy as np
import pytest
import torch

from moe_workloads import MoEConfig, make_inputs
from oracle import moe_oracle as O

CFGS = [MoEConfig("c_skew", N=48, H=64, F=32, E=6, K=2, dtype="f32", zipf_s=1.2, zipf_tau=1.5),
        MoEConfig("c_k3", N=40, H=64, F=32, E=5, K=3, dtype="f32")]


def _inputs(cfg, seed):
    return {k: (None if v is None else O.as_f64(v)) for k, v in make_inputs(cfg, seed, with_dy=True).items()}


def _fwd(inp, K, capacity, store="f64"):
    return O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], K, bias=inp["bias"],
                     store=store, capacity=capacity)


def _kept_bruteforce(topk, C):
    """Slot (n, k) is kept when fewer than C earlier slots (flat order) went
    to the same expert."""
    flat = topk.reshape(-1)
    kept = np.zeros(flat.size, dtype=bool)
    for f in range(flat.size):
        kept[f] = int(np.sum(flat[:f] == flat[f])) < C
    return kept.reshape(topk.shape)


def _ffn(v, wg, wu, wd):
    g = v @ wg
    return ((g / (1.0 + np.exp(-g))) * (v @ wu)) @ wd


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
@pytest.mark.parametrize("cf", [0.5, 1.0, 1.25])
def test_output_matches_bruteforce_keep_rule(cfg, cf):
    inp = _inputs(cfg, 1)
    C = O.capacity_of(cfg.N, cfg.K, cfg.E, cf)
    f = _fwd(inp, cfg.K, C)
    kept = _kept_bruteforce(f["topk"], C)
    assert np.array_equal(f["inv"].reshape(cfg.N, cfg.K) >= 0, kept)
    for n in range(cfg.N):
        l = inp["x"][n] @ inp["w_r"] + (0 if inp["bias"] is None else inp["bias"])
        sel = f["topk"][n].astype(np.int64)
        z = np.exp(l[sel] - l[sel].max())
        g = z / z.sum()
        y = sum(g[k] * _ffn(inp["x"][n], inp["w_gate"][sel[k]], inp["w_up"][sel[k]], inp["w_down"][sel[k]])
                for k in range(cfg.K) if kept[n, k])
        y = np.zeros(cfg.H) if isinstance(y, int) else y
        assert np.allclose(f["y"][n], y, rtol=1e-12, atol=1e-12), n


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
def test_metadata_invariants(cfg):
    inp = _inputs(cfg, 2)
    C = O.capacity_of(cfg.N, cfg.K, cfg.E, 0.8)
    f = _fwd(inp, cfg.K, C)
    flat = f["topk"].reshape(-1).astype(np.int64)
    counts, offsets, sf, inv = f["counts"], f["offsets"], f["sorted_flat"], f["inv"]
    assert np.array_equal(counts, np.bincount(flat, minlength=cfg.E))
    kept_counts = np.minimum(counts, C)
    assert np.array_equal(np.diff(offsets), kept_counts) and offsets[0] == 0
    nk = int(offsets[-1])
    assert np.all(sf[nk:] == -1) and np.all(sf[:nk] >= 0)
    for e in range(cfg.E):
        rows = sf[offsets[e]:offsets[e + 1]]
        assert np.array_equal(rows, np.where(flat == e)[0][:C])       # the C lowest flat indices, ascending
    assert np.array_equal(inv[sf[:nk]], np.arange(nk))
    assert np.sum(inv < 0) == flat.size - nk
    assert np.sum(counts - kept_counts) > 0, "the case must drop rows"
    tiles = f["tiles"]
    assert int(tiles[:, 2].sum()) == nk


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
def test_capacity_at_or_above_max_count_is_the_dropless_layer(cfg):
    inp = _inputs(cfg, 3)
    ref = _fwd(inp, cfg.K, None, store="bf16")
    rb = O.backward(ref, inp["dy"])
    for C in (int(ref["counts"].max()), cfg.N * cfg.K):
        f = _fwd(inp, cfg.K, C, store="bf16")
        b = O.backward(f, inp["dy"])
        for k in ("y", "xs", "G", "U", "A", "ys", "offsets", "sorted_flat", "inv"):
            assert np.array_equal(f[k], ref[k]), k
        for k, v in rb.items():
            assert np.array_equal(b[k], v), k


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
def test_zero_capacity_computes_nothing(cfg):
    inp = _inputs(cfg, 4)
    f = _fwd(inp, cfg.K, 0)
    b = O.backward(f, inp["dy"])
    assert np.all(f["y"] == 0) and int(f["offsets"][-1]) == 0 and len(f["tiles"]) == 0
    for k in ("dgates", "dlogits", "dx", "dw_r", "dw_gate", "dw_up", "dw_down", "dys", "dxs"):
        assert np.all(b[k] == 0), k


def _dense_autograd_keep(inp, K, topk, keep):
    """y[n] = sum_e w[n,e] FFN_e(x[n]) with w[n,e] = g[n,k] where e =
    topk[n,k] and slot (n,k) is kept, else 0; g = softmax over the selected
    logits; gradients of <y, dy> by torch autograd in float64."""
    t = {k: (None if v is None else torch.tensor(v, dtype=torch.float64, requires_grad=(k not in ("bias", "dy"))))
         for k, v in inp.items()}
    x, w_r = t["x"], t["w_r"]
    N, E = x.shape[0], w_r.shape[1]
    l = x @ w_r
    if t["bias"] is not None:
        l = l + t["bias"]
    l.retain_grad()
    idx = torch.tensor(topk.astype(np.int64))
    sel = torch.gather(l, 1, idx)
    g = torch.softmax(sel, dim=1) * torch.tensor(keep, dtype=torch.float64)
    W = torch.zeros_like(l).scatter(1, idx, g)
    y = torch.zeros_like(x)
    for e in range(E):
        h = torch.nn.functional.silu(x @ t["w_gate"][e]) * (x @ t["w_up"][e])
        y = y + W[:, e:e + 1] * (h @ t["w_down"][e])
    (y * t["dy"]).sum().backward()
    return dict(y=y.detach().numpy(), dx=x.grad.numpy(), dw_r=w_r.grad.numpy(), dlogits=l.grad.numpy(),
                dw_gate=t["w_gate"].grad.numpy(), dw_up=t["w_up"].grad.numpy(), dw_down=t["w_down"].grad.numpy())


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
def test_backward_matches_dense_autograd_with_fixed_keep_mask(cfg):
    inp = _inputs(cfg, 5)
    C = O.capacity_of(cfg.N, cfg.K, cfg.E, 0.75)
    f = _fwd(inp, cfg.K, C)
    b = O.backward(f, inp["dy"])
    keep = _kept_bruteforce(f["topk"], C)
    assert not keep.all()
    ref = _dense_autograd_keep(inp, cfg.K, f["topk"], keep)
    assert np.allclose(f["y"], ref["y"], rtol=1e-10, atol=1e-12)
    for k in ("dx", "dw_r", "dlogits", "dw_gate", "dw_up", "dw_down"):
        assert np.allclose(b[k], ref[k], rtol=1e-10, atol=1e-12), k


def test_planted_mistake_keeping_the_last_rows_is_caught(monkeypatch):
    good = O.routing_metadata

    def last_c(topk, E, capacity=None):
        if capacity is None:
            return good(topk, E)
        # mirror image: keep the last C rows of each expert
        N, K = topk.shape
        rev = topk.reshape(-1)[::-1].reshape(N, K)
        c, o, sf, inv = good(rev, E, capacity)
        n = topk.size
        sf = np.where(sf >= 0, n - 1 - sf, -1)
        inv2 = inv[::-1].copy()
        return c, o, sf, inv2

    monkeypatch.setattr(O, "routing_metadata", last_c)
    with pytest.raises(AssertionError):
        test_output_matches_bruteforce_keep_rule(CFGS[0], 0.5)
    monkeypatch.setattr(O, "routing_metadata", good)
    test_output_matches_bruteforce_keep_rule(CFGS[0], 0.5)


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
def test_bands_with_capacity(cfg):
    """Rounding bands: with C >= max count they are the dropless bands; with
    a binding C the dropped slots carry no band and the float32 evaluation of
    the kept rows' combine lands inside the y band."""
    inp = _inputs(cfg, 6)
    cfg16 = dict(store="bf16")
    ref = _fwd(inp, cfg.K, None, **cfg16)
    rb = O.backward(ref, inp["dy"])
    band_ref = O.rounding_bands(ref, rb, inp["dy"])
    big = _fwd(inp, cfg.K, int(ref["counts"].max()), **cfg16)
    band_big = O.rounding_bands(big, O.backward(big, inp["dy"]), inp["dy"])
    for k, v in band_ref.items():
        assert np.array_equal(band_big[k], v), k
    C = O.capacity_of(cfg.N, cfg.K, cfg.E, 0.75)
    f = _fwd(inp, cfg.K, C, **cfg16)
    b = O.backward(f, inp["dy"])
    band = O.rounding_bands(f, b, inp["dy"])
    dropped = f["inv"].reshape(cfg.N, cfg.K) < 0
    assert dropped.any() and np.all(b["dgates"][dropped] == 0)
    for k, v in band.items():
        assert np.all(np.isfinite(v)) and np.all(v >= 0), k
    # float32 combine of the kept rows (k ascending) stays inside the y band
    inv = np.maximum(f["inv"], 0).reshape(cfg.N, cfg.K)
    y32 = np.zeros((cfg.N, cfg.H), dtype=np.float32)
    for k in range(cfg.K):
        y32 += (f["gates"][:, k:k + 1] * ~dropped[:, k:k + 1]).astype(np.float32) * f["ys"][inv[:, k]].astype(np.float32)
    y32 = O.round_bf16(y32.astype(np.float64))
    assert np.all(np.abs(y32 - f["y"]) <= band["y"] + 1e-30)
