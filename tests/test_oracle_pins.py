"""Pins of the CPU oracle to things other than itself (CPU only).

Each pin is computed without the oracle's code path: brute-force per-token
loops, library routines (numpy bincount/cumsum, torch softmax, torch
autograd), closed forms and central finite differences.  The mutation tests
at the end plant plausible mistakes in the oracle and check that at least
one pin catches each.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from moe_workloads import TEST_CONFIGS, TINY, MoEConfig, make_inputs
from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _np(t):
    return O.as_f64(t)


def _inputs(cfg, seed=0):
    d = make_inputs(cfg, seed)
    return {k: (None if v is None else _np(v)) for k, v in d.items()}


# --------------------------------------------------------------------------
# pin helpers (independent of the oracle's code)
# --------------------------------------------------------------------------

def brute_topk(logits_row, K):
    E = len(logits_row)
    return sorted(range(E), key=lambda e: (-float(logits_row[e]), e))[:K]


def brute_forward(inp, K):
    """y_n = sum_k g_k FFN_{e_k}(x_n), evaluated token by token, no sorting."""
    x, w_r, b = inp["x"], inp["w_r"], inp["bias"]
    N, H = x.shape
    E = w_r.shape[1]
    y = np.zeros_like(x)
    tops, gates = [], []
    for n in range(N):
        l = [sum(x[n, h] * w_r[h, e] for h in range(H)) + (0.0 if b is None else b[e]) for e in range(E)]
        top = brute_topk(l, K)
        z = [math.exp(l[e] - l[top[0]]) for e in top]
        g = [v / sum(z) for v in z]
        for k, e in enumerate(top):
            gpre = x[n] @ inp["w_gate"][e]
            upre = x[n] @ inp["w_up"][e]
            a = gpre / (1.0 + np.exp(-gpre)) * upre
            y[n] += g[k] * (a @ inp["w_down"][e])
        tops.append(top)
        gates.append(g)
    return y, np.array(tops), np.array(gates)


def dense_masked_autograd(inp, K):
    """Independent formulation: y = sum_e M_ne g_ne FFN_e(x) over ALL experts,
    with M the top-K mask and g the softmax restricted to the mask; gradients
    from torch autograd in float64."""
    t = {k: (None if v is None else torch.tensor(v, dtype=torch.float64, requires_grad=(k != "bias" and k != "dy")))
         for k, v in inp.items()}
    x, w_r = t["x"], t["w_r"]
    l = x @ w_r
    if t["bias"] is not None:
        l = l + t["bias"]
    l.retain_grad()
    idx = torch.topk(l.detach(), K, dim=1).indices
    M = torch.zeros_like(l).scatter_(1, idx, 1.0)
    z = torch.exp(l - l.max(dim=1, keepdim=True).values) * M
    g = z / z.sum(dim=1, keepdim=True)
    y = torch.zeros_like(x)
    for e in range(w_r.shape[1]):
        h = torch.nn.functional.silu(x @ t["w_gate"][e]) * (x @ t["w_up"][e])
        y = y + g[:, e:e + 1] * (h @ t["w_down"][e])
    loss = (y * t["dy"]).sum()
    loss.backward()
    return dict(y=y.detach().numpy(), dx=x.grad.numpy(), dw_r=w_r.grad.numpy(), dlogits=l.grad.numpy(),
                dw_gate=t["w_gate"].grad.numpy(), dw_up=t["w_up"].grad.numpy(), dw_down=t["w_down"].grad.numpy())


def min_topk_gap(logits, K):
    s = -np.sort(-logits, axis=1)
    if K >= logits.shape[1]:
        return np.inf
    return float(np.min(s[:, K - 1] - s[:, K]))


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(1e-30, np.max(np.abs(b))))


SMALL = [TINY, MoEConfig("p_bias", N=24, H=64, F=64, E=6, K=3, dtype="f32", zipf_s=1.2, zipf_tau=1.25),
         MoEConfig("p_k1", N=20, H=64, F=32, E=5, K=1, dtype="f32"),
         MoEConfig("p_keqe", N=16, H=64, F=32, E=3, K=3, dtype="f32")]


# --------------------------------------------------------------------------
# rounding
# --------------------------------------------------------------------------

def test_round_bf16_matches_torch_rne():
    g = torch.Generator().manual_seed(1)
    v = torch.randn(200000, generator=g, dtype=torch.float32) * torch.exp(torch.randn(200000, generator=g) * 4)
    ref = v.to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(v.to(torch.float64).numpy())
    assert np.array_equal(ref, got)


def test_round_bf16_ties_to_even():
    one = 1.0
    ulp = 2.0 ** -7
    # exactly halfway between 1 and 1+ulp: ties to the even mantissa (1.0)
    assert O.round_bf16(np.array([one + ulp / 2]))[0] == one
    # halfway between 1+ulp (odd) and 1+2ulp (even): rounds up to even
    assert O.round_bf16(np.array([one + 1.5 * ulp]))[0] == one + 2 * ulp
    # just above halfway rounds up
    assert O.round_bf16(np.array([one + ulp / 2 + 1e-12]))[0] == one + ulp
    assert O.round_bf16(np.array([-(one + ulp / 2 + 1e-12)]))[0] == -(one + ulp)


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------

def test_topk_matches_bruteforce_with_ties():
    rng = np.random.default_rng(3)
    l = rng.integers(-3, 4, size=(300, 9)).astype(np.float64)   # many exact ties
    for K in (1, 2, 4, 9):
        got = O.topk_experts(l, K)
        for n in range(l.shape[0]):
            assert list(got[n]) == brute_topk(l[n], K)


def test_gates_sum_to_one_and_two_formulas_agree():
    rng = np.random.default_rng(4)
    l = rng.normal(size=(500, 17)) * 3
    for K in (1, 2, 5, 17):
        top = O.topk_experts(l, K)
        g1 = O.gates_topk_softmax(l, top)
        g2 = O.gates_renormalised_softmax(l, top)
        assert np.allclose(g1.sum(axis=1), 1.0, atol=1e-12)
        assert np.allclose(g1, g2, rtol=1e-12, atol=1e-15)
        # the first slot holds the largest gate
        assert np.all(g1[:, :1] >= g1 - 1e-15)
    # gates equal torch's softmax over the selected values
    top = O.topk_experts(l, 3)
    sel = np.take_along_axis(l, top.astype(np.int64), axis=1)
    ref = torch.softmax(torch.tensor(sel), dim=1).numpy()
    assert np.allclose(O.gates_topk_softmax(l, top), ref, rtol=1e-13, atol=1e-15)


def brute_metadata(topk, E, tile_m):
    flat = [int(v) for v in topk.reshape(-1)]
    counts = [0] * E
    for e in flat:
        counts[e] += 1
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    sorted_flat = [f for e in range(E) for f in range(len(flat)) if flat[f] == e]
    inv = [0] * len(flat)
    for i, f in enumerate(sorted_flat):
        inv[f] = i
    tiles = []
    for e in range(E):
        start = offsets[e]
        while start < offsets[e + 1]:
            tiles.append([e, start, min(tile_m, offsets[e + 1] - start)])
            start += tile_m
    return counts, offsets, sorted_flat, inv, tiles


@pytest.mark.parametrize("E,K,N,tile_m", [(4, 2, 32, 128), (8, 2, 1000, 64), (64, 6, 300, 128), (256, 8, 200, 16),
                                          (1, 1, 77, 32), (5, 5, 40, 8)])
def test_metadata_matches_bruteforce(E, K, N, tile_m):
    rng = np.random.default_rng(E * 1000 + K)
    # each token picks K distinct experts, skewed towards low ids
    p = np.arange(1, E + 1, dtype=np.float64) ** -1.5
    p /= p.sum()
    topk = np.stack([rng.choice(E, size=K, replace=False, p=p) for _ in range(N)]).astype(np.int32)
    counts, offsets, sorted_flat, inv = O.routing_metadata(topk, E)
    tiles = O.tile_list(counts, offsets, tile_m)
    bc, bo, bs, bi, bt = brute_metadata(topk, E, tile_m)
    assert list(counts) == bc and list(offsets) == bo
    assert list(sorted_flat) == bs and list(inv) == bi
    assert tiles.tolist() == bt
    # invariants
    assert counts.sum() == N * K and offsets[-1] == N * K
    assert np.array_equal(np.sort(sorted_flat), np.arange(N * K))
    assert np.array_equal(sorted_flat[inv], np.arange(N * K))
    for e in range(E):
        seg = sorted_flat[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(topk.reshape(-1)[seg] == e)
    assert len(tiles) <= (N * K + E * (tile_m - 1)) // tile_m


def test_maxvio():
    assert O.maxvio(np.array([4, 4, 4, 4]), 8, 2, 4) == 0.0
    assert O.maxvio(np.array([16, 0, 0, 0]), 8, 2, 4) == 3.0


# --------------------------------------------------------------------------
# forward
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_forward_matches_bruteforce_per_token(cfg):
    inp = _inputs(cfg)
    fwd = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.K, bias=inp["bias"],
                    store="f64")
    y, tops, gates = brute_forward(inp, cfg.K)
    assert np.array_equal(fwd["topk"], tops)
    assert np.allclose(fwd["gates"], gates, rtol=1e-12, atol=1e-15)
    assert np.allclose(fwd["gates"].sum(axis=1), 1.0, atol=1e-12)
    assert fwd["counts"].sum() == cfg.N * cfg.K
    assert _rel(fwd["y"], y) < 1e-12


def test_forward_identical_experts_is_dense_swiglu():
    cfg = MoEConfig("p_same", N=40, H=64, F=96, E=6, K=2, dtype="f32")
    inp = _inputs(cfg)
    for name in ("w_gate", "w_up", "w_down"):
        inp[name][:] = inp[name][0]
    fwd = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.K, store="f64")
    x = torch.tensor(inp["x"])
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(x @ torch.tensor(inp["w_gate"][0])) * (x @ torch.tensor(inp["w_up"][0])),
        torch.tensor(inp["w_down"][0]).T)
    assert _rel(fwd["y"], ref.numpy()) < 1e-12


def test_forward_k_equals_e_is_dense_softmax_mixture():
    cfg = MoEConfig("p_keqe2", N=30, H=64, F=32, E=4, K=4, dtype="f32")
    inp = _inputs(cfg)
    fwd = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.K, store="f64")
    x = torch.tensor(inp["x"])
    p = torch.softmax(x @ torch.tensor(inp["w_r"]), dim=1)
    ref = 0
    for e in range(cfg.E):
        h = torch.nn.functional.silu(x @ torch.tensor(inp["w_gate"][e])) * (x @ torch.tensor(inp["w_up"][e]))
        ref = ref + p[:, e:e + 1] * (h @ torch.tensor(inp["w_down"][e]))
    assert _rel(fwd["y"], ref.numpy()) < 1e-12


def test_forward_k1_gate_is_one_and_picks_argmax():
    cfg = MoEConfig("p_k1b", N=50, H=64, F=32, E=7, K=1, dtype="f32")
    inp = _inputs(cfg)
    fwd = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], 1, store="f64")
    assert np.all(fwd["gates"] == 1.0)
    l = torch.tensor(inp["x"]) @ torch.tensor(inp["w_r"])
    assert np.array_equal(fwd["topk"][:, 0], torch.argmax(l, dim=1).numpy())


def test_forward_e1_is_textbook_swiglu_and_zero_down_gives_zero():
    cfg = MoEConfig("p_e1", N=20, H=64, F=32, E=1, K=1, dtype="f32")
    inp = _inputs(cfg)
    fwd = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], 1, store="f64")
    x = torch.tensor(inp["x"])
    ref = (torch.nn.functional.silu(x @ torch.tensor(inp["w_gate"][0])) * (x @ torch.tensor(inp["w_up"][0]))) \
        @ torch.tensor(inp["w_down"][0])
    assert _rel(fwd["y"], ref.numpy()) < 1e-12
    inp["w_down"][:] = 0.0
    fwd = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], 1, store="bf16")
    assert np.all(fwd["y"] == 0.0)


def test_forward_token_permutation_equivariance():
    cfg = TINY
    inp = _inputs(cfg)
    perm = np.random.default_rng(5).permutation(cfg.N)
    a = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.K, store="f64")
    b = O.forward(inp["x"][perm], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.K, store="f64")
    assert _rel(b["y"], a["y"][perm]) < 1e-13


def test_forward_expert_relabelling_invariance():
    cfg = TINY
    inp = _inputs(cfg)
    perm = np.array([2, 0, 3, 1])
    a = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.K, store="f64")
    b = O.forward(inp["x"], inp["w_r"][:, perm], inp["w_gate"][perm], inp["w_up"][perm], inp["w_down"][perm],
                  cfg.K, store="f64")
    assert _rel(b["y"], a["y"]) < 1e-13
    assert np.array_equal(np.sort(perm[b["topk"]], axis=1), np.sort(a["topk"], axis=1))


def test_token_forward_backward_match_whole_layer():
    cfg = MoEConfig("p_tok", N=30, H=64, F=64, E=5, K=2, dtype="bf16", zipf_s=1.2, zipf_tau=1.0)
    d = make_inputs(cfg, 2)
    inp = {k: (None if v is None else _np(v)) for k, v in d.items()}
    fwd = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.K, bias=inp["bias"],
                    store="bf16")
    bwd = O.backward(fwd, inp["dy"])
    ew = lambda e: (inp["w_gate"][e], inp["w_up"][e], inp["w_down"][e])  # noqa: E731
    for n in (0, 7, 29):
        tf = O.token_forward(inp["x"][n], inp["w_r"], inp["bias"], ew, cfg.K, "bf16")
        assert np.array_equal(tf["topk"], fwd["topk"][n])
        assert np.allclose(tf["y"], fwd["y"][n], rtol=0, atol=1e-2)
        tb = O.token_backward(tf, inp["dy"][n], inp["w_r"], ew, "bf16")
        assert np.allclose(tb["dx"], bwd["dx"][n], rtol=0, atol=2e-2)
        assert np.allclose(tb["dlogits"], bwd["dlogits"][n], rtol=1e-5, atol=1e-6)


def test_mirror_mode_close_to_exact():
    cfg = MoEConfig("p_mirror", N=64, H=128, F=128, E=4, K=2, dtype="bf16")
    d = make_inputs(cfg, 1)
    inp = {k: (None if v is None else _np(v)) for k, v in d.items()}
    ex = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], 2, store="f64")
    mi = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], 2, store="bf16")
    rms = np.sqrt(np.mean((ex["y"] - mi["y"]) ** 2) / np.mean(ex["y"] ** 2))
    assert 0 < rms < 1e-2
    # stored activations are bf16 values
    for k in ("G", "U", "A", "ys", "y"):
        assert np.array_equal(O.round_bf16(mi[k]), mi[k])


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_backward_matches_dense_masked_autograd(cfg):
    inp = _inputs(cfg)
    fwd = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.K, bias=inp["bias"],
                    store="f64")
    assert min_topk_gap(fwd["logits"], cfg.K) > 1e-9
    bwd = O.backward(fwd, inp["dy"])
    ref = dense_masked_autograd(inp, cfg.K)
    assert _rel(fwd["y"], ref["y"]) < 1e-12
    for name in ("dx", "dw_r", "dlogits", "dw_gate", "dw_up", "dw_down"):
        assert _rel(bwd[name], ref[name]) < 1e-10, name


def test_backward_finite_differences():
    cfg = TINY
    inp = _inputs(cfg, 0)
    fwd = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.K, store="f64")
    gap = min_topk_gap(fwd["logits"], cfg.K)
    bwd = O.backward(fwd, inp["dy"])
    rng = np.random.default_rng(11)
    names = {"x": "dx", "w_r": "dw_r", "w_gate": "dw_gate", "w_up": "dw_up", "w_down": "dw_down"}

    def loss(v):
        f = O.forward(v["x"], v["w_r"], v["w_gate"], v["w_up"], v["w_down"], cfg.K, store="f64")
        return float(np.sum(f["y"] * inp["dy"])), f["topk"]

    eps = 1e-6
    for name, gname in names.items():
        for _ in range(25):
            idx = tuple(int(rng.integers(0, s)) for s in inp[name].shape)
            v = {k: (a.copy() if isinstance(a, np.ndarray) else a) for k, a in inp.items()}
            v[name][idx] += eps
            lp, tp = loss(v)
            v[name][idx] -= 2 * eps
            lm, tm = loss(v)
            if not (np.array_equal(tp, fwd["topk"]) and np.array_equal(tm, fwd["topk"])):
                continue  # the step crossed a selection boundary (gap %g)
            fd = (lp - lm) / (2 * eps)
            an = bwd[gname][idx]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, idx, fd, an, gap)


def test_unselected_logits_get_zero_gradient():
    cfg = MoEConfig("p_zero", N=40, H=64, F=32, E=8, K=2, dtype="f32")
    inp = _inputs(cfg)
    fwd = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.K, store="f64")
    bwd = O.backward(fwd, inp["dy"])
    mask = np.zeros((cfg.N, cfg.E), dtype=bool)
    np.put_along_axis(mask, fwd["topk"].astype(np.int64), True, axis=1)
    assert np.all(bwd["dlogits"][~mask] == 0.0)
    # softmax gradient rows sum to zero over the selected experts
    assert np.allclose(bwd["dlogits"].sum(axis=1), 0.0, atol=1e-12)


def test_empty_experts_get_zero_weight_gradients():
    cfg = TEST_CONFIGS["t_skew"]
    d = make_inputs(cfg, 0)
    inp = {k: (None if v is None else _np(v)) for k, v in d.items()}
    fwd = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.K, bias=inp["bias"],
                    store="bf16")
    empty = np.where(fwd["counts"] == 0)[0]
    assert empty.size > 0
    bwd = O.backward(fwd, inp["dy"])
    for e in empty:
        assert np.all(bwd["dw_gate"][e] == 0) and np.all(bwd["dw_up"][e] == 0) and np.all(bwd["dw_down"][e] == 0)


# --------------------------------------------------------------------------
# closed form
# --------------------------------------------------------------------------

def _golden():
    with open(os.path.join(GOLDEN, "closed_form_e3_k2.json")) as fh:
        return json.load(fh)


def _ev(a):
    env = {"log": math.log, "__builtins__": {}}
    if isinstance(a, list):
        return [_ev(v) for v in a]
    return float(eval(a, env)) if isinstance(a, str) else a  # noqa: S307 - fixture expressions only


def test_closed_form_fixture():
    gd = _golden()
    inp = {k: np.array(_ev(v), dtype=np.float64) for k, v in gd["inputs"].items()}
    fwd = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], gd["K"], store="f64",
                    tile_m=gd["tile_m"])
    bwd = O.backward(fwd, inp["dy"])
    ex = gd["expected"]
    for k in ("topk", "counts", "offsets", "sorted_flat", "inv", "tiles"):
        assert np.array_equal(np.asarray(fwd[k]), np.asarray(ex[k])), k
    for k in ("gates", "y"):
        assert np.allclose(fwd[k], np.array(_ev(ex[k])), rtol=0, atol=1e-14), k
    for k in ("dgates", "dlogits", "dw_r", "dw_down", "dw_gate", "dw_up", "dx"):
        assert np.allclose(bwd[k], np.array(_ev(ex[k])), rtol=0, atol=1e-14), k


# --------------------------------------------------------------------------
# mutation tests: plant a mistake in the oracle, a pin must fail
# --------------------------------------------------------------------------


# --------------------------------------------------------------------------
# given assignment, and weight-gradient slices (used by the full-size checks)
# --------------------------------------------------------------------------

def test_forward_given_assignment_matches_bruteforce():
    """forward(topk=...) with an arbitrary assignment of distinct experts:
    per token, y = sum_k softmax(l[sel])_k FFN_{sel_k}(x), brute force."""
    cfg = MoEConfig("p_given", N=12, H=64, F=32, E=5, K=2, dtype="f32", zipf_s=1.2, zipf_tau=1.25)
    inp = _inputs(cfg)
    rng = np.random.default_rng(5)
    topk = np.stack([rng.permutation(cfg.E)[:cfg.K] for _ in range(cfg.N)])
    f = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.K, bias=inp["bias"],
                  store="f64", topk=topk)
    assert np.array_equal(f["topk"], topk)
    for n in range(cfg.N):
        l = [sum(inp["x"][n, h] * inp["w_r"][h, e] for h in range(cfg.H)) + inp["bias"][e] for e in range(cfg.E)]
        z = [math.exp(l[e]) for e in topk[n]]
        ref = np.zeros(cfg.H)
        for k, e in enumerate(topk[n]):
            a = inp["x"][n] @ inp["w_gate"][e]
            ref += z[k] / sum(z) * ((a / (1 + np.exp(-a)) * (inp["x"][n] @ inp["w_up"][e])) @ inp["w_down"][e])
        assert np.allclose(f["y"][n], ref, rtol=1e-12, atol=1e-12)
    # the own selection passed back in changes nothing
    g = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.K, bias=inp["bias"],
                  store="f64")
    h = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.K, bias=inp["bias"],
                  store="f64", topk=g["topk"])
    assert np.array_equal(g["y"], h["y"])


@pytest.mark.parametrize("store", ["bf16", "f64"])
def test_weight_grad_slices_match_whole_layer(store):
    """Columns of dW_gate / dW_up and rows of dW_down from
    weight_grad_slices equal the pinned whole-layer backward's, including an
    expert with no rows (exact zeros)."""
    cfg = TEST_CONFIGS["t_skew"]
    inp = _inputs(cfg, seed=2)
    inp_dy = O.as_f64(make_inputs(cfg, 2, with_dy=True)["dy"])
    f = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.K, bias=inp["bias"],
                  store=store)
    b = O.backward(f, inp_dy)
    empty = int(np.where(f["counts"] == 0)[0][0])
    hot = int(np.argmax(f["counts"]))
    cols = [0, 7, cfg.F - 1]
    for e in (hot, empty, int(np.argsort(f["counts"])[cfg.E // 2])):
        s = O.weight_grad_slices(inp["x"], inp_dy, f["topk"], f["gates"], e, inp["w_gate"][e], inp["w_up"][e],
                                 inp["w_down"][e], cols, store)
        assert np.allclose(s["dw_gate"], b["dw_gate"][e][:, cols], rtol=1e-12, atol=1e-12)
        assert np.allclose(s["dw_up"], b["dw_up"][e][:, cols], rtol=1e-12, atol=1e-12)
        assert np.allclose(s["dw_down"], b["dw_down"][e][cols, :], rtol=1e-12, atol=1e-12)
        if e == empty:
            assert not s["dw_gate"].any() and not s["dw_down"].any()


@pytest.mark.parametrize("store", ["bf16", "f32"])
def test_expert_rows_match_whole_layer(store):
    """Any subset of one expert's rows from expert_rows equals the pinned
    whole-layer forward and backward on those rows, bit for bit."""
    cfg = TEST_CONFIGS["t_ragged"]
    inp = _inputs(cfg, seed=4)
    dy = O.as_f64(make_inputs(cfg, 4, with_dy=True)["dy"])
    f = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.K, store=store)
    b = O.backward(f, dy)
    rng = np.random.default_rng(0)
    for e in range(cfg.E):
        r0, r1 = int(f["offsets"][e]), int(f["offsets"][e + 1])
        rows = np.sort(rng.choice(np.arange(r0, r1), size=min(9, r1 - r0), replace=False))
        sf = f["sorted_flat"][rows]
        got = O.expert_rows(inp["x"][sf // cfg.K], f["gates"].reshape(-1)[sf], dy[sf // cfg.K], inp["w_gate"][e],
                            inp["w_up"][e], inp["w_down"][e], store)
        for k in ("xs", "G", "U", "A", "ys"):
            assert np.array_equal(got[k], f[k][rows]), (e, k)
        for k in ("dys", "dG", "dU", "dxs"):
            assert np.array_equal(got[k], b[k][rows]), (e, k)


def _pins_pass():
    """Run a compact set of pins; True when all hold."""
    try:
        test_closed_form_fixture()
        for cfg in SMALL[:2]:
            test_forward_matches_bruteforce_per_token(cfg)
            test_backward_matches_dense_masked_autograd(cfg)
        test_topk_matches_bruteforce_with_ties()
        test_gates_sum_to_one_and_two_formulas_agree()
        test_metadata_matches_bruteforce(8, 2, 100, 16)
    except AssertionError:
        return False
    return True


def test_pins_pass_on_unmodified_oracle():
    assert _pins_pass()


MUTATIONS = {
    "silu_on_up_branch": ("swiglu_expert", lambda xs, wg, wu, wd, store: (
        O.rho(xs @ wg, store), O.rho(xs @ wu, store),
        O.rho((xs @ wg) * O.silu(xs @ wu), store), O.rho(O.rho((xs @ wg) * O.silu(xs @ wu), store) @ wd, store))),
    "gates_not_renormalised": ("gates_topk_softmax", lambda l, top: np.take_along_axis(
        np.exp(l - l.max(axis=1, keepdims=True)) / np.exp(l - l.max(axis=1, keepdims=True)).sum(axis=1, keepdims=True),
        top.astype(np.int64), axis=1)),
    "tiebreak_id_descending": ("topk_experts", lambda l, K: np.ascontiguousarray(
        (l.shape[1] - 1 - np.argsort(-l[:, ::-1], axis=1, kind="stable"))[:, :K]).astype(np.int32)),
    "unstable_sort": ("routing_metadata", lambda topk, E, capacity=None: (lambda c, o, s, i: (c, o, s[::-1].copy(), i))(
        *_orig_meta(topk, E, capacity))),
    "sigmoid_wrong_sign": ("sigmoid", lambda z: 1.0 / (1.0 + np.exp(z))),
    "silu_wrong": ("silu", lambda z: z / (1.0 + np.exp(z))),
    "bias_dropped": ("router_logits", lambda x, w_r, bias=None: x @ w_r),
    "tiles_off_by_one": ("tile_list", lambda counts, offsets, tile_m: _orig_tiles(counts + 1, offsets, tile_m)),
}

_orig_meta = O.routing_metadata
_orig_tiles = O.tile_list


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    assert not _pins_pass(), f"no pin caught mutation {name}"
