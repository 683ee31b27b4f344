"""Pins of the oracle's shared expert (CPU only).

A dense SwiGLU expert every token passes through with weight 1, added to the
routed output ("MegaBlocks - architecture and principles", section 2.1).
Pinned by: W_down_s = 0 leaves every routed output and gradient unchanged;
with one routed expert (E = K = 1, gate 1) whose weights equal the shared
ones, y is exactly twice one expert; torch autograd of an independent dense
formulation; the bands cover a float32 evaluation of the shared term; and a
planted mistake (the shared term scaled by the first gate) is caught.
"""
import numpy as np
import pytest
import torch

from moe_workloads import MoEConfig, make_inputs
from oracle import moe_oracle as O

CFG = MoEConfig("s_small", N=24, H=64, F=32, E=5, K=2, dtype="f32")
FS = 48


def _shared(seed, H=64, F=FS):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((H, F)) / np.sqrt(H), rng.standard_normal((H, F)) / np.sqrt(H),
            rng.standard_normal((F, H)) / np.sqrt(F))


def _inputs(cfg, seed):
    return {k: (None if v is None else O.as_f64(v)) for k, v in make_inputs(cfg, seed, with_dy=True).items()}


def _fwd(inp, K, shared, store="f64", **kw):
    return O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], K, bias=inp["bias"],
                     store=store, shared=shared, **kw)


def test_zero_down_projection_changes_nothing_routed():
    inp = _inputs(CFG, 1)
    wg, wu, _ = _shared(2)
    ref = _fwd(inp, CFG.K, None)
    rb = O.backward(ref, inp["dy"])
    f = _fwd(inp, CFG.K, (wg, wu, np.zeros((FS, CFG.H))))
    b = O.backward(f, inp["dy"])
    assert np.array_equal(f["y"], ref["y"])
    for k, v in rb.items():
        assert np.array_equal(b[k], v), k
    assert np.all(b["dG_s"] == 0) and np.all(b["dU_s"] == 0) and np.all(b["dxs_s"] == 0)
    assert np.allclose(b["dw_down_s"], f["shared"]["A"].T @ inp["dy"])


def test_shared_copy_of_the_single_routed_expert_doubles_the_output():
    cfg = MoEConfig("s_one", N=16, H=64, F=32, E=1, K=1, dtype="f32")
    inp = _inputs(cfg, 3)
    f = _fwd(inp, 1, (inp["w_gate"][0], inp["w_up"][0], inp["w_down"][0]))
    g = inp["x"] @ inp["w_gate"][0]
    one = ((g / (1 + np.exp(-g))) * (inp["x"] @ inp["w_up"][0])) @ inp["w_down"][0]
    assert np.allclose(f["y"], 2 * one, rtol=1e-13, atol=1e-13)
    b = O.backward(f, inp["dy"])
    # the shared expert sees the same rows and the same upstream gradient
    assert np.allclose(b["dw_gate_s"], b["dw_gate"][0], rtol=1e-12, atol=1e-12)
    assert np.allclose(b["dw_down_s"], b["dw_down"][0], rtol=1e-12, atol=1e-12)


def _dense_autograd(inp, K, shared):
    t = {k: (None if v is None else torch.tensor(v, dtype=torch.float64, requires_grad=(k not in ("bias", "dy"))))
         for k, v in inp.items()}
    ws = [torch.tensor(w, dtype=torch.float64, requires_grad=True) for w in shared]
    x, w_r = t["x"], t["w_r"]
    E = w_r.shape[1]
    l = x @ w_r + (0 if t["bias"] is None else t["bias"])
    idx = torch.topk(l.detach(), K, dim=1).indices
    M = torch.zeros_like(l).scatter_(1, idx, 1.0)
    z = torch.exp(l - l.max(dim=1, keepdim=True).values) * M
    g = z / z.sum(dim=1, keepdim=True)
    y = torch.zeros_like(x)
    for e in range(E):
        h = torch.nn.functional.silu(x @ t["w_gate"][e]) * (x @ t["w_up"][e])
        y = y + g[:, e:e + 1] * (h @ t["w_down"][e])
    y = y + (torch.nn.functional.silu(x @ ws[0]) * (x @ ws[1])) @ ws[2]
    (y * t["dy"]).sum().backward()
    return dict(y=y.detach().numpy(), dx=x.grad.numpy(), dw_r=w_r.grad.numpy(), dw_gate=t["w_gate"].grad.numpy(),
                dw_up=t["w_up"].grad.numpy(), dw_down=t["w_down"].grad.numpy(), dw_gate_s=ws[0].grad.numpy(),
                dw_up_s=ws[1].grad.numpy(), dw_down_s=ws[2].grad.numpy())


def test_backward_matches_dense_autograd():
    inp = _inputs(CFG, 4)
    sh = _shared(5)
    f = _fwd(inp, CFG.K, sh)
    b = O.backward(f, inp["dy"])
    ref = _dense_autograd(inp, CFG.K, sh)
    assert np.allclose(f["y"], ref["y"], rtol=1e-11, atol=1e-12)
    for k in ("dx", "dw_r", "dw_gate", "dw_up", "dw_down", "dw_gate_s", "dw_up_s", "dw_down_s"):
        assert np.allclose(b[k], ref[k], rtol=1e-10, atol=1e-12), k


def test_bands_cover_a_float32_shared_term():
    cfg = MoEConfig("s_bf16", N=24, H=64, F=32, E=5, K=2, dtype="bf16")
    inp = _inputs(cfg, 6)
    sh = tuple(O.round_bf16(w) for w in _shared(7))
    f = _fwd(inp, cfg.K, sh, store="bf16")
    b = O.backward(f, inp["dy"])
    band = O.rounding_bands(f, b, inp["dy"])
    x32 = torch.tensor(inp["x"], dtype=torch.float32)
    w = [torch.tensor(v, dtype=torch.float32) for v in sh]
    g32 = (x32 @ w[0]).to(torch.bfloat16).float()
    u32 = (x32 @ w[1]).to(torch.bfloat16).float()
    a32 = (torch.nn.functional.silu(g32) * u32).to(torch.bfloat16).float()
    ys32 = (a32 @ w[2]).double().numpy()
    sh_o = f["shared"]
    for name, got in (("G_s", g32), ("U_s", u32), ("A_s", a32)):
        ref = sh_o[name[0]]
        assert np.all(np.abs(got.double().numpy() - ref) <= band[name] + 1e-30), name
    ysr = O.round_bf16(ys32)
    assert np.all(np.abs(ysr - sh_o["ys"]) <= band["ys_s"] + 1e-30)


def test_planted_mistake_gated_shared_term_is_caught(monkeypatch):
    good = O.forward

    def gated(*a, **kw):
        f = good(*a, **kw)
        if f.get("shared") is not None:
            g0 = f["gates"][:, :1]
            f["y"] = O.rho(f["y"] - f["shared"]["ys"] + g0 * f["shared"]["ys"], f["store"])
        return f

    monkeypatch.setattr(O, "forward", gated)
    with pytest.raises(AssertionError):
        test_backward_matches_dense_autograd()
    monkeypatch.setattr(O, "forward", good)
    test_backward_matches_dense_autograd()


def test_bands_cover_a_float32_backward_and_combine():
    """float32 evaluations of the combine with the shared addend, of the
    shared expert's activation backward and of its input gradient land inside
    the oracle's bands."""
    cfg = MoEConfig("s_bf16b", N=32, H=64, F=32, E=4, K=2, dtype="bf16")
    inp = _inputs(cfg, 8)
    sh = tuple(O.round_bf16(w) for w in _shared(9))
    f = _fwd(inp, cfg.K, sh, store="bf16")
    b = O.backward(f, inp["dy"])
    band = O.rounding_bands(f, b, inp["dy"])
    s = f["shared"]
    inv = f["inv"].reshape(cfg.N, cfg.K)
    y32 = s["ys"].astype(np.float32)
    for k in range(cfg.K):
        y32 = y32 + f["gates"][:, k:k + 1].astype(np.float32) * f["ys"][inv[:, k]].astype(np.float32)
    assert np.all(np.abs(O.round_bf16(y32.astype(np.float64)) - f["y"]) <= band["y"] + 1e-30)
    t = lambda a: torch.tensor(a, dtype=torch.float32)
    dA = t(inp["dy"]) @ t(s["w_down"]).T
    G, U = t(s["G"]), t(s["U"])
    sg = torch.sigmoid(G)
    dG = (dA * U * sg * (1 + G * (1 - sg))).to(torch.bfloat16).float()
    dU = (dA * G * sg).to(torch.bfloat16).float()
    for name, got in (("dG_s", dG), ("dU_s", dU)):
        assert np.all(np.abs(got.double().numpy() - b[name]) <= band[name] + 1e-30), name
    dxs = (t(b["dG_s"]) @ t(s["w_gate"]).T + t(b["dU_s"]) @ t(s["w_up"]).T).to(torch.bfloat16).double().numpy()
    assert np.all(np.abs(dxs - b["dxs_s"]) <= band["dxs_s"] + 1e-30)
