"""Pins of the oracle's Switch load-balancing loss (CPU only).

L_aux = alpha * E * sum_i f_i P_i with f_i = counts_i / (N*K) and P_i the mean
over tokens of the full router softmax ("MoE computation principle and
execution process", section 4.2).  Pinned by its closed-form values at
uniform and at fully collapsed routing, by central finite differences, by
torch autograd of an independent dense formulation of the whole layer plus
the loss, and by a planted mistake that the pins must catch.
"""
import numpy as np
import pytest
import torch

from moe_workloads import TEST_CONFIGS, MoEConfig, make_inputs
from oracle import moe_oracle as O


def test_uniform_routing_gives_alpha():
    N, E, K, alpha = 64, 8, 2, 0.037
    logits = np.zeros((N, E))
    counts = np.full(E, N * K // E)
    assert O.aux_loss(logits, counts, K, alpha) == pytest.approx(alpha, rel=1e-15)


def test_collapsed_routing_gives_alpha_times_e():
    N, E, K, alpha = 32, 6, 1, 0.01
    logits = np.full((N, E), -60.0)
    logits[:, 0] = 60.0
    counts = np.zeros(E, dtype=np.int64)
    counts[0] = N
    assert O.aux_loss(logits, counts, K, alpha) == pytest.approx(alpha * E, rel=1e-12)


def test_grad_matches_central_differences():
    rng = np.random.default_rng(4)
    N, E, K, scale = 12, 7, 3, 0.3
    logits = rng.standard_normal((N, E)) * 1.5
    counts = rng.multinomial(N * K, np.ones(E) / E)
    g = O.aux_loss_grad(logits, counts, K, scale)
    h = 1e-6
    for n in range(N):
        for e in range(E):
            lp, lm = logits.copy(), logits.copy()
            lp[n, e] += h
            lm[n, e] -= h
            fd = (O.aux_loss(lp, counts, K, scale) - O.aux_loss(lm, counts, K, scale)) / (2 * h)
            assert abs(fd - g[n, e]) <= 1e-8 + 1e-6 * abs(fd)
    # each token's gradient sums to zero over the experts (softmax invariance)
    assert np.allclose(g.sum(axis=1), 0.0, atol=1e-15)


def _dense_autograd_with_aux(inp, K, alpha):
    """Independent formulation: y = sum over ALL experts of M g FFN, plus
    L_aux from the full softmax and the top-K mask counts (detached);
    gradients of <y, dy> + L_aux by torch autograd in float64."""
    t = {k: (None if v is None else torch.tensor(v, dtype=torch.float64, requires_grad=(k not in ("bias", "dy"))))
         for k, v in inp.items()}
    x, w_r = t["x"], t["w_r"]
    N, E = x.shape[0], w_r.shape[1]
    l = x @ w_r
    if t["bias"] is not None:
        l = l + t["bias"]
    l.retain_grad()
    idx = torch.topk(l.detach(), K, dim=1).indices
    M = torch.zeros_like(l).scatter_(1, idx, 1.0)
    z = torch.exp(l - l.max(dim=1, keepdim=True).values) * M
    g = z / z.sum(dim=1, keepdim=True)
    y = torch.zeros_like(x)
    for e in range(E):
        h = torch.nn.functional.silu(x @ t["w_gate"][e]) * (x @ t["w_up"][e])
        y = y + g[:, e:e + 1] * (h @ t["w_down"][e])
    f = M.sum(dim=0) / (N * K)
    P = torch.softmax(l, dim=1).mean(dim=0)
    loss = (y * t["dy"]).sum() + alpha * E * (f * P).sum()
    loss.backward()
    return dict(dx=x.grad.numpy(), dw_r=w_r.grad.numpy(), dlogits=l.grad.numpy(),
                dw_gate=t["w_gate"].grad.numpy(), dw_up=t["w_up"].grad.numpy(), dw_down=t["w_down"].grad.numpy())


@pytest.mark.parametrize("cfg", [MoEConfig("a_small", N=20, H=64, F=32, E=6, K=2, dtype="f32"),
                                 MoEConfig("a_bias", N=16, H=64, F=32, E=8, K=3, dtype="f32", zipf_s=1.2,
                                           zipf_tau=1.25)], ids=lambda c: c.name)
def test_backward_with_aux_matches_dense_autograd(cfg):
    alpha = 0.05
    inp = {k: (None if v is None else O.as_f64(v)) for k, v in make_inputs(cfg, 6, with_dy=True).items()}
    f = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.K, bias=inp["bias"],
                  store="f64")
    b = O.backward(f, inp["dy"], aux_scale=alpha)
    ref = _dense_autograd_with_aux(inp, cfg.K, alpha)
    for k, v in ref.items():
        assert np.allclose(b[k], v, rtol=1e-10, atol=1e-12), k
    # the aux term makes every router logit's gradient nonzero
    assert np.count_nonzero(b["dlogits"]) == b["dlogits"].size


def test_planted_mistake_in_the_aux_gradient_is_caught(monkeypatch):
    good = O.aux_loss_grad

    def wrong(logits, counts, K, scale):  # drops the softmax's coupling term
        N, E = logits.shape
        p = O.router_probs(logits)
        f = np.asarray(counts, dtype=np.float64) / (N * K)
        return scale * E / N * p * f[None, :]

    monkeypatch.setattr(O, "aux_loss_grad", wrong)
    with pytest.raises(AssertionError):
        test_grad_matches_central_differences()
    monkeypatch.setattr(O, "aux_loss_grad", good)
    test_grad_matches_central_differences()


def test_bands_with_aux_cover_a_float32_evaluation():
    """The float32 evaluation of tests/standin.py plus the aux term in
    float32 lands inside the band of dx."""
    from tests.standin import float32_layer
    cfg = TEST_CONFIGS["t_skew"]
    alpha = 0.05
    inp = {k: (None if v is None else O.as_f64(v)) for k, v in make_inputs(cfg, 3, with_dy=True).items()}
    fwd = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.K, bias=inp["bias"],
                    store="bf16")
    bwd = O.backward(fwd, inp["dy"], aux_scale=alpha)
    band = O.rounding_bands(fwd, bwd, inp["dy"], aux_scale=alpha)
    alt = float32_layer(inp, fwd, cfg.K)
    # float32 aux gradient from float32 logits, added before dW_r and dx
    x32 = torch.tensor(inp["x"], dtype=torch.float32)
    w32 = torch.tensor(inp["w_r"], dtype=torch.float32)
    l32 = x32 @ w32 + (0 if inp["bias"] is None else torch.tensor(inp["bias"], dtype=torch.float32))
    p32 = torch.softmax(l32, dim=1)
    N, E = l32.shape
    f32 = torch.tensor(fwd["counts"], dtype=torch.float32) / (N * cfg.K)
    aux = alpha * E / N * p32 * (f32[None, :] - (p32 @ f32)[:, None])
    dl = torch.tensor(alt["dlogits"], dtype=torch.float32) + aux
    dxs = torch.tensor(alt["dxs"], dtype=torch.float32)
    inv = torch.tensor(fwd["inv"], dtype=torch.int64).view(N, cfg.K)
    dx = (sum(dxs[inv[:, k]] for k in range(cfg.K)) + dl @ w32.T).to(torch.bfloat16).to(torch.float32)
    got = {"dx": dx.double().numpy()}
    for k, a in got.items():
        dev = np.abs(a - bwd[k])
        assert np.all(dev <= band[k]), (k, float((dev - band[k]).max()))
