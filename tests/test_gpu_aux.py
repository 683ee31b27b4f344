"""Parity of the Switch load-balancing loss on the GPU (through the C ABI)
with the CPU oracle: the loss value, the router probabilities, and the whole
backward with the loss's gradient folded into dlogits (dense router term),
on both router paths (matrix cores for bf16 with E % 8 == 0, vector ALUs
otherwise), the fp32 storage type and the default workload at full size.
"""
import numpy as np
import pytest
import torch

from moe_workloads import BASE, TEST_CONFIGS, TINY, MoEConfig
from oracle import moe_oracle as O
from tests.gpu_common import assert_close, check_runner_steps, gpu_inputs, oracle_fwd, store_of, sync, to_np

pytestmark = pytest.mark.gpu

ALPHA = 0.5  # large enough that the dense term stands well above float32 rounding
U32 = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_sort_amd import _lib
    _lib.lib()


def _check_aux_dlogits(dl_on, dl_off, logits, counts, dcount, sig, N, E, K):
    """dlogits with the loss minus dlogits without it (same routing, float32
    both) equals the oracle's aux gradient to within the float32 logits'
    effect on p, the rounding of the sum, and (full size) near-tie swaps of
    the oracle's counts."""
    coef = ALPHA * E / N
    p_ref = O.router_probs(logits)
    aux_ref = O.aux_loss_grad(logits, counts, K, ALPHA)
    diff = dl_on - dl_off
    shift = (dcount[None, :] + p_ref @ dcount[:, None]) / (N * K)     # f and sum_i f_i p_i under swaps
    bound = (coef * p_ref * (4 * sig + shift) + 4 * U32 * np.abs(dl_on) + 8 * U32 * np.abs(aux_ref) + 1e-12)
    dev = np.abs(diff - aux_ref)
    worst = float((dev - bound).max())
    print(f"aux dlogits: max|dev| {float(dev.max()):.3e} (aux term up to {float(np.abs(aux_ref).max()):.3e}), "
          f"worst dev - bound {worst:.3e}", flush=True)
    assert worst <= 0, "dlogits(aux) - dlogits(no aux) != aux gradient"
    assert np.count_nonzero(dl_on) == N * E


def _check_dw_r_and_dx(x, w_r, dl, dw_r, dx, dxs, inv, K, dtype):
    """dW_r = x^T dlogits and dx = sum_k dxs[inv] + dlogits W_r^T over every
    element, with the dense dlogits the device produced."""
    ref = x.T @ dl
    assert np.all(np.abs(dw_r - ref) <= O.gemm_sigma(x.T, dl) + 2 * U32 * np.abs(ref)), "dW_r = x^T dlogits"
    rows = dxs[inv.reshape(-1, K)]
    pre = rows.sum(axis=1) + dl @ w_r.T
    sig = 8 * U32 * (np.abs(rows).sum(axis=1) + np.abs(dl) @ np.abs(w_r.T)) + O.gemm_sigma(dl, w_r.T)
    if dtype == "f32":
        assert np.all(np.abs(dx - pre) <= sig), "dx = sum_k dxs[inv] + dlogits W_r^T"
    else:
        rounded = O.round_bf16(pre)
        assert np.all(np.abs(dx - rounded) <= O.bf16_flip(pre, rounded, sig)), "dx = sum_k dxs[inv] + dlogits W_r^T"


CASES = [TEST_CONFIGS["t_skew"], TEST_CONFIGS["t_wide_e"], TEST_CONFIGS["t_ragged"], TEST_CONFIGS["t_f32"], TINY, BASE,
         # fp32 storage with more than 8 experts (token-tiled dense gather backward)
         MoEConfig("t_aux_f32_e12", N=150, H=128, F=256, E=12, K=2, dtype="f32")]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_aux_loss_forward_and_backward(cfg):
    from mixture_experts_layer_sort_amd.layer import MoELayerRunner
    print(f"[aux] {cfg.name}", flush=True)
    cpu, dev = gpu_inputs(cfg, 5, with_dy=True)
    of = oracle_fwd(cfg, cpu)
    # the oracle's assignment (ties between experts aside, the router's own),
    # without and with the loss
    topk = torch.from_numpy(of["topk"]).cuda()
    gates = torch.from_numpy(of["gates"].astype(np.float32)).cuda()
    r0 = MoELayerRunner(cfg.N, cfg.H, cfg.F, cfg.E, cfg.K, cfg.torch_dtype, "cuda")
    r0.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"], topk=topk, gates=gates)
    dl_off = to_np(r0.backward(dev["dy"])["dlogits"])
    r = MoELayerRunner(cfg.N, cfg.H, cfg.F, cfg.E, cfg.K, cfg.torch_dtype, "cuda", aux_alpha=ALPHA)
    r.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"], topk=topk, gates=gates)
    grads = r.backward(dev["dy"])
    sync()
    dt = store_of(cfg)

    # loss and probabilities: float32 logits are within gemm_sigma of the
    # exact ones; a probability moves by at most 2 p max sigma under that
    p_ref = O.router_probs(of["logits"])
    sig = O.gemm_sigma(of["x"], of["w_r"]).max(axis=1, keepdims=True)
    p_gpu = to_np(r.probs)
    assert np.all(np.abs(p_gpu - p_ref) <= 2 * p_ref * sig + 8 * U32), "router probabilities"
    loss_ref = O.aux_loss(of["logits"], of["counts"], cfg.K, ALPHA)
    loss_gpu = float(r.aux_loss.item())
    print(f"loss gpu {loss_gpu:.8g} oracle {loss_ref:.8g}", flush=True)
    assert abs(loss_gpu - loss_ref) <= 1e-5 * abs(loss_ref) + 4 * ALPHA * cfg.E * float(sig.max())

    # the loss's gradient, tightly; then the products of the dense dlogits
    dl_on = to_np(grads["dlogits"])
    _check_aux_dlogits(dl_on, dl_off, of["logits"], of["counts"], np.zeros(cfg.E), sig, cfg.N, cfg.E, cfg.K)
    _check_dw_r_and_dx(O.as_f64(cpu["x"]), O.as_f64(cpu["w_r"]), dl_on, to_np(grads["dw_r"]), to_np(grads["dx"]),
                       to_np(r.dxs), r.inv.cpu().numpy().astype(np.int64), cfg.K, dt)

    # the whole backward with the loss's gradient against the oracle
    ob = O.backward(of, cpu["dy"], aux_scale=ALPHA)
    bd = O.rounding_bands(of, ob, cpu["dy"], aux_scale=ALPHA) if dt == "bf16" else {}
    for name in ("dlogits", "dw_r", "dx", "dgates", "dw_gate", "dw_up", "dw_down"):
        assert_close(name, grads[name], ob[name], dt, band=bd.get(name))
    # every step from its own stored inputs, the loss term from the stored probabilities
    check_runner_steps(cfg, cpu, r, None, grads,
                       aux=dict(probs=to_np(r.probs), counts=r.counts.cpu().numpy(), scale=ALPHA))


def test_aux_loss_bitwise_reproducible():
    from mixture_experts_layer_sort_amd.layer import MoELayerRunner
    cfg = TEST_CONFIGS["t_skew"]
    cpu, dev = gpu_inputs(cfg, 7, with_dy=True)
    outs = []
    for _ in range(2):
        r = MoELayerRunner(cfg.N, cfg.H, cfg.F, cfg.E, cfg.K, cfg.torch_dtype, "cuda", aux_alpha=ALPHA)
        r.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"])
        g = r.backward(dev["dy"])
        sync()
        outs.append([r.aux_loss.clone(), r.probs.clone(), g["dlogits"].clone(), g["dw_r"].clone(),
                     g["dx"].clone()])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                           b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16))


def test_aux_at_full_size_skewed_workload():
    """The skewed workload (N=16384, H=2048, F=1408, E=64, K=6) at full size,
    in the configuration the benchmark times: the loss and every probability
    against the oracle's (computed from the oracle's own routing); and, with
    the same routing run once with and once without the loss, the change in
    dlogits equals the oracle's aux gradient and dW_r = x^T dlogits holds over
    every element of the dense result."""
    from mixture_experts_layer_sort_amd.layer import MoELayerRunner
    from moe_workloads import SKEWED
    cfg = SKEWED
    N, E, K = cfg.N, cfg.E, cfg.K
    print(f"[aux-full] {cfg.name}", flush=True)
    cpu, dev = gpu_inputs(cfg, 0, with_dy=True)
    res = {}
    for alpha in (None, ALPHA):
        r = MoELayerRunner(N, cfg.H, cfg.F, E, K, cfg.torch_dtype, "cuda", aux_alpha=alpha)
        r.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"])
        g = r.backward(dev["dy"])
        sync()
        res[alpha] = dict(topk=r.topk.cpu().numpy(), counts=r.counts.cpu().numpy().astype(np.int64),
                          dl=to_np(g["dlogits"]), dw_r=to_np(g["dw_r"]))
        if alpha is not None:
            res[alpha].update(dx=to_np(g["dx"]), dxs=to_np(r.dxs), inv=r.inv.cpu().numpy().astype(np.int64),
                              probs=to_np(r.probs), loss=float(r.aux_loss.item()))
        del r, g
        torch.cuda.empty_cache()
    assert np.array_equal(res[None]["topk"], res[ALPHA]["topk"])
    on = res[ALPHA]

    x, w_r = O.as_f64(cpu["x"]), O.as_f64(cpu["w_r"])
    logits = O.router_logits(x, w_r, O.as_f64(cpu["bias"]))
    counts = O.routing_metadata(O.topk_experts(logits, K), E)[0]
    dcount = np.abs(on["counts"] - counts)          # near-tie swaps only
    assert dcount.sum() <= 2 * max(1, N // 1000), dcount.sum()

    sig = O.gemm_sigma(x, w_r).max(axis=1, keepdims=True)
    p_ref = O.router_probs(logits)
    assert np.all(np.abs(on["probs"] - p_ref) <= 2 * p_ref * sig + 8 * U32), "router probabilities"
    loss_ref = O.aux_loss(logits, counts, K, ALPHA)
    slack = ALPHA * E * (float(dcount.sum()) / (N * K) + 4 * float(sig.max()))
    print(f"loss gpu {on['loss']:.8g} oracle {loss_ref:.8g}", flush=True)
    assert abs(on["loss"] - loss_ref) <= 1e-5 * loss_ref + slack

    _check_aux_dlogits(on["dl"], res[None]["dl"], logits, counts, dcount, sig, N, E, K)
    _check_dw_r_and_dx(x, w_r, on["dl"], on["dw_r"], on["dx"], on["dxs"], on["inv"], K, "bf16")
