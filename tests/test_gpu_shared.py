"""Parity of the shared expert on the GPU (through the C ABI) with the CPU
oracle.

A shared expert is one dense SwiGLU expert that every token passes through
with weight 1, its output added to the routed combine ("MegaBlocks -
architecture and principles", section 2.1).  Checked: the whole forward and
backward against the oracle (routed and shared intermediates, y, dx and all
eight weight gradients) on ragged shapes, the fp32 storage type, a split
weight-gradient contraction with a short last chunk, and the default workload
at full size; a zero down projection leaves every routed result unchanged;
the side-stream schedule gives the same bits; the dense gather backward (with
the load-balancing loss) adds the shared input gradient; and the shared
expert together with a binding expert capacity.
"""
import numpy as np
import pytest
import torch

from moe_workloads import BASE, TEST_CONFIGS, MoEConfig, make_shared_weights
from oracle import moe_oracle as O
from tests.gpu_common import assert_close, check_runner_steps, gpu_inputs, store_of, sync, to_np

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_sort_amd import _lib
    _lib.lib()


def _runner(cfg, Fs, **kw):
    from mixture_experts_layer_sort_amd.layer import MoELayerRunner
    return MoELayerRunner(cfg.N, cfg.H, cfg.F, cfg.E, cfg.K, cfg.torch_dtype, "cuda", shared_ffn=Fs, **kw)


def _assignment(of):
    return (torch.from_numpy(of["topk"]).cuda(), torch.from_numpy(of["gates"].astype(np.float32)).cuda())


CASES = [(TEST_CONFIGS["t_skew"], 256), (TEST_CONFIGS["t_ragged"], 512), (TEST_CONFIGS["t_f32"], 256),
         (TEST_CONFIGS["t_k1"], 384), (TEST_CONFIGS["t_bigtile"], 1024),
         (MoEConfig("t_sh_chunks", N=1500, H=256, F=256, E=4, K=2, dtype="bf16"), 768), (BASE, 1024)]


@pytest.mark.parametrize("cfg,Fs", CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_shared_layer_matches_oracle(cfg, Fs):
    print(f"[shared] {cfg.name} Fs={Fs}", flush=True)
    cpu, dev = gpu_inputs(cfg, 12, with_dy=True)
    ws_cpu = make_shared_weights(cfg, 12, Fs)
    ws_dev = tuple(w.cuda() for w in ws_cpu)
    dt = store_of(cfg)
    of = O.forward(cpu["x"], cpu["w_r"], cpu["w_gate"], cpu["w_up"], cpu["w_down"], cfg.K, bias=cpu["bias"],
                   store=dt, tile_m=256, shared=tuple(O.as_f64(w) for w in ws_cpu))
    r = _runner(cfg, Fs)
    topk, gates = _assignment(of)
    y = r.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"], topk=topk,
                  gates=gates, shared=ws_dev)
    g = r.backward(dev["dy"])
    sync()
    ob = O.backward(of, cpu["dy"])
    bd = O.rounding_bands(of, ob, cpu["dy"]) if dt == "bf16" else {}
    sh = of["shared"]
    ref = dict(of)
    ref.update(ob)
    ref.update(G_s=sh["G"], U_s=sh["U"], A_s=sh["A"], ys_s=sh["ys"])
    got = {"G_s": r.g_s, "U_s": r.u_s, "A_s": r.act_s, "ys_s": r.ys_s, "dG_s": r.dg_s, "dU_s": r.du_s,
           "dxs_s": r.dx_s, "G": r.g, "U": r.u, "A": r.act, "ys": r.ys, "dG": r.dg, "dU": r.du, "dxs": r.dxs,
           "y": y, "dx": g["dx"], "dgates": g["dgates"], "dlogits": g["dlogits"], "dw_r": g["dw_r"],
           "dw_gate": g["dw_gate"], "dw_up": g["dw_up"], "dw_down": g["dw_down"], "dw_gate_s": g["dw_gate_s"],
           "dw_up_s": g["dw_up_s"], "dw_down_s": g["dw_down_s"]}
    for name, t in got.items():
        assert_close(name, t, ref[name], dt, band=bd.get(name))
    check_runner_steps(cfg, cpu, r, y, g, shared=ws_cpu)


def test_zero_down_projection_leaves_routed_results_unchanged():
    cfg, Fs = TEST_CONFIGS["t_ragged"], 256
    cpu, dev = gpu_inputs(cfg, 13, with_dy=True)
    wg, wu, _ = (w.cuda() for w in make_shared_weights(cfg, 13, Fs))
    wd = torch.zeros((Fs, cfg.H), dtype=cfg.torch_dtype, device="cuda")
    from mixture_experts_layer_sort_amd.layer import MoELayerRunner
    r0 = MoELayerRunner(cfg.N, cfg.H, cfg.F, cfg.E, cfg.K, cfg.torch_dtype, "cuda")
    y0 = r0.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"]).clone()
    g0 = {k: v.clone() for k, v in r0.backward(dev["dy"]).items()}
    r = _runner(cfg, Fs)
    y = r.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"], shared=(wg, wu, wd))
    g = r.backward(dev["dy"])
    sync()
    assert torch.equal(y, y0)          # values: +0 and -0 may differ in sign only
    for k, v in g0.items():
        assert torch.equal(g[k], v), k
    assert torch.count_nonzero(r.dx_s).item() == 0 and torch.count_nonzero(g["dw_gate_s"]).item() == 0
    ref = to_np(r.act_s).T @ to_np(dev["dy"])
    assert np.all(np.abs(to_np(g["dw_down_s"]) - ref) <= O.gemm_sigma(to_np(r.act_s).T, to_np(dev["dy"]))
                  + 2 * U32 * np.abs(ref))


@pytest.mark.parametrize("cfg,Fs", [(TEST_CONFIGS["t_skew"], 256), (BASE, 1024)], ids=lambda v: getattr(v, "name", str(v)))
def test_side_stream_schedule_is_bitwise_identical(cfg, Fs):
    cpu, dev = gpu_inputs(cfg, 14, with_dy=True)
    ws = tuple(w.cuda() for w in make_shared_weights(cfg, 14, Fs))
    outs = []
    for side in (None, torch.cuda.Stream()):
        r = _runner(cfg, Fs)
        y = r.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"], shared=ws,
                      side_stream=side)
        g = r.backward(dev["dy"], side_stream=side)
        sync()
        outs.append({k: v.clone() for k, v in dict(y=y, **g).items()})
    for k, v in outs[0].items():
        assert torch.equal(v.view(torch.uint8), outs[1][k].view(torch.uint8)), k


@pytest.mark.parametrize("cfg", [TEST_CONFIGS["t_skew"], TEST_CONFIGS["t_ragged"],
                                 MoEConfig("t_aux_f32_e12", N=150, H=128, F=256, E=12, K=2, dtype="f32")],
                         ids=lambda c: c.name)
def test_dense_gather_backward_adds_the_shared_gradient(cfg):
    """With the load-balancing loss on, dx = sum_k dxs[inv] + dlogits W_r^T +
    dx_shared over every element (dense router term; token-tiled for E > 8),
    and every routed result equals the run without the shared expert."""
    Fs = 256
    cpu, dev = gpu_inputs(cfg, 15, with_dy=True)
    ws = tuple(w.cuda() for w in make_shared_weights(cfg, 15, Fs))
    from mixture_experts_layer_sort_amd.layer import MoELayerRunner
    r0 = MoELayerRunner(cfg.N, cfg.H, cfg.F, cfg.E, cfg.K, cfg.torch_dtype, "cuda", aux_alpha=0.5)
    r0.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"])
    g0 = {k: v.clone() for k, v in r0.backward(dev["dy"]).items()}
    r = _runner(cfg, Fs, aux_alpha=0.5)
    r.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"], shared=ws)
    g = r.backward(dev["dy"])
    sync()
    for k in ("dlogits", "dw_r", "dw_gate", "dw_up", "dw_down", "dgates"):
        assert torch.equal(g[k], g0[k]), k
    dl, dxs, inv = to_np(g["dlogits"]), to_np(r.dxs), r.inv.cpu().numpy()
    w_r, dxsh = to_np(dev["w_r"]), to_np(r.dx_s)
    rows = dxs[inv.reshape(-1, cfg.K)]
    pre = rows.sum(axis=1) + dl @ w_r.T + dxsh
    sig = (8 * U32 * (np.abs(rows).sum(axis=1) + np.abs(dl) @ np.abs(w_r.T) + np.abs(dxsh))
           + O.gemm_sigma(dl, w_r.T))
    dx = to_np(g["dx"])
    if cfg.dtype == "f32":
        assert np.all(np.abs(dx - pre) <= sig)
    else:
        rounded = O.round_bf16(pre)
        assert np.all(np.abs(dx - rounded) <= O.bf16_flip(pre, rounded, sig))


def test_shared_expert_with_binding_capacity():
    cfg, Fs = TEST_CONFIGS["t_skew"], 384
    C = O.capacity_of(cfg.N, cfg.K, cfg.E, 1.0)
    cpu, dev = gpu_inputs(cfg, 16, with_dy=True)
    ws_cpu = make_shared_weights(cfg, 16, Fs)
    of = O.forward(cpu["x"], cpu["w_r"], cpu["w_gate"], cpu["w_up"], cpu["w_down"], cfg.K, bias=cpu["bias"],
                   store="bf16", tile_m=256, capacity=C, shared=tuple(O.as_f64(w) for w in ws_cpu))
    assert int(of["offsets"][-1]) < cfg.N * cfg.K
    r = _runner(cfg, Fs, capacity=C)
    topk, gates = _assignment(of)
    y = r.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"], topk=topk,
                  gates=gates, shared=tuple(w.cuda() for w in ws_cpu))
    g = r.backward(dev["dy"])
    sync()
    ob = O.backward(of, cpu["dy"])
    bd = O.rounding_bands(of, ob, cpu["dy"])
    ref = dict(of)
    ref.update(ob)
    for name, t in dict(y=y, **g).items():
        assert_close(name, t, ref[name], "bf16", band=bd.get(name))
    check_runner_steps(cfg, cpu, r, y, g, capacity=C, shared=ws_cpu)


def test_forward_only_runner_with_shared_expert_equals_training_forward():
    """Without a backward the shared expert keeps no G/U (g_save = u_save =
    NULL) and the routed gather is fused into gate/up; y is the same bytes."""
    cfg, Fs = TEST_CONFIGS["t_ragged"], 512
    cpu, dev = gpu_inputs(cfg, 17)
    ws = tuple(w.cuda() for w in make_shared_weights(cfg, 17, Fs))
    f = _runner(cfg, Fs, backward=False)
    t = _runner(cfg, Fs)
    assert f.g_s is None and f.gather_fused
    yf = f.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"], shared=ws)
    yt = t.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"], shared=ws)
    sync()
    assert torch.equal(yf.view(torch.uint8), yt.view(torch.uint8))
