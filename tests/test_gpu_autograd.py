"""The torch.autograd wrapper (moe_layer / MoEFunction) on the GPU: the same
bytes as the layer runner it drives, with and without the optional parts
(shared expert, expert capacity, load-balancing loss, weight gradients
gathered from x), and end to end against the CPU oracle on the tiny fp32
workload.
"""
import numpy as np
import pytest
import torch

from moe_workloads import TEST_CONFIGS, TINY, make_shared_weights
from oracle import moe_oracle as O
from tests.gpu_common import gpu_inputs, sync, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_sort_amd import _lib
    _lib.lib()


def _leaf(t):
    return t.detach().clone().requires_grad_(True)


def _bytes_equal(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.mark.parametrize("opts", ["plain", "all"])
@pytest.mark.parametrize("cfg", [TEST_CONFIGS["t_skew"], TEST_CONFIGS["t_ragged"], TEST_CONFIGS["t_f32"]],
                         ids=lambda c: c.name)
def test_moe_layer_equals_the_runner(cfg, opts):
    from mixture_experts_layer_sort_amd.layer import MoELayerRunner, moe_layer
    cpu, dev = gpu_inputs(cfg, 41, with_dy=True)
    Fs = 256
    kw = {}
    rkw = {}
    shared = None
    if opts == "all":
        shared = tuple(w.cuda() for w in make_shared_weights(cfg, 41, Fs))
        C = O.capacity_of(cfg.N, cfg.K, cfg.E, 1.0)
        kw = dict(capacity=C, shared=tuple(_leaf(w) for w in shared), aux_alpha=0.5, aux_grad=1.0, dw_gather=True)
        rkw = dict(capacity=C, shared_ffn=Fs, aux_alpha=0.5, dw_gather=True)
    leaves = {k: _leaf(dev[k]) for k in ("x", "w_r", "w_gate", "w_up", "w_down")}
    out = moe_layer(leaves["x"], leaves["w_r"], leaves["w_gate"], leaves["w_up"], leaves["w_down"], cfg.K,
                    dev["bias"], **kw)
    y, aux = (out if opts == "all" else (out, None))
    y.backward(dev["dy"])
    sync()
    r = MoELayerRunner(cfg.N, cfg.H, cfg.F, cfg.E, cfg.K, cfg.torch_dtype, "cuda", **rkw)
    yr = r.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"], shared=shared)
    g = r.backward(dev["dy"], aux_grad=1.0)
    sync()
    assert _bytes_equal(y.detach(), yr)
    assert _bytes_equal(leaves["x"].grad, g["dx"])
    for k in ("w_r", "w_gate", "w_up", "w_down"):
        assert _bytes_equal(leaves[k].grad, g["d" + k].to(cfg.torch_dtype)), k
    if opts == "all":
        assert _bytes_equal(aux, r.aux_loss) and not aux.requires_grad
        for leaf, name in zip(kw["shared"], ("dw_gate_s", "dw_up_s", "dw_down_s")):
            assert _bytes_equal(leaf.grad, g[name].to(cfg.torch_dtype)), name


def test_moe_layer_matches_the_oracle_end_to_end():
    """Tiny fp32 workload: y and every gradient from autograd against the
    float64 oracle, to the fp32 bar."""
    from mixture_experts_layer_sort_amd.layer import moe_layer
    cfg = TINY
    cpu, dev = gpu_inputs(cfg, 42, with_dy=True)
    leaves = {k: _leaf(dev[k]) for k in ("x", "w_r", "w_gate", "w_up", "w_down")}
    y = moe_layer(leaves["x"], leaves["w_r"], leaves["w_gate"], leaves["w_up"], leaves["w_down"], cfg.K)
    y.backward(dev["dy"])
    sync()
    of = O.forward(cpu["x"], cpu["w_r"], cpu["w_gate"], cpu["w_up"], cpu["w_down"], cfg.K, store="f32")
    ob = O.backward(of, cpu["dy"])
    assert np.max(np.abs(to_np(y.detach()) - of["y"])) <= 1e-4
    assert np.max(np.abs(to_np(leaves["x"].grad) - ob["dx"])) <= 1e-4
    for k in ("w_r", "w_gate", "w_up", "w_down"):
        assert np.max(np.abs(to_np(leaves[k].grad) - ob["d" + k])) <= 1e-4, k
