"""The router and the routing metadata fused into two launches
(moe_route_meta) against the unfused calls (moe_route, then
moe_permute_meta_capacity), byte for byte on poisoned outputs: top-K, gates,
counts, offsets, sorted_flat, inv, the tile list and its length.  Covers both
router paths (matrix cores and fp32 / E % 8 != 0), K = 1 .. 8, one expert,
256 experts, a binding capacity and capacity 0, ragged last blocks, and the
fallback to the unfused kernels when the block histograms are too many to
re-read (ceil(N/32) * E > 32768).  The unfused metadata is checked against
the oracle in the parity tests.
"""
import numpy as np
import pytest
import torch

from moe_workloads import BASE, SKEWED, TEST_CONFIGS, TINY, MoEConfig
from oracle import moe_oracle as O
from tests.gpu_common import gpu_inputs, sync

pytestmark = pytest.mark.gpu

INT_MAX = 2 ** 31 - 1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_sort_amd import _lib
    _lib.lib()


def _bufs(cfg):
    from mixture_experts_layer_sort_amd import _lib as L
    d = L.dims(cfg.N, cfg.H, cfg.F, cfg.E, cfg.K, L.dtype_code(cfg.torch_dtype))
    mt = L.moe_max_tiles(d)
    i32 = dict(dtype=torch.int32, device="cuda")
    b = dict(topk=torch.full((cfg.N, cfg.K), -7, **i32), gates=torch.full((cfg.N, cfg.K), float("nan"), device="cuda"),
             sorted_flat=torch.full((cfg.NK,), -7, **i32), inv=torch.full((cfg.NK,), -7, **i32),
             counts=torch.full((cfg.E,), -7, **i32), offsets=torch.full((cfg.E + 1,), -7, **i32),
             tiles=torch.full((3 * max(1, mt),), -7, **i32), num_tiles=torch.full((1,), -7, **i32))
    return d, b


def _ws(d, entry):
    from mixture_experts_layer_sort_amd import _lib as L
    n = L.moe_workspace_bytes(d, entry)
    return torch.full((max(16, n),), 0x5A, dtype=torch.uint8, device="cuda")


CASES = [(TEST_CONFIGS["t_skew"], None), (TEST_CONFIGS["t_skew"], 1.0), (TEST_CONFIGS["t_ragged"], None),
         (TEST_CONFIGS["t_ragged"], 0.75), (TEST_CONFIGS["t_k1"], None), (TEST_CONFIGS["t_keqe"], None),
         (TEST_CONFIGS["t_e1"], None), (TEST_CONFIGS["t_wide_e"], None), (TEST_CONFIGS["t_f32"], 0.8),
         (TEST_CONFIGS["t_bigtile"], None), (TINY, None), (BASE, None), (BASE, 1.0), (SKEWED, None),
         (SKEWED, 1.25), (TEST_CONFIGS["t_skew"], 0.0),
         # E % 8 != 0 on bf16 (vector-ALU router) with K = 5
         (MoEConfig("t_rm_e13_k5", N=777, H=256, F=128, E=13, K=5, dtype="bf16"), None),
         # too many block histograms to re-read: the unfused kernels run
         (MoEConfig("t_rm_fallback", N=8192, H=256, F=128, E=256, K=8, dtype="bf16"), None),
         (MoEConfig("t_rm_fallback_cap", N=8192, H=256, F=128, E=256, K=8, dtype="bf16"), 1.0)]


@pytest.mark.parametrize("cfg,cf", CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_route_meta_equals_route_then_meta(cfg, cf):
    from mixture_experts_layer_sort_amd import _lib as L
    print(f"[route_meta] {cfg.name} cf={cf}", flush=True)
    cpu, dev = gpu_inputs(cfg, 31)
    C = INT_MAX if cf is None else O.capacity_of(cfg.N, cfg.K, cfg.E, cf)
    d, a = _bufs(cfg)
    L.moe_route(d, dev["x"], dev["w_r"], dev["bias"], a["topk"], a["gates"])
    L.moe_permute_meta_capacity(d, a["topk"], C, a["sorted_flat"], a["inv"], a["counts"], a["offsets"], a["tiles"],
                                a["num_tiles"], _ws(d, L.MOE_ENTRY_PERMUTE_META))
    _, b = _bufs(cfg)
    L.moe_route_meta(d, dev["x"], dev["w_r"], dev["bias"], C, b["topk"], b["gates"], b["sorted_flat"], b["inv"],
                     b["counts"], b["offsets"], b["tiles"], b["num_tiles"], _ws(d, L.MOE_ENTRY_ROUTE_META))
    sync()
    nt = int(a["num_tiles"].item())
    assert nt == int(b["num_tiles"].item())
    for k in ("topk", "gates", "sorted_flat", "inv", "counts", "offsets"):
        assert torch.equal(a[k].view(torch.uint8) if k == "gates" else a[k],
                           b[k].view(torch.uint8) if k == "gates" else b[k]), k
    assert torch.equal(a["tiles"][:3 * nt], b["tiles"][:3 * nt])
    if cf is not None and cf > 0:
        assert int(b["offsets"][-1].item()) <= cfg.NK


def test_runner_forward_uses_the_fused_call_and_matches_the_oracle_metadata():
    from mixture_experts_layer_sort_amd.layer import MoELayerRunner
    cfg = TEST_CONFIGS["t_skew"]
    cpu, dev = gpu_inputs(cfg, 32)
    r = MoELayerRunner(cfg.N, cfg.H, cfg.F, cfg.E, cfg.K, cfg.torch_dtype, "cuda", backward=False)
    r.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"])
    sync()
    topk = r.topk.cpu().numpy().astype(np.int64)
    counts, offsets, sf, inv = O.routing_metadata(topk, cfg.E)
    assert np.array_equal(r.counts.cpu().numpy(), counts)
    assert np.array_equal(r.offsets.cpu().numpy(), offsets)
    assert np.array_equal(r.sorted_flat.cpu().numpy(), sf)
    assert np.array_equal(r.inv.cpu().numpy(), inv)
