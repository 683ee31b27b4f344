"""moe_route_meta_noalloc (scratch in a library-held device array) against
moe_route_meta (caller workspace), through the C ABI, byte for byte: two
calls in a row on different problems, the second smaller, on both the fused
router + metadata path and the unfused one, with and without a capacity."""
import numpy as np
import pytest
import torch

from moe_workloads import MoEConfig, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_sort_amd import _lib
    _lib.lib()


def _outputs(L, d, N, K, E):
    i32, dev = torch.int32, "cuda"
    mt = L.moe_max_tiles(d)
    return dict(topk=torch.full((N, K), -7, dtype=i32, device=dev),
                gates=torch.full((N, K), float("nan"), dtype=torch.float32, device=dev),
                sorted_flat=torch.full((N * K,), -7, dtype=i32, device=dev),
                inv=torch.full((N * K,), -7, dtype=i32, device=dev),
                counts=torch.full((E,), -7, dtype=i32, device=dev),
                offsets=torch.full((E + 1,), -7, dtype=i32, device=dev),
                tiles=torch.full((3 * mt,), -7, dtype=i32, device=dev),
                num_tiles=torch.full((1,), -7, dtype=i32, device=dev))


def _run(cfg, capacity, seed):
    from mixture_experts_layer_sort_amd import _lib as L
    inp = make_inputs(cfg, seed, device="cuda")
    d = L.dims(cfg.N, cfg.H, cfg.F, cfg.E, cfg.K, L.dtype_code(cfg.torch_dtype))
    need = L.moe_workspace_bytes(d, L.MOE_ENTRY_ROUTE_META)
    assert 0 < need <= L.MOE_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ref = _outputs(L, d, cfg.N, cfg.K, cfg.E)
    L.moe_route_meta(d, inp["x"], inp["w_r"], inp["bias"], capacity, ref["topk"], ref["gates"], ref["sorted_flat"],
                     ref["inv"], ref["counts"], ref["offsets"], ref["tiles"], ref["num_tiles"], ws)
    got = _outputs(L, d, cfg.N, cfg.K, cfg.E)
    L.moe_route_meta_noalloc(d, inp["x"], inp["w_r"], inp["bias"], capacity, got["topk"], got["gates"],
                             got["sorted_flat"], got["inv"], got["counts"], got["offsets"], got["tiles"],
                             got["num_tiles"])
    torch.cuda.synchronize()
    nt = int(ref["num_tiles"].item())
    assert 0 < nt <= L.moe_max_tiles(d)
    for k in ref:
        a, b = ref[k], got[k]
        if k == "tiles":
            a, b = a[:3 * nt], b[:3 * nt]
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (cfg.name, k)
    return need


INT_MAX = 2 ** 31 - 1
# (first, second): the second call smaller than the first
PAIRS = [
    # unfused metadata (ceil(N/32) * E > 32768), then the fused path
    ((MoEConfig("na_unfused", N=8192, H=1024, F=128, E=256, K=8, dtype="bf16"), INT_MAX),
     (MoEConfig("na_fused_small", N=2000, H=512, F=128, E=8, K=2, dtype="bf16"), INT_MAX)),
    # fused path twice, with a binding capacity, then a smaller dropless call
    ((MoEConfig("na_fused", N=16384, H=512, F=128, E=8, K=2, dtype="bf16"), 3000),
     (MoEConfig("na_fused_skew", N=600, H=128, F=128, E=16, K=2, dtype="bf16", zipf_s=1.2, zipf_tau=3.0), INT_MAX)),
]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0][0].name}-then-{p[1][0].name}")
def test_noalloc_equals_route_meta_twice(pair):
    (c1, cap1), (c2, cap2) = pair
    print(f"[noalloc] {c1.name} then {c2.name}", flush=True)
    n1 = _run(c1, cap1, 1)
    n2 = _run(c2, cap2, 2)
    assert c2.N * c2.K < c1.N * c1.K and n2 <= n1
