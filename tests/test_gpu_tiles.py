"""Every bf16 GEMM tile shape against the oracle, element by element.

The dispatcher picks the GEMM tile shape per stage from the problem size, so
at small sizes only the 128-wide kernels run.  moe_dims.gemm_tiles forces one
family for every stage (256: the 256 x 256 kernels, 8 waves on the
mixed-depth LDS DMA loop; 128x256: the register-staged 128 x 256
kernels; 128: the 128 x 128 kernels and the 128 x 256 LDS DMA dA tiles);
each is run here on inputs
with ragged row tiles, partial column tiles, empty experts, K = E and a single
expert, with the oracle's assignment, and every stored intermediate and
gradient is compared with the oracle under the usual bf16 bars and rounding
bands; a second run of the same family must be bitwise identical.
"""
import numpy as np
import pytest
import torch

from moe_workloads import TEST_CONFIGS, MoEConfig
from oracle import moe_oracle as O
from tests.gpu_common import assert_close, check_runner_steps, gpu_inputs, oracle_fwd, sync

pytestmark = pytest.mark.gpu

CASES = [TEST_CONFIGS["t_bigtile"], TEST_CONFIGS["t_ragged"], TEST_CONFIGS["t_skew"], TEST_CONFIGS["t_keqe"],
         TEST_CONFIGS["t_e1"],
         # several 256-row tiles per expert, F a multiple of 128 but not of 256
         MoEConfig("t_tiles_f640", N=1500, H=384, F=640, E=3, K=2, dtype="bf16")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_sort_amd import _lib
    _lib.lib()


def _family(tiles):
    """moe_gemm_tiles value of a family name (None: the library's choice)."""
    from mixture_experts_layer_sort_amd import _lib as L
    return {None: L.MOE_TILES_AUTO, "256": L.MOE_TILES_256, "128x256": L.MOE_TILES_128X256,
            "128": L.MOE_TILES_128}[tiles]


def _run(cfg, cpu, dev, of, tiles):
    from mixture_experts_layer_sort_amd.layer import MoELayerRunner
    r = MoELayerRunner(cfg.N, cfg.H, cfg.F, cfg.E, cfg.K, cfg.torch_dtype, "cuda", gemm_tiles=_family(tiles))
    y = r.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"],
                  topk=torch.from_numpy(of["topk"]).cuda(),
                  gates=torch.from_numpy(of["gates"].astype(np.float32)).cuda())
    g = r.backward(dev["dy"])
    sync()
    got = {"G": r.g, "U": r.u, "A": r.act, "ys": r.ys, "y": y, "dys": r.dys, "dG": r.dg, "dU": r.du, "dxs": r.dxs,
           "dx": g["dx"], "dw_gate": g["dw_gate"], "dw_up": g["dw_up"], "dw_down": g["dw_down"]}
    return {k: v.clone() for k, v in got.items()}, (r, y, g)


@pytest.mark.parametrize("tiles", ["256", "128x256", "128"])
@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_gemm_tiles_match_oracle(cfg, tiles):
    print(f"[tiles {tiles}] {cfg.name}", flush=True)
    cpu, dev = gpu_inputs(cfg, 11, with_dy=True)
    of = oracle_fwd(cfg, cpu)
    got, (r, y, g) = _run(cfg, cpu, dev, of, tiles)
    check_runner_steps(cfg, cpu, r, y, g)
    del r, y, g
    ob = O.backward(of, cpu["dy"])
    bd = O.rounding_bands(of, ob, cpu["dy"])
    ref = dict(of)
    ref.update(ob)
    for name, t in got.items():
        assert_close(name, t, ref[name], "bf16", band=bd.get(name))
    for e in np.where(of["counts"] == 0)[0]:
        for name in ("dw_gate", "dw_up", "dw_down"):
            assert torch.count_nonzero(got[name][int(e)]).item() == 0
    again, _ = _run(cfg, cpu, dev, of, tiles)
    for name, t in got.items():
        assert torch.equal(t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32),
                           again[name].view(torch.int16) if t.dtype == torch.bfloat16 else again[name].view(torch.int32)), name


@pytest.mark.parametrize("tiles", ["256", "128x256", "128"])
@pytest.mark.parametrize("cfg", [TEST_CONFIGS["t_bigtile"], TEST_CONFIGS["t_ragged"], TEST_CONFIGS["t_skew"],
                                 TEST_CONFIGS["t_f32"], TEST_CONFIGS["t_wide_e"]], ids=lambda c: c.name)
def test_gate_up_gather_equals_permute_then_gate_up(cfg, tiles):
    """moe_ffn_gate_up_gather (rows read as x[sorted_flat / K]) gives the same
    bytes as moe_permute followed by moe_ffn_gate_up, for every tile family."""
    from mixture_experts_layer_sort_amd import _lib as L
    from mixture_experts_layer_sort_amd.layer import MoELayerRunner
    print(f"[gather {tiles}] {cfg.name}", flush=True)
    cpu, dev = gpu_inputs(cfg, 2)
    r = MoELayerRunner(cfg.N, cfg.H, cfg.F, cfg.E, cfg.K, cfg.torch_dtype, "cuda", gather=False,
                       gemm_tiles=_family(tiles))
    r.route(dev["x"], dev["w_r"], dev["bias"])
    r.meta()
    L.moe_permute(r.d, dev["x"], r.sorted_flat, r.xs)
    L.moe_ffn_gate_up(r.d, r.xs, dev["w_gate"], dev["w_up"], r.tiles, r.num_tiles, r.g, r.u, r.act)
    ref = {k: getattr(r, k).clone() for k in ("g", "u", "act")}
    for k in ref:
        getattr(r, k).view(torch.uint8).fill_(0xFF)
    L.moe_ffn_gate_up_gather(r.d, dev["x"], r.sorted_flat, dev["w_gate"], dev["w_up"], r.tiles, r.num_tiles, r.g,
                             r.u, r.act)
    sync()
    for k, v in ref.items():
        assert torch.equal(getattr(r, k).view(torch.uint8), v.view(torch.uint8)), k
    # the forward-only runner takes this path and holds no xs
    f = MoELayerRunner(cfg.N, cfg.H, cfg.F, cfg.E, cfg.K, cfg.torch_dtype, "cuda", backward=False,
                       gemm_tiles=_family(tiles))
    assert f.gather_fused and f.xs is None
    y = f.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"])
    r.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"])
    sync()
    assert torch.equal(y.view(torch.uint8), r.y.view(torch.uint8))


@pytest.mark.parametrize("cfg", [TEST_CONFIGS["t_skew"], TEST_CONFIGS["t_ragged"], TEST_CONFIGS["t_e1"],
                                 MoEConfig("t_tiles_f640", N=1500, H=384, F=640, E=3, K=2, dtype="bf16"),
                                 MoEConfig("t_dxdw_base_shape", N=4096, H=512, F=1024, E=8, K=2, dtype="bf16")],
                         ids=lambda c: c.name)
def test_merged_dx_dw_launch_equals_separate_launches(cfg):
    """moe_ffn_bwd_dx_dw (one launch: weight-gradient tiles first, dX tiles
    after) gives the same bytes as the separate 256 x 256 dX and dW launches,
    on poisoned outputs, with empty experts and ragged tails."""
    from mixture_experts_layer_sort_amd import _lib as L
    from mixture_experts_layer_sort_amd.layer import MoELayerRunner
    print(f"[dx_dw] {cfg.name}", flush=True)
    cpu, dev = gpu_inputs(cfg, 21, with_dy=True)
    r = MoELayerRunner(cfg.N, cfg.H, cfg.F, cfg.E, cfg.K, cfg.torch_dtype, "cuda", gather=False)
    r.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"])
    r.backward(dev["dy"])
    sync()
    outs = []
    for forced in (None, "256"):
        d = L.dims(cfg.N, cfg.H, cfg.F, cfg.E, cfg.K, L.dtype_code(cfg.torch_dtype), _family(forced))
        dxs = torch.full_like(r.dxs, float("nan"))
        dwg, dwu, dwd = (torch.full_like(t, float("nan")) for t in (r.dw_gate, r.dw_up, r.dw_down))
        L.moe_ffn_bwd_dx_dw(d, r.dg, r.du, dev["w_gate"], dev["w_up"], r.tiles, r.num_tiles, dxs, r.xs, r.act,
                            r.dys, r.offsets, dwg, dwu, dwd)
        sync()
        outs.append((dxs, dwg, dwu, dwd))
    nk = int(r.offsets[-1].item())
    for name, a, b in zip(("dxs", "dw_gate", "dw_up", "dw_down"), outs[0], outs[1]):
        if name == "dxs":
            a, b = a[:nk], b[:nk]
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), name
    # and the runner's own backward (merged launch) wrote the same dW
    assert torch.equal(outs[0][1].view(torch.uint8), r.dw_gate.view(torch.uint8))


@pytest.mark.parametrize("cfg", [TEST_CONFIGS["t_skew"], TEST_CONFIGS["t_ragged"], TEST_CONFIGS["t_f32"]],
                         ids=lambda c: c.name)
def test_grouped_entry_points_equal_the_single_gemm_calls(cfg):
    """moe_expert_ffn (gate/up + down) and moe_expert_ffn_bwd (dA, then dX
    and dW) give the same bytes as the per-GEMM calls the layer runner
    makes, on poisoned outputs."""
    from mixture_experts_layer_sort_amd import _lib as L
    from mixture_experts_layer_sort_amd.layer import MoELayerRunner
    cpu, dev = gpu_inputs(cfg, 22, with_dy=True)
    r = MoELayerRunner(cfg.N, cfg.H, cfg.F, cfg.E, cfg.K, cfg.torch_dtype, "cuda", gather=False)
    r.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"])
    r.backward(dev["dy"])
    sync()
    nk = int(r.offsets[-1].item())
    poison = lambda t: torch.full_like(t, float("nan"))
    g, u, a, ys = (poison(t) for t in (r.g, r.u, r.act, r.ys))
    L.moe_expert_ffn(r.d, r.xs, dev["w_gate"], dev["w_up"], dev["w_down"], r.tiles, r.num_tiles, g, u, a, ys)
    dg, du, dxs = (poison(t) for t in (r.dg, r.du, r.dxs))
    dwg, dwu, dwd = (poison(t) for t in (r.dw_gate, r.dw_up, r.dw_down))
    L.moe_expert_ffn_bwd(r.d, r.dys, r.xs, dev["w_gate"], dev["w_up"], dev["w_down"], r.g, r.u, r.act, r.offsets,
                         r.tiles, r.num_tiles, dg, du, dxs, dwg, dwu, dwd)
    sync()
    for name, got, ref in (("G", g, r.g), ("U", u, r.u), ("A", a, r.act), ("ys", ys, r.ys), ("dG", dg, r.dg),
                           ("dU", du, r.du), ("dxs", dxs, r.dxs)):
        assert torch.equal(got[:nk].view(torch.uint8), ref[:nk].view(torch.uint8)), name
    for name, got, ref in (("dw_gate", dwg, r.dw_gate), ("dw_up", dwu, r.dw_up), ("dw_down", dwd, r.dw_down)):
        assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), name


@pytest.mark.parametrize("cfg", [TEST_CONFIGS["t_skew"], TEST_CONFIGS["t_bigtile"], TEST_CONFIGS["t_f32"]],
                         ids=lambda c: c.name)
def test_separate_dx_and_dw_entries(cfg):
    """moe_ffn_bwd_dx and moe_ffn_bwd_dw called on their own: dW is the same
    bytes as the merged launch (same 256 x 256 kernel); dX, whose tile shape
    follows the per-stage choice, is checked against the oracle's dxs for
    the same dG, dU."""
    from mixture_experts_layer_sort_amd import _lib as L
    from mixture_experts_layer_sort_amd.layer import MoELayerRunner
    cpu, dev = gpu_inputs(cfg, 23, with_dy=True)
    r = MoELayerRunner(cfg.N, cfg.H, cfg.F, cfg.E, cfg.K, cfg.torch_dtype, "cuda", gather=False)
    r.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"])
    r.backward(dev["dy"])
    sync()
    nk = int(r.offsets[-1].item())
    dxs = torch.full_like(r.dxs, float("nan"))
    dwg, dwu, dwd = (torch.full_like(t, float("nan")) for t in (r.dw_gate, r.dw_up, r.dw_down))
    L.moe_ffn_bwd_dx(r.d, r.dg, r.du, dev["w_gate"], dev["w_up"], r.tiles, r.num_tiles, dxs)
    L.moe_ffn_bwd_dw(r.d, r.xs, r.act, r.dys, r.dg, r.du, r.offsets, dwg, dwu, dwd)
    sync()
    for name, got, ref in (("dw_gate", dwg, r.dw_gate), ("dw_up", dwu, r.dw_up), ("dw_down", dwd, r.dw_down)):
        assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), name
    # dxs = dG W_gate^T + dU W_up^T per expert, from the device's own dG, dU
    dg, du = O.as_f64(r.dg[:nk]), O.as_f64(r.du[:nk])
    wg, wu = O.as_f64(cpu["w_gate"]), O.as_f64(cpu["w_up"])
    offs = r.offsets.cpu().numpy()
    ref = np.zeros((nk, cfg.H))
    for e in range(cfg.E):
        a, b = offs[e], offs[e + 1]
        ref[a:b] = dg[a:b] @ wg[e].T + du[a:b] @ wu[e].T
    got = O.as_f64(dxs[:nk])
    if cfg.dtype == "f32":
        assert np.max(np.abs(got - ref)) <= 1e-4
    else:
        # one bf16 rounding (half a unit: 2^-9 relative) plus the fp32 summation order
        assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-3), "dxs"


@pytest.mark.parametrize("tiles", [None, "256", "128x256", "128"], ids=lambda t: t or "default")
@pytest.mark.parametrize("cfg", [TEST_CONFIGS["t_skew"], TEST_CONFIGS["t_ragged"], TEST_CONFIGS["t_f32"],
                                 MoEConfig("t_tiles_f640", N=1500, H=384, F=640, E=3, K=2, dtype="bf16")],
                         ids=lambda c: c.name)
def test_gathered_weight_gradients_equal_the_xs_path(cfg, tiles):
    """moe_ffn_bwd_dx_dw_gather (dW_gate and dW_up read x[sorted_flat / K])
    gives the same bytes as moe_permute + moe_ffn_bwd_dx_dw, for every tile
    family and the fp32 path, on poisoned outputs."""
    from mixture_experts_layer_sort_amd import _lib as L
    from mixture_experts_layer_sort_amd.layer import MoELayerRunner
    cpu, dev = gpu_inputs(cfg, 24, with_dy=True)
    r = MoELayerRunner(cfg.N, cfg.H, cfg.F, cfg.E, cfg.K, cfg.torch_dtype, "cuda", gather=False,
                       gemm_tiles=_family(tiles))
    r.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"])
    r.backward(dev["dy"])
    sync()
    nk = int(r.offsets[-1].item())
    dxs = torch.full_like(r.dxs, float("nan"))
    dwg, dwu, dwd = (torch.full_like(t, float("nan")) for t in (r.dw_gate, r.dw_up, r.dw_down))
    L.moe_ffn_bwd_dx_dw_gather(r.d, r.dg, r.du, dev["w_gate"], dev["w_up"], r.tiles, r.num_tiles, dxs, dev["x"],
                               r.sorted_flat, r.act, r.dys, r.offsets, dwg, dwu, dwd)
    sync()
    assert torch.equal(dxs[:nk].view(torch.uint8), r.dxs[:nk].view(torch.uint8))
    for name, got, ref in (("dw_gate", dwg, r.dw_gate), ("dw_up", dwu, r.dw_up), ("dw_down", dwd, r.dw_down)):
        assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), name
