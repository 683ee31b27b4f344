"""The 256 x 256 GEMM tiles' mixed-depth LDS DMA K loop at its edge lengths.

That loop keeps operand A one K tile (64 deep) ahead in two LDS slots and
operand B two tiles ahead in three, so its prologue, its last two steps and
the weight gradients' ragged last tile are where it could go wrong.  Here
the experts get 0, 1, 63, 64, 65, 128, 129 and 191 rows (K = 1, a given
assignment): weight-gradient contractions of one, two and three K tiles,
full and ragged (1 and 63 valid rows in the last tile), and an empty expert.
H = F = 128 (the smallest the library takes) give gate/up, dA and down two K
tiles and dX four; H = 384 and F = 256 give six, six, four and eight.  Both
the library's own tile choice (at these sizes the 128-wide tiles for the
forward GEMMs and dA, the 256 x 256 tile for the merged dX / weight-gradient
launch) and the forced 256 x 256 family (every stage on the DMA loop) run,
with xs and with the weight gradients' rows gathered from x, and everything
is compared with the oracle element by element under the usual bf16 bars and
rounding bands.
"""
import numpy as np
import pytest
import torch

from moe_workloads import MoEConfig
from oracle import moe_oracle as O
from tests.gpu_common import assert_close, gpu_inputs, sync

pytestmark = pytest.mark.gpu

COUNTS = [0, 1, 63, 64, 65, 128, 129, 191]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_sort_amd import _lib
    _lib.lib()


def _assignment(counts, seed=5):
    topk = np.concatenate([np.full(c, e, dtype=np.int64) for e, c in enumerate(counts)])
    np.random.default_rng(seed).shuffle(topk)
    return topk.reshape(-1, 1)


@pytest.mark.parametrize("dw_gather", [False, True], ids=["xs", "gathered"])
@pytest.mark.parametrize("tiles", ["auto", "256"])
@pytest.mark.parametrize("H,F", [(128, 128), (384, 256)], ids=["h128_f128", "h384_f256"])
def test_dma_loop_edge_lengths(H, F, tiles, dw_gather):
    from mixture_experts_layer_sort_amd import _lib as L
    from mixture_experts_layer_sort_amd.layer import MoELayerRunner

    cfg = MoEConfig(f"t_dma_h{H}_f{F}", N=sum(COUNTS), H=H, F=F, E=len(COUNTS), K=1, dtype="bf16")
    print(f"[dma edges] H={H} F={F} tiles={tiles} dw_gather={dw_gather}", flush=True)
    cpu, dev = gpu_inputs(cfg, 21, with_dy=True)
    topk = _assignment(COUNTS)
    of = O.forward(cpu["x"], cpu["w_r"], cpu["w_gate"], cpu["w_up"], cpu["w_down"], cfg.K, bias=cpu["bias"],
                   store="bf16", topk=topk)
    assert list(of["counts"]) == COUNTS
    fam = L.MOE_TILES_AUTO if tiles == "auto" else L.MOE_TILES_256
    r = MoELayerRunner(cfg.N, cfg.H, cfg.F, cfg.E, cfg.K, cfg.torch_dtype, "cuda", gemm_tiles=fam,
                       dw_gather=dw_gather)
    y = r.forward(dev["x"], dev["w_r"], dev["w_gate"], dev["w_up"], dev["w_down"], dev["bias"],
                  topk=torch.from_numpy(of["topk"].astype(np.int32)).cuda(),
                  gates=torch.from_numpy(of["gates"].astype(np.float32)).cuda())
    g = r.backward(dev["dy"])
    sync()
    got = {"G": r.g, "U": r.u, "A": r.act, "ys": r.ys, "y": y, "dys": r.dys, "dG": r.dg, "dU": r.du, "dxs": r.dxs,
           "dw_gate": g["dw_gate"], "dw_up": g["dw_up"], "dw_down": g["dw_down"]}
    ob = O.backward(of, cpu["dy"])
    bd = O.rounding_bands(of, ob, cpu["dy"])
    ref = dict(of)
    ref.update(ob)
    for name, t in got.items():
        assert_close(name, t, ref[name], "bf16", band=bd.get(name))
    for name in ("dw_gate", "dw_up", "dw_down"):
        assert torch.count_nonzero(got[name][0]).item() == 0, name  # the empty expert's gradients are exact zeros
