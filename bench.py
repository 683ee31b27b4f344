"""Benchmark of the dropless top-k MoE layer (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

A step is one pass of the whole layer over one batch of synthetic input:
route, routing metadata, gather, gate/up and down grouped GEMMs, combine,
and (for configurations with a backward) the combine, router, expert and
gather backward passes.  Inputs are resident in HBM before the timed
region; W untimed warm-up steps run first, then exactly K timed steps
bracketed by torch.cuda.synchronize().

Prints one JSON line: throughput in tokens/s (value), the per-stage
breakdown from an untimed event-instrumented pass, the grouped-GEMM rate as
a fraction of the bf16 MFMA peak, a roofline entry for the dominant kernel
(its duration measured with HIP events on the launch stream during the timed
steps), and the CPU oracle timed on the host as a reported baseline.
"""
from __future__ import annotations

import argparse
import math
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# HBM bytes per launch of each GEMM stage, from two rocprofv3 --pmc runs of
# this benchmark (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled
# by what the same counter reads for the plain copy of --copy-calibration
# (FETCH_SIZE x 2.0000, WRITE_SIZE x 1.0000; FETCH_SIZE counts this GPU's
# 128-byte read requests as 64 bytes, which the L2's read requests by size
# confirm for every kernel).  The readings belong to the kernel sources whose
# hash is stored with them; once any source under csrc/ changes, the figure
# is reported as null until the counters are taken again.
TRAFFIC = {
    "sources": "3416889ba7e8276e",
    "bytes": {
        ('bf16_fwd_n8192_h7168_f2048_e256_k8', 'down'): 12791171584,
        ('bf16_fwd_n8192_h7168_f2048_e256_k8', 'gate_up'): 22410343765,
        ('bf16_n16384_h4096_f14336_e8_k2', 'dact'): 10616806741,
        ('bf16_n16384_h4096_f14336_e8_k2', 'down'): 7964579563,
        ('bf16_n16384_h4096_f14336_e8_k2', 'dx_dw'): 42883770901,
        ('bf16_n16384_h4096_f14336_e8_k2', 'gate_up'): 17380177856,
        ('bf16_n16384_h512_f1024_e8_k2', 'dact'): 352213269,
        ('bf16_n16384_h512_f1024_e8_k2', 'down'): 148100416,
        ('bf16_n16384_h512_f1024_e8_k2', 'dx_dw'): 668934891,
        ('bf16_n16384_h512_f1024_e8_k2', 'gate_up'): 338635456,
        ('bf16_skewed_n16384_h2048_f1408_e64_k6', 'dact'): 2819030315,
        ('bf16_skewed_n16384_h2048_f1408_e64_k6', 'down'): 1923069099,
        ('bf16_skewed_n16384_h2048_f1408_e64_k6', 'dx_dw'): 9121219861,
        ('bf16_skewed_n16384_h2048_f1408_e64_k6', 'gate_up'): 3910642133,
    },
}

def kernel_sources_hash():
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "mixture_experts_layer_sort_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(cfg_name, stage):
    if kernel_sources_hash() != TRAFFIC["sources"]:
        return None
    return TRAFFIC["bytes"].get((cfg_name, stage))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    # the largest fwd+bwd workload that fits one GPU: the large-FFN deterministic one
    p.add_argument("--config", default="bf16_n16384_h4096_f14336_e8_k2")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--aux-alpha", type=float, default=None,
                   help="also compute the Switch load-balancing loss with this weight (forward and its gradient)")
    p.add_argument("--capacity-factor", type=float, default=None,
                   help="token-dropping variant: expert capacity ceil(cf * N * K / E), overflow dropped")
    p.add_argument("--shared-ffn", type=int, default=None,
                   help="add a shared expert of this intermediate size that every token passes through")
    p.add_argument("--dw-gather", action="store_true",
                   help="weight gradients read the x rows through sorted_flat: no grouped copy xs (less memory)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain 1 GiB streaming copy (for scaling HBM byte counters) and exit")
    return p.parse_args()


COPY_BYTES = 2 ** 30


def copy_calibration():
    """A plain streaming copy of known size, dst = -src over COPY_BYTES of
    float32 each way, run 3 times.  Under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
    it gives the factor that turns those counters into bytes on this chip."""
    import torch

    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES, "launches": 3}}),
          flush=True)


def stage_flops(cfg, rows=None, shared_ffn=None):
    """Algorithmic flops of the grouped GEMMs over `rows` routed rows (all
    N*K by default; the kept rows of the token-dropping variant), and of the
    shared expert's GEMMs over all N tokens when it is on."""
    hf = cfg.H * cfg.F * (cfg.NK if rows is None else rows)
    # dx_dw: dX (4 H F per row) and the three weight gradients (6 H F) in one launch
    out = {"gate_up": 4 * hf, "down": 2 * hf, "dact": 2 * hf, "dx_dw": 10 * hf}
    if shared_ffn is not None:
        hs = cfg.H * shared_ffn * cfg.N
        out["shared_ffn"] = 6 * hs
        if cfg.backward:
            out["shared_bwd"] = 12 * hs
    return out


def gemm_bytes(cfg, rows, experts_used, save_gu):
    """Algorithmic HBM bytes of the grouped-GEMM stages over `rows` routed
    rows: each operand row and each used expert's weights read once, each
    output written once (dG and dU counted once in the merged dX/dW launch;
    the fp32 weight gradients of all E experts are written, empty ones as
    zeros)."""
    e = 2 if cfg.dtype == "bf16" else 4
    H, F = cfg.H, cfg.F
    w = experts_used * H * F * e
    return {
        "gate_up": rows * H * e + 2 * w + (3 if save_gu else 1) * rows * F * e,
        "down": rows * F * e + w + rows * H * e,
        "dact": rows * H * e + w + 4 * rows * F * e,
        "dx_dw": 2 * rows * F * e + 2 * w + rows * H * e + 2 * rows * H * e + rows * F * e + 3 * cfg.E * H * F * 4,
    }


# stages that are one call of several launches (not a single kernel)
COMPOSITE = {"route_meta", "route_bwd", "permute_bwd", "shared_ffn", "shared_bwd"}


def stage_bytes(cfg, aux=False, shared=False):
    """Algorithmic HBM bytes of the row-movement and metadata stages."""
    e = 2 if cfg.dtype == "bf16" else 4
    N, NK, H, E, K = cfg.N, cfg.NK, cfg.H, cfg.E, cfg.K
    out = {
        # router (x and W_r read, top-K and gates written) + metadata (topk read,
        # sorted_flat and inv written, counts and offsets)
        "route_meta": N * H * e + H * E * e + N * K * 8 + NK * 4 + NK * 8 + (2 * E + 1) * 4,
        "permute": (N + NK) * H * e + NK * 4,           # read each token once (cached), write NK rows
        "combine": (NK + N) * H * e + NK * 8,
        "combine_bwd": (N + 2 * NK) * H * e + NK * 12,
        "permute_bwd": (NK + N) * H * e + NK * 8 + N * K * 4,
        "route_bwd": N * H * e + N * K * 12 + N * E * 4 + H * E * 4,
    }
    if aux:
        # load-balancing loss: x and W_r read, probabilities [N, E] written;
        # its gradient reads them back (dense dlogits) and dx reads all E
        out["aux_loss"] = N * H * e + H * E * e + N * E * 4 + E * 4
        out["route_bwd"] += 2 * N * E * 4
        out["permute_bwd"] += N * E * 4
    if shared:
        # the shared expert's output / input gradient: one more [N, H] read
        out["combine"] += N * H * e
        out["permute_bwd"] += N * H * e
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this layer runs on one GPU; --gpus {args.gpus} is not supported "
              "(no sharding or collectives are built)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import numpy as np
    import torch

    from mixture_experts_layer_sort_amd import _lib as L
    from mixture_experts_layer_sort_amd.layer import MoELayerRunner
    from moe_workloads import get_config, make_inputs, make_shared_weights

    cfg = get_config(args.config)
    torch.cuda.set_device(0)
    dev = "cuda:0"
    big = cfg.E * cfg.H * cfg.F * 3 * 2 > 8 * 2 ** 30
    if big:
        # generate the weights expert by expert on the device (same recipe and
        # seeds, device generator): the host copy would be tens of GB
        inp = make_inputs(cfg, args.seed, device=dev, with_dy=cfg.backward)
    else:
        cpu = make_inputs(cfg, args.seed, with_dy=cfg.backward)
        inp = {k: (None if v is None else v.to(dev)) for k, v in cpu.items()}
    torch.cuda.synchronize()
    aux = args.aux_alpha
    capacity = None
    if args.capacity_factor is not None:
        capacity = int(math.ceil(args.capacity_factor * cfg.N * cfg.K / cfg.E))
    Fs = args.shared_ffn
    shared = None
    if Fs is not None:
        shared_cpu = make_shared_weights(cfg, args.seed, Fs)
        shared = tuple(w.to(dev) for w in shared_cpu)
    r = MoELayerRunner(cfg.N, cfg.H, cfg.F, cfg.E, cfg.K, cfg.torch_dtype, dev, backward=cfg.backward,
                       aux_alpha=aux, capacity=capacity, shared_ffn=Fs, dw_gather=args.dw_gather)
    d = r.d
    x, w_r, wg, wu, wd, bias, dy = (inp[k] for k in ("x", "w_r", "w_gate", "w_up", "w_down", "bias", "dy"))
    stream = torch.cuda.current_stream()
    # the backward runs the router backward beside dA on a second stream
    # (default priority), as MoELayerRunner does; the GEMMs keep the GPU
    side = torch.cuda.Stream() if (cfg.backward or shared is not None) else None
    permute_bwd = L.moe_permute_bwd if aux is None else L.moe_permute_bwd_dense
    fns = {
        "route_meta": lambda st: L.moe_route_meta(d, x, w_r, bias, 2 ** 31 - 1 if capacity is None else capacity,
                                                  r.topk, r.gates, r.sorted_flat, r.inv, r.counts, r.offsets,
                                                  r.tiles, r.num_tiles, r.route_meta_ws, st),
        "permute": lambda st: L.moe_permute(d, x, r.sorted_flat, r.xs, st),
        "gate_up": ((lambda st: L.moe_ffn_gate_up_gather(d, x, r.sorted_flat, wg, wu, r.tiles, r.num_tiles, r.g, r.u,
                                                         r.act, st)) if r.gather_fused else
                    (lambda st: L.moe_ffn_gate_up(d, r.xs, wg, wu, r.tiles, r.num_tiles, r.g, r.u, r.act, st))),
        "down": lambda st: L.moe_ffn_down(d, r.act, wd, r.tiles, r.num_tiles, r.ys, st),
        "combine": ((lambda st: L.moe_combine(d, r.ys, r.gates, r.inv, r.y, st)) if shared is None else
                    (lambda st: L.moe_combine_shared(d, r.ys, r.gates, r.inv, r.ys_s, r.y, st))),
        "shared_ffn": lambda st: L.moe_shared_ffn(r.ds, x, shared[0], shared[1], shared[2], r.g_s, r.u_s, r.act_s,
                                                  r.ys_s, r.shared_ws, st),
        "shared_bwd": lambda st: L.moe_shared_ffn_bwd(r.ds, x, dy, shared[0], shared[1], shared[2], r.g_s, r.u_s,
                                                      r.act_s, r.dg_s, r.du_s, r.dx_s, r.dw_gate_s, r.dw_up_s,
                                                      r.dw_down_s, r.shared_ws, st),
        "aux_loss": lambda st: L.moe_aux_loss(d, x, w_r, bias, r.counts, aux, r.probs, r.aux_loss, r.aux_ws, st),
        "combine_bwd": lambda st: L.moe_combine_bwd(d, dy, r.ys, r.gates, r.inv, r.dys, r.dgates, st),
        "route_bwd": ((lambda st: L.moe_route_bwd(d, x, r.topk, r.gates, r.dgates, r.dlogits, r.dw_r, r.route_ws,
                                                  st)) if aux is None else
                      (lambda st: L.moe_route_bwd_aux(d, x, r.topk, r.gates, r.dgates, r.probs, r.counts, aux,
                                                      r.dlogits, r.dw_r, r.route_ws, st))),
        "dact": lambda st: L.moe_ffn_bwd_dact(d, r.dys, wd, r.g, r.u, r.tiles, r.num_tiles, r.dg, r.du, st),
        "dx_dw": ((lambda st: L.moe_ffn_bwd_dx_dw_gather(d, r.dg, r.du, wg, wu, r.tiles, r.num_tiles, r.dxs, x,
                                                         r.sorted_flat, r.act, r.dys, r.offsets, r.dw_gate, r.dw_up,
                                                         r.dw_down, st)) if r.dw_gather else
                  (lambda st: L.moe_ffn_bwd_dx_dw(d, r.dg, r.du, wg, wu, r.tiles, r.num_tiles, r.dxs, r.xs, r.act,
                                                  r.dys, r.offsets, r.dw_gate, r.dw_up, r.dw_down, st))),
        "permute_bwd": ((lambda st: permute_bwd(d, r.dxs, r.inv, r.topk, r.dlogits, w_r, r.dx, r.perm_ws, st))
                        if shared is None else
                        (lambda st: L.moe_permute_bwd_add(d, r.dxs, r.inv, r.topk, r.dlogits, w_r, aux is not None,
                                                          r.dx_s, r.dx, r.perm_ws, st))),
    }
    fwd_names = ((["shared_ffn"] if shared is not None else []) + ["route_meta"] +
                 (["permute", "gate_up"] if not r.gather_fused else
                  ["gate_up"] + (["permute"] if r.xs is not None else [])) + ["down", "combine"] +
                 (["aux_loss"] if aux is not None else []))
    bwd_names = ((["combine_bwd", "route_bwd"] + (["shared_bwd"] if shared is not None else []) +
                  ["dact", "dx_dw", "permute_bwd"]) if cfg.backward else [])

    def step(ev=None, only=None, overlap=False):
        def run(name, st):
            if ev is not None and (only is None or name == only):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(st)
                fns[name](st)
                b.record(st)
                ev.setdefault(name, []).append((a, b))
            else:
                fns[name](st)

        def hand_over(frm, to):
            e = torch.cuda.Event()
            e.record(frm)
            to.wait_event(e)

        if not overlap:
            for name in fwd_names + bwd_names:
                run(name, stream)
            return
        # the shared expert's forward runs beside the routed forward and
        # joins before the combine
        for name in fwd_names:
            if name == "shared_ffn":
                hand_over(stream, side)
                run(name, side)
                shared_done = torch.cuda.Event()
                shared_done.record(side)
                continue
            if name == "combine" and shared is not None:
                stream.wait_event(shared_done)
            run(name, stream)
        if not cfg.backward:
            return
        run("combine_bwd", stream)
        hand_over(stream, side)
        run("route_bwd", side)
        if shared is not None:
            run("shared_bwd", side)
        route_done = torch.cuda.Event()
        route_done.record(side)
        run("dact", stream)
        run("dx_dw", stream)
        stream.wait_event(route_done)
        run("permute_bwd", stream)
        hand_over(side, stream)

    # warm-up (untimed)
    for _ in range(args.warmup):
        step(overlap=True)
    torch.cuda.synchronize()
    # untimed per-stage breakdown
    ev = {}
    for _ in range(max(3, min(10, args.steps))):
        step(ev)
    torch.cuda.synchronize()
    stage_ms = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in ev.items()}
    kept_rows = int(r.offsets[cfg.E].item())
    fl = stage_flops(cfg, kept_rows, Fs)
    gemm_ms = sum(stage_ms[k] for k in fl if k in stage_ms)
    gemm_flops = sum(v for k, v in fl.items() if k in stage_ms)
    # the roofline entry is for one kernel: stages of several launches are
    # reported in the breakdown only
    dominant = max((k for k in stage_ms if k not in COMPOSITE), key=stage_ms.get)

    # timed region: exactly K steps; events only around the dominant kernel
    ev_dom = {}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(ev_dom, only=dominant, overlap=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    dom_ms = float(np.mean([a.elapsed_time(b) for a, b in ev_dom[dominant]]))
    tokens_per_s = cfg.N * args.steps / (t1 - t0)

    peak_flops = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    used = int((np.diff(r.offsets.cpu().numpy()) > 0).sum())
    gb = gemm_bytes(cfg, kept_rows, used, r.g is not None)
    if dominant in fl and fl[dominant] / (peak_flops * 1e12) < gb[dominant] / (PEAK_HBM_GBS * 1e9):
        # a grouped GEMM whose bytes at HBM peak take longer than its flops at
        # the matrix-core peak (the wide-expert forward streams every expert's
        # weights for about 256 rows each): HBM-bound
        achieved = gb[dominant] / (dom_ms * 1e-3) / 1e9
        roof = {"kernel": dominant, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "algorithmic_bytes_per_launch": gb[dominant], "algorithmic_flops_per_launch": fl[dominant],
                "launch_ms": round(dom_ms, 5)}
    elif dominant in fl:
        achieved = fl[dominant] / (dom_ms * 1e-3) / 1e12
        roof = {"kernel": dominant, "bound": "mfma" if cfg.dtype == "bf16" else "alu", "achieved": round(achieved, 2),
                "peak": peak_flops,
                "unit": "TFLOP/s", "frac": round(achieved / peak_flops, 4),
                "algorithmic_flops_per_launch": fl[dominant], "algorithmic_bytes_per_launch": gb.get(dominant),
                "launch_ms": round(dom_ms, 5)}
    else:
        byt = stage_bytes(cfg, aux is not None, shared is not None)[dominant]
        achieved = byt / (dom_ms * 1e-3) / 1e9
        roof = {"kernel": dominant, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "algorithmic_bytes_per_launch": byt, "launch_ms": round(dom_ms, 5)}
    roof["traffic"] = measured_traffic(cfg.name, dominant) if (aux is None and shared is None) else None

    counts = r.counts.cpu().numpy().astype(np.float64)
    tbar = cfg.NK / cfg.E
    maxvio = float(counts.max() / tbar - 1.0)

    # every grouped-GEMM stage against its own bound (from the event-timed breakdown)
    gemm_roof = {}
    for k in gb:
        if k in stage_ms and stage_ms[k] > 0:
            t = stage_ms[k] * 1e-3
            if fl[k] / (peak_flops * 1e12) < gb[k] / (PEAK_HBM_GBS * 1e9):
                gemm_roof[k] = {"bound": "hbm", "frac": round(gb[k] / t / 1e9 / PEAK_HBM_GBS, 4)}
            else:
                gemm_roof[k] = {"bound": "mfma" if cfg.dtype == "bf16" else "alu",
                                "frac": round(fl[k] / t / 1e12 / peak_flops, 4)}

    hbm = {}
    for k, b in stage_bytes(cfg, aux is not None, shared is not None).items():
        if k in stage_ms and stage_ms[k] > 0:
            hbm[k] = round(b / (stage_ms[k] * 1e-3) / 1e9, 1)

    cpu_base = None
    if not args.no_cpu_baseline and not big:
        cpu_base = cpu_baseline(cfg, cpu, aux, shared_cpu if shared is not None else None)

    out = {
        "metric": "MoE layer tokens/sec fwd+bwd; grouped-GEMM % of bf16 MFMA peak",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.description, "N": cfg.N, "H": cfg.H, "F": cfg.F, "E": cfg.E, "K": cfg.K,
                   "backward": cfg.backward, "parallelism": "single GPU", "maxvio": round(maxvio, 4),
                   "load_balancing_loss_alpha": aux,
                   "gather_fused_into_gate_up": r.gather_fused,
                   "gather_fused_into_dw": r.dw_gather,
                   "capacity": capacity,
                   "dropped_rows": cfg.NK - kept_rows,
                   "shared_expert_ffn": Fs,
                   "streams": ("router backward beside dA" if cfg.backward else "one") +
                              ("; shared expert beside the routed path" if shared is not None else ""),
                   "empty_experts": int((counts == 0).sum())},
        "grouped_gemm": {"tflops": round(gemm_flops / (gemm_ms * 1e-3) / 1e12, 2),
                         "frac_of_bf16_peak": round(gemm_flops / (gemm_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "ms": round(gemm_ms, 4), "algorithmic_flops": gemm_flops},
        "stages_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "stages_hbm_gbs": hbm,
        "gemm_stages_roofline": gemm_roof,
        "roofline": roof,
        "cpu_baseline": cpu_base,
        "host": {"cpu": host_cpu_model(), "cores": os.cpu_count(), "blas_threads": blas_threads()},
    }
    print(json.dumps(out), flush=True)


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def blas_threads():
    """Threads of the BLAS that NumPy's matmuls (the oracle's) run on."""
    try:
        from threadpoolctl import threadpool_info
        n = [d.get("num_threads") for d in threadpool_info() if d.get("user_api") == "blas"]
        if n and n[0]:
            return int(n[0])
    except Exception:  # noqa: BLE001 - reporting only
        pass
    return os.cpu_count()


# float64 multiply-adds per second the host is assumed to sustain in the
# oracle's matmuls; only sizes the sample so that it takes 10-30 s
CPU_SAMPLE_FLOPS = 40e9
CPU_SAMPLE_SECONDS = 12.0


def cpu_baseline(cfg, cpu, aux=None, shared=None):
    """The oracle (as it stands) on the host, on a bounded sample of the
    workload: whole-layer passes over its first S tokens, with S sized by the
    layer's flops per token for about CPU_SAMPLE_SECONDS of work, repeated
    until that much time has passed (at most 20 passes)."""
    from oracle import moe_oracle as O
    per_token = (18 if cpu["dy"] is not None else 6) * cfg.H * cfg.F * cfg.K
    S = int(min(cfg.N, max(16, CPU_SAMPLE_FLOPS * CPU_SAMPLE_SECONDS / per_token)))
    x = cpu["x"][:S]
    dy = cpu["dy"][:S] if cpu["dy"] is not None else None
    store = "bf16" if cfg.dtype == "bf16" else "f32"
    t0 = time.perf_counter()
    passes = 0
    while True:
        f = O.forward(x, cpu["w_r"], cpu["w_gate"], cpu["w_up"], cpu["w_down"], cfg.K, bias=cpu["bias"], store=store,
                      shared=shared)
        if aux is not None:
            O.aux_loss(f["logits"], f["counts"], cfg.K, aux)
        if dy is not None:
            O.backward(f, dy, aux_scale=aux)
        del f
        passes += 1
        if time.perf_counter() - t0 > CPU_SAMPLE_SECONDS or passes >= 20:
            break
    dt = time.perf_counter() - t0
    return {"value": round(S * passes / dt, 1), "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            "cpu": host_cpu_model(),
            "sample": f"first {S} of {cfg.N} tokens of the workload (all {cfg.E} experts' weights), {passes} "
                      f"whole-layer pass(es) ({'fwd+bwd' if dy is not None else 'fwd'}), float64 NumPy on "
                      f"{blas_threads()} BLAS threads, {dt:.1f} s"}


if __name__ == "__main__":
    main()
