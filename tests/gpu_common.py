"""Shared helpers of the GPU parity tests (oracle on the CPU, HIP path on the GPU)."""
from __future__ import annotations

import numpy as np
import torch

from moe_workloads import MoEConfig, make_inputs
from oracle import moe_oracle as O
from tests import parity as P

# spec tolerances
TOL_F32_ABS = P.TOL_F32_ABS
TOL_BF16_ABS = P.TOL_BF16_ABS
TOL_BF16_RELRMS = P.TOL_BF16_RELRMS
# logit gap below which float32 and float64 may rank two experts differently
NEAR_TIE = 1e-4


def to_np(t) -> np.ndarray:
    return O.as_f64(t)


rel_rms = P.rel_rms


def assert_close(name: str, got, ref: np.ndarray, dtype: str, band=None, abs_tol=None, rel_tol=None):
    """Level 1 of tests/parity.py: one tensor against the oracle's.  fp32:
    max|err| <= 1e-4 (or abs_tol).  bf16: rel-RMS <= 1e-2 and, for
    bf16-stored tensors, |err| <= 2e-2 + band per element (band from
    oracle.rounding_bands, capped at two bf16 spacings); float32 outputs are
    held element by element by the per-step checks (check_runner_steps)."""
    g = to_np(got)
    if dtype == "f32":
        err = float(np.max(np.abs(g - ref))) if g.size else 0.0
        tol = TOL_F32_ABS if abs_tol is None else abs_tol
        print(f"[oracle] {name}: max|err| {err:.3e}", flush=True)
        assert err <= tol, f"{name}: max|err| {err:.3e} > {tol:.1e}"
        return err
    return P.compare_with_oracle(name, g, np.asarray(ref, dtype=np.float64), "bf16", band=band)["max_err"]


def runner_run(r, y=None, grads=None) -> P.Run:
    """The stored tensors of a MoELayerRunner after forward (and backward)."""
    t = dict(topk=r.topk, gates=r.gates, sorted_flat=r.sorted_flat, inv=r.inv, counts=r.counts, offsets=r.offsets,
             tiles=r.tiles, num_tiles=r.num_tiles, xs=r.xs, G=r.g, U=r.u, A=r.act, ys=r.ys,
             y=r.y if y is None else y)
    if grads is not None:
        t.update(dys=r.dys, dG=r.dg, dU=r.du, dxs=r.dxs, dgates=grads["dgates"], dlogits=grads["dlogits"],
                 dx=grads["dx"], dw_r=grads["dw_r"], dw_gate=grads["dw_gate"], dw_up=grads["dw_up"],
                 dw_down=grads["dw_down"])
    return P.Run(**t)


def check_runner_steps(cfg: MoEConfig, cpu: dict, r, y=None, grads=None, capacity=None, aux=None, shared=None,
                       **kw):
    """Level 2 of tests/parity.py on a runner's stored tensors: every step
    from its own stored inputs (every row, every column unless kw narrows)."""
    run = runner_run(r, y, grads)
    if shared is not None:
        for k, attr in (("G_s", "g_s"), ("U_s", "u_s"), ("A_s", "act_s"), ("ys_s", "ys_s")):
            run.t[k] = getattr(r, attr)
        if grads is not None:
            for k, attr in (("dG_s", "dg_s"), ("dU_s", "du_s"), ("dxs_s", "dx_s"), ("dw_gate_s", "dw_gate_s"),
                            ("dw_up_s", "dw_up_s"), ("dw_down_s", "dw_down_s")):
                run.t[k] = getattr(r, attr)
    x = O.as_f64(cpu["x"])
    P.check_steps(x, O.as_f64(cpu["w_r"]), P.weights_of(cpu["w_gate"], cpu["w_up"], cpu["w_down"]), cfg.K, run,
                  store_of(cfg), dy=None if grads is None else O.as_f64(cpu["dy"]), capacity=capacity,
                  shared_w=shared, aux=aux, **kw)
    return run


def store_of(cfg: MoEConfig) -> str:
    return "f32" if cfg.dtype == "f32" else "bf16"


def gpu_inputs(cfg: MoEConfig, seed: int = 0, with_dy=None):
    cpu = make_inputs(cfg, seed, with_dy=with_dy)
    dev = {k: (None if v is None else v.to("cuda")) for k, v in cpu.items()}
    return cpu, dev


def oracle_fwd(cfg: MoEConfig, cpu: dict):
    return O.forward(cpu["x"], cpu["w_r"], cpu["w_gate"], cpu["w_up"], cpu["w_down"], cfg.K, bias=cpu["bias"],
                     store=store_of(cfg))


def assignment_mismatch(topk_gpu: np.ndarray, ofwd: dict, K: int):
    """Tokens whose GPU top-K differs from the oracle's; asserts each one is a
    near-tie (several assignments are correct there)."""
    tg = topk_gpu.astype(np.int64)
    to = ofwd["topk"].astype(np.int64)
    bad = np.where(np.any(tg != to, axis=1))[0]
    l = ofwd["logits"]
    for n in bad:
        lv = l[n]
        # every expert the GPU picked must be within NEAR_TIE of the oracle's
        # value at the same rank
        assert len(set(tg[n].tolist())) == K, f"token {n}: repeated expert"
        ref_sorted = np.sort(lv)[::-1]
        for k in range(K):
            assert abs(lv[tg[n, k]] - ref_sorted[k]) <= NEAR_TIE, (n, k, lv[tg[n, k]], ref_sorted[k])
    return bad


def sync():
    torch.cuda.synchronize()
