"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the algorithmic
flop and byte counts the roofline figures divide by, and the guard that turns
the stored traffic readings off once the kernel sources change."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from moe_workloads import get_config  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_gemm_flops_per_step_large_ffn():
    # forward 6 H F and backward 12 H F flops per routed row: 18 x 4096 x 14336 x 32768
    cfg = get_config("bf16_n16384_h4096_f14336_e8_k2")
    fl = bench.stage_flops(cfg)
    assert sum(fl.values()) == 18 * 4096 * 14336 * 32768 == 34634616274944
    assert fl["dx_dw"] == 10 * 4096 * 14336 * 32768  # dX 4 H F + dW 6 H F


def test_gemm_bytes_count_each_operand_once():
    cfg = get_config("bf16_n16384_h512_f1024_e8_k2")
    rows, E = cfg.NK, cfg.E
    b = bench.gemm_bytes(cfg, rows, E, True)
    H, F = cfg.H, cfg.F
    # xs read, both weight halves read, G, U and A written, all bf16
    assert b["gate_up"] == 2 * (rows * H + 2 * E * H * F + 3 * rows * F)
    # A read, W_down read, ys written
    assert b["down"] == 2 * (rows * F + E * H * F + rows * H)
    # forward only (no G and U saved): A alone is written
    assert bench.gemm_bytes(cfg, rows, E, False)["gate_up"] == 2 * (rows * H + 2 * E * H * F + rows * F)


def test_row_kernel_bytes():
    cfg = get_config("bf16_n16384_h4096_f14336_e8_k2")
    s = bench.stage_bytes(cfg)
    N, NK, H = cfg.N, cfg.NK, cfg.H
    assert s["combine"] == 2 * (NK + N) * H + 8 * NK
    assert s["combine_bwd"] == 2 * (N + 2 * NK) * H + 12 * NK


def test_traffic_is_dropped_once_the_sources_change(monkeypatch):
    key = next(iter(bench.TRAFFIC["bytes"]))
    monkeypatch.setattr(bench, "kernel_sources_hash", lambda: bench.TRAFFIC["sources"])
    assert bench.measured_traffic(*key) == bench.TRAFFIC["bytes"][key]
    monkeypatch.setattr(bench, "kernel_sources_hash", lambda: "0" * 16)
    assert bench.measured_traffic(*key) is None


@pytest.mark.parametrize("name", ["bf16_n16384_h4096_f14336_e8_k2", "bf16_n16384_h512_f1024_e8_k2",
                                  "bf16_skewed_n16384_h2048_f1408_e64_k6", "bf16_fwd_n8192_h7168_f2048_e256_k8"])
def test_traffic_readings_cover_every_gemm_stage(name):
    cfg = get_config(name)
    stages = ["gate_up", "down"] + (["dact", "dx_dw"] if cfg.backward else [])
    for st in stages:
        v = bench.TRAFFIC["bytes"].get((name, st))
        assert v is not None and v > 0, (name, st)
