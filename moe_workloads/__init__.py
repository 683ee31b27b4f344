"""Seeded synthetic workloads for the dropless top-k MoE layer.

This module only draws random inputs: it holds none of the layer's
arithmetic, so both the CPU oracle and the HIP path can take their inputs
from it without sharing any computation.

Recipe (identical for every configuration):
  * one CPU ``torch.Generator`` per (tensor, expert), seeded from the base
    seed, the tensor's name and the expert id, so a single expert's weights
    can be regenerated on their own;
  * x ~ N(0, 1); W_r ~ 0.02 * N(0, 1) (the tiny example of the page
    "MoE computation principle and execution process", section 2.4, draws
    the router weight as randn * 0.02);
  * W_gate, W_up ~ N(0, 1) / sqrt(H); W_down ~ N(0, 1) / sqrt(F)
    (std = 1/sqrt(fan_in));
  * dY ~ N(0, 1) (upstream gradient of the layer output);
  * bf16 configurations round every drawn tensor to bfloat16 with
    round-to-nearest-even (``Tensor.to(torch.bfloat16)``); the fp32
    configuration keeps fp32;
  * the skewed configuration adds a fixed per-expert logit bias
    b_e = tau * ln(w_e), w_e = (e+1)^-s / sum_j (j+1)^-s (Zipf rank weights,
    s = 1.2, tau = 1.25) so that one expert receives close to the maximum
    possible share and some experts receive no token.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

__all__ = ["MoEConfig", "CONFIGS", "TEST_CONFIGS", "make_inputs", "make_expert_weights", "make_shared_weights",
           "zipf_bias", "tensor_seed"]


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    N: int          # tokens
    H: int          # hidden size
    F: int          # expert FFN (intermediate) size
    E: int          # experts
    K: int          # experts per token
    dtype: str      # "f32" or "bf16"
    backward: bool = True
    zipf_s: Optional[float] = None   # Zipf exponent of the logit bias (None: no bias)
    zipf_tau: float = 1.0            # scale of the log rank weight
    description: str = ""

    @property
    def NK(self) -> int:
        return self.N * self.K

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def gemm_flops_fwd(self) -> int:
        return 6 * self.H * self.F * self.NK

    def gemm_flops_bwd(self) -> int:
        return 12 * self.H * self.F * self.NK


def _cfgs(*cfgs: MoEConfig) -> Dict[str, MoEConfig]:
    return {c.name: c for c in cfgs}


# The workloads: named by dtype, routing and sizes.
CONFIGS = _cfgs(
    MoEConfig("f32_n32_h128_f256_e4_k2", N=32, H=128, F=256, E=4, K=2, dtype="f32",
              description="tiny fp32 MoE, N=32 H=128 F=256 E=4 K=2"),
    MoEConfig("bf16_n16384_h512_f1024_e8_k2", N=16384, H=512, F=1024, E=8, K=2, dtype="bf16",
              description="bf16 dropless MoE fwd+bwd, N=16384 (seq 1024 x batch 16) H=512 F=1024 E=8 K=2"),
    MoEConfig("bf16_skewed_n16384_h2048_f1408_e64_k6", N=16384, H=2048, F=1408, E=64, K=6, dtype="bf16",
              zipf_s=1.2, zipf_tau=1.25,
              description="skewed-routing bf16 fwd+bwd, N=16384 H=2048 F=1408 E=64 K=6, Zipf(1.2) logit bias"),
    MoEConfig("bf16_fwd_n8192_h7168_f2048_e256_k8", N=8192, H=7168, F=2048, E=256, K=8, dtype="bf16",
              backward=False,
              description="wide-expert bf16 forward, N=8192 H=7168 F=2048 E=256 K=8 (22.5 GB weights)"),
    MoEConfig("bf16_n16384_h4096_f14336_e8_k2", N=16384, H=4096, F=14336, E=8, K=2, dtype="bf16",
              description="large-FFN bf16 deterministic fwd+bwd, N=16384 H=4096 F=14336 E=8 K=2"),
)

TINY = CONFIGS["f32_n32_h128_f256_e4_k2"]
BASE = CONFIGS["bf16_n16384_h512_f1024_e8_k2"]
SKEWED = CONFIGS["bf16_skewed_n16384_h2048_f1408_e64_k6"]
WIDE = CONFIGS["bf16_fwd_n8192_h7168_f2048_e256_k8"]
LARGE = CONFIGS["bf16_n16384_h4096_f14336_e8_k2"]

# Small shapes for parity tests: several tiles per expert, ragged tails,
# empty experts, K=1, K=E, E=1 and the fp32 path.
TEST_CONFIGS = {
    "t_ragged": MoEConfig("t_ragged", N=700, H=256, F=384, E=6, K=3, dtype="bf16"),
    "t_skew": MoEConfig("t_skew", N=600, H=128, F=256, E=16, K=2, dtype="bf16", zipf_s=1.2, zipf_tau=3.0),
    "t_k1": MoEConfig("t_k1", N=333, H=256, F=128, E=5, K=1, dtype="bf16"),
    "t_keqe": MoEConfig("t_keqe", N=257, H=128, F=256, E=4, K=4, dtype="bf16"),
    "t_e1": MoEConfig("t_e1", N=300, H=128, F=384, E=1, K=1, dtype="bf16"),
    "t_wide_e": MoEConfig("t_wide_e", N=512, H=256, F=128, E=256, K=8, dtype="bf16"),
    "t_f32": MoEConfig("t_f32", N=203, H=256, F=384, E=7, K=3, dtype="f32"),
    "t_bigtile": MoEConfig("t_bigtile", N=2048, H=512, F=768, E=4, K=2, dtype="bf16"),
}

_TENSOR_IDS = {"x": 1, "w_r": 2, "w_gate": 3, "w_up": 4, "w_down": 5, "dy": 6, "w_gate_s": 7, "w_up_s": 8,
               "w_down_s": 9}


def tensor_seed(base_seed: int, name: str, expert: int = 0) -> int:
    """Seed of one (tensor, expert) stream; distinct for every pair."""
    return (base_seed * 1_000_003 + _TENSOR_IDS[name] * 65_537 + expert) & 0x7FFF_FFFF_FFFF


def _randn(shape, seed: int, device="cpu") -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32, device=device)


def zipf_bias(E: int, s: float, tau: float) -> torch.Tensor:
    """Per-expert logit bias tau * ln(w_e) with Zipf(s) rank weights (rank = e+1)."""
    w = torch.tensor([(e + 1) ** (-s) for e in range(E)], dtype=torch.float64)
    w = w / w.sum()
    return (tau * torch.log(w)).to(torch.float32)


def make_expert_weights(cfg: MoEConfig, seed: int, expert: int, device="cpu"):
    """(W_gate[e] [H,F], W_up[e] [H,F], W_down[e] [F,H]) of one expert, in cfg's dtype."""
    dt = cfg.torch_dtype
    wg = (_randn((cfg.H, cfg.F), tensor_seed(seed, "w_gate", expert), device) / math.sqrt(cfg.H)).to(dt)
    wu = (_randn((cfg.H, cfg.F), tensor_seed(seed, "w_up", expert), device) / math.sqrt(cfg.H)).to(dt)
    wd = (_randn((cfg.F, cfg.H), tensor_seed(seed, "w_down", expert), device) / math.sqrt(cfg.F)).to(dt)
    return wg, wu, wd


def make_inputs(cfg: MoEConfig, seed: int = 0, device="cpu", with_dy: Optional[bool] = None):
    """All layer inputs of a configuration as contiguous tensors on ``device``.

    Returns a dict with x [N,H], w_r [H,E], bias [E] fp32 or None,
    w_gate [E,H,F], w_up [E,H,F], w_down [E,F,H] and dy [N,H] (if the
    configuration has a backward pass or ``with_dy`` is set).
    The same seed gives the same values on the same device type.
    """
    dt = cfg.torch_dtype
    out = {}
    out["x"] = _randn((cfg.N, cfg.H), tensor_seed(seed, "x"), device).to(dt)
    out["w_r"] = (_randn((cfg.H, cfg.E), tensor_seed(seed, "w_r"), device) * 0.02).to(dt)
    out["bias"] = (zipf_bias(cfg.E, cfg.zipf_s, cfg.zipf_tau).to(device)
                   if cfg.zipf_s is not None else None)
    wg = torch.empty((cfg.E, cfg.H, cfg.F), dtype=dt, device=device)
    wu = torch.empty((cfg.E, cfg.H, cfg.F), dtype=dt, device=device)
    wd = torch.empty((cfg.E, cfg.F, cfg.H), dtype=dt, device=device)
    for e in range(cfg.E):
        g, u, d = make_expert_weights(cfg, seed, e, device)
        wg[e].copy_(g)
        wu[e].copy_(u)
        wd[e].copy_(d)
        del g, u, d
    out["w_gate"], out["w_up"], out["w_down"] = wg, wu, wd
    if with_dy if with_dy is not None else cfg.backward:
        out["dy"] = _randn((cfg.N, cfg.H), tensor_seed(seed, "dy"), device).to(dt)
    else:
        out["dy"] = None
    return out


def make_shared_weights(cfg: MoEConfig, seed: int, F_s: int, device="cpu"):
    """(W_gate_s [H,Fs], W_up_s [H,Fs], W_down_s [Fs,H]) of a shared expert of
    intermediate size F_s, drawn like a routed expert's (std 1/sqrt(fan_in)),
    in cfg's dtype."""
    dt = cfg.torch_dtype
    wg = (_randn((cfg.H, F_s), tensor_seed(seed, "w_gate_s"), device) / math.sqrt(cfg.H)).to(dt)
    wu = (_randn((cfg.H, F_s), tensor_seed(seed, "w_up_s"), device) / math.sqrt(cfg.H)).to(dt)
    wd = (_randn((F_s, cfg.H), tensor_seed(seed, "w_down_s"), device) / math.sqrt(F_s)).to(dt)
    return wg, wu, wd


def get_config(name: str) -> MoEConfig:
    if name in CONFIGS:
        return CONFIGS[name]
    if name in TEST_CONFIGS:
        return TEST_CONFIGS[name]
    raise KeyError(f"unknown MoE configuration {name!r}")
