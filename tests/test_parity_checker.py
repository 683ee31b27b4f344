"""Pins of the parity checks themselves (CPU only).

The two-level checks of tests/parity.py must accept a second correct
implementation of the layer (tests/standin.py: torch float32, its own
summation order, bf16 storage at the same points) and must reject it as soon
as one plausible device mistake is planted in one of its outputs: a token
missing from dW_r, an expert row missing from dW_down, a combine that drops
one k slot, a transposed 256 x 256 weight-gradient tile, and more.  The
shapes are the default workload's (H = 512, F = 1024, E = 8, K = 2), at its
full N = 16384 tokens for the router-gradient case and N = 2048 otherwise.

They also show why the float32 outputs are not held to 2e-2 per element
against the oracle: the stand-in, a correct evaluation, differs from the
oracle by more than that in dgates, dW_r and the weight gradients.
"""
import functools

import numpy as np
import pytest

from moe_workloads import MoEConfig, make_inputs
from oracle import moe_oracle as O
from tests import parity as P
from tests.standin import float32_layer

SHAPE = dict(H=512, F=1024, E=8, K=2, dtype="bf16")


@functools.lru_cache(maxsize=2)
def _case(N):
    cfg = MoEConfig(f"c1_shape_n{N}", N=N, **SHAPE)
    inp = {k: (None if v is None else O.as_f64(v)) for k, v in make_inputs(cfg, 0, with_dy=True).items()}
    fwd = O.forward(inp["x"], inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.K, store="bf16")
    bwd = O.backward(fwd, inp["dy"])
    alt = float32_layer(inp, fwd, cfg.K)
    return cfg, inp, fwd, bwd, alt


def _quiet(msg):
    pass


def _check_all(cfg, inp, fwd, bwd, run_t, names=None, steps=True, level1=True):
    """Both levels on the stand-in's (possibly mutated) tensors."""
    ref = dict(fwd)
    ref.update(bwd)
    if level1:
        band = O.rounding_bands(fwd, bwd, inp["dy"])
        for name in (names or (P.BF16_STORED + P.F32_OUTPUTS)):
            if name in run_t and name in ref:
                P.compare_with_oracle(name, run_t[name], np.asarray(ref[name]), "bf16", band=band.get(name),
                                      log=_quiet)
    if steps:
        run = P.Run(**run_t)
        P.check_steps(inp["x"], inp["w_r"], P.weights_of(inp["w_gate"], inp["w_up"], inp["w_down"]), cfg.K, run,
                      "bf16", dy=inp["dy"], log=_quiet)


def test_standin_passes_both_levels():
    cfg, inp, fwd, bwd, alt = _case(2048)
    _check_all(cfg, inp, fwd, bwd, dict(alt))


def test_float32_outputs_of_a_correct_run_exceed_2e2_against_the_oracle():
    """dgates, dW_r and dW_down of the stand-in are a correct evaluation,
    yet differ from the oracle by more than 2e-2 in some elements: the
    per-element absolute bound cannot hold for them, which is why Level 2
    holds them instead.  Their rel-RMS stays far below 1e-2."""
    cfg, inp, fwd, bwd, alt = _case(16384)
    over = {}
    for name in ("dgates", "dw_r", "dw_down"):
        err = np.abs(alt[name] - bwd[name])
        over[name] = float(err.max())
        assert P.rel_rms(alt[name], bwd[name]) < 1e-3
    assert max(over.values()) > 2e-2, over


# every planted mistake: (name, function of (cfg, inp, fwd, bwd, tensors) -> None, mutating the tensors)
def _drop_token_from_dw_r(cfg, inp, fwd, bwd, t):
    n = 123
    t["dw_r"] = t["dw_r"] - np.outer(inp["x"][n], t["dlogits"][n])


def _drop_row_from_dw_down(cfg, inp, fwd, bwd, t):
    e = 3
    r = int(fwd["offsets"][e]) + 17
    t["dw_down"] = t["dw_down"].copy()
    t["dw_down"][e] -= np.outer(t["A"][r], t["dys"][r])


def _combine_drops_a_slot(cfg, inp, fwd, bwd, t):
    n, k = 77, 1
    r = int(fwd["inv"][n * cfg.K + k])
    t["y"] = t["y"].copy()
    pre = sum(fwd["gates"][n, j] * t["ys"][int(fwd["inv"][n * cfg.K + j])] for j in range(cfg.K) if j != k)
    t["y"][n] = O.round_bf16(pre)
    assert r >= 0


def _transposed_dw_tile(cfg, inp, fwd, bwd, t):
    e = 2
    t["dw_gate"] = t["dw_gate"].copy()
    blk = t["dw_gate"][e][256:512, 512:768].copy()
    t["dw_gate"][e][256:512, 512:768] = blk.T


def _dgates_wrong_slot(cfg, inp, fwd, bwd, t):
    t["dgates"] = t["dgates"].copy()
    t["dgates"][5] = t["dgates"][5][::-1]


def _dx_without_router_term(cfg, inp, fwd, bwd, t):
    n = 999
    inv = fwd["inv"].reshape(cfg.N, cfg.K)
    t["dx"] = t["dx"].copy()
    t["dx"][n] = O.round_bf16(sum(t["dxs"][inv[n, k]] for k in range(cfg.K)))


def _g_row_shift_in_a_tile(cfg, inp, fwd, bwd, t):
    r0 = int(fwd["offsets"][1]) + 256 + 40
    t["G"] = t["G"].copy()
    t["G"][r0] = t["G"][r0 + 1]


def _silu_on_the_up_branch(cfg, inp, fwd, bwd, t):
    r = slice(int(fwd["offsets"][4]), int(fwd["offsets"][4]) + 64)
    t["A"] = t["A"].copy()
    t["A"][r] = O.round_bf16(O.silu(t["U"][r]) * t["G"][r])


def _dlogits_sign(cfg, inp, fwd, bwd, t):
    t["dlogits"] = t["dlogits"].copy()
    t["dlogits"][321] = -t["dlogits"][321]


def _dxs_row_zeroed(cfg, inp, fwd, bwd, t):
    t["dxs"] = t["dxs"].copy()
    t["dxs"][1500] = 0.0


def _dys_ungated(cfg, inp, fwd, bwd, t):
    r = 2000
    f = int(fwd["sorted_flat"][r])
    t["dys"] = t["dys"].copy()
    t["dys"][r] = O.round_bf16(inp["dy"][f // cfg.K])


def _empty_tail_tile_dw_up(cfg, inp, fwd, bwd, t):
    # the last rows of an expert left out of its weight gradient (a ragged tail tile skipped)
    e = 5
    r0, r1 = int(fwd["offsets"][e]), int(fwd["offsets"][e + 1])
    tail = slice(r1 - (r1 - r0) % 256 or r1 - 256, r1)
    src = inp["x"][fwd["sorted_flat"][tail] // cfg.K]
    t["dw_up"] = t["dw_up"].copy()
    t["dw_up"][e] -= src.T @ t["dU"][tail]


MUTATIONS = {
    "dw_r_missing_one_token": _drop_token_from_dw_r,
    "dw_down_missing_one_row": _drop_row_from_dw_down,
    "combine_drops_one_k_slot": _combine_drops_a_slot,
    "transposed_256x256_dw_tile": _transposed_dw_tile,
    "dgates_slots_swapped": _dgates_wrong_slot,
    "dx_without_router_term": _dx_without_router_term,
    "g_row_shifted_inside_a_tile": _g_row_shift_in_a_tile,
    "silu_on_the_up_branch": _silu_on_the_up_branch,
    "dlogits_sign_flipped": _dlogits_sign,
    "dxs_row_zeroed": _dxs_row_zeroed,
    "dys_without_gate": _dys_ungated,
    "dw_up_ragged_tail_skipped": _empty_tail_tile_dw_up,
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_rejected(name):
    N = 16384 if name == "dw_r_missing_one_token" else 2048
    cfg, inp, fwd, bwd, alt = _case(N)
    t = dict(alt)
    MUTATIONS[name](cfg, inp, fwd, bwd, t)
    with pytest.raises(AssertionError):
        if name == "dw_r_missing_one_token":
            # the router backward step alone (the whole-layer check at this N
            # is slow on the CPU); it is the step that holds dW_r
            P.check_route_bwd(inp["x"], cfg.K, P.Run(**t), "bf16", log=_quiet)
        else:
            _check_all(cfg, inp, fwd, bwd, t)


def test_dw_r_with_all_tokens_passes_the_router_step_at_full_n():
    """The unmutated stand-in passes the router-gradient step at N = 16384 (the
    control of the planted missing token above)."""
    cfg, inp, fwd, bwd, alt = _case(16384)
    P.check_route_bwd(inp["x"], cfg.K, P.Run(**alt), "bf16", log=_quiet)


def test_level1_alone_misses_a_missing_token_in_dw_r():
    """Documentation of the split: against the oracle alone, a dW_r missing
    one token of 16384 stays within rel-RMS 1e-2, so the per-step check is
    what catches it (test_planted_mistake_is_rejected)."""
    cfg, inp, fwd, bwd, alt = _case(16384)
    t = dict(alt)
    _drop_token_from_dw_r(cfg, inp, fwd, bwd, t)
    P.compare_with_oracle("dw_r", t["dw_r"], bwd["dw_r"], "bf16", log=_quiet)
