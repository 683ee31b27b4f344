"""ctypes binding of the C ABI in include/moe.h (argument marshalling only).

Each function here has the name of the C entry point it calls and takes
torch tensors (device memory) instead of raw pointers; every step of the
layer runs in the HIP library.  There is no fallback: if the library is not
built or cannot be loaded, ``lib()`` raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP, MOE_ESCRATCH = 0, -1, -2, -3, -4, -5
MOE_NOALLOC_SCRATCH_BYTES = 4 << 20
MOE_F32, MOE_BF16 = 0, 1
MOE_ENTRY_PERMUTE_META, MOE_ENTRY_ROUTE_BWD, MOE_ENTRY_PERMUTE_BWD = 1, 2, 3
MOE_ENTRY_AUX_LOSS, MOE_ENTRY_ROUTE_BWD_AUX = 4, 5
MOE_ENTRY_SHARED_FFN, MOE_ENTRY_SHARED_FFN_BWD, MOE_ENTRY_ROUTE_META = 6, 7, 8
MOE_TILE_M = 256
# moe_gemm_tiles (moe_dims.gemm_tiles): AUTO, or one bf16 tile family forced on every GEMM stage
MOE_TILES_AUTO, MOE_TILES_256, MOE_TILES_128X256, MOE_TILES_128 = 0, 1, 2, 3

# Every exported symbol with (restype, argtypes); the tests check this list
# against include/moe.h and against the built library.
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_F = ctypes.c_float


class moe_dims(ctypes.Structure):
    _fields_ = [("N", _I64), ("H", _I64), ("F", _I64), ("E", _I64), ("K", _I64), ("dtype", _I32), ("gemm_tiles", _I32)]


_DP = ctypes.POINTER(moe_dims)

SIGNATURES = {
    "moe_abi_version": (ctypes.c_int, []),
    "moe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_max_tiles": (_I64, [_DP]),
    "moe_workspace_bytes": (_SZ, [_DP, _I32]),
    "moe_route": (ctypes.c_int, [_DP, _P, _P, _P, _P, _P, _P]),
    "moe_permute_meta": (ctypes.c_int, [_DP, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_permute_meta_capacity": (ctypes.c_int, [_DP, _P, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_permute": (ctypes.c_int, [_DP, _P, _P, _P, _P]),
    "moe_expert_ffn": (ctypes.c_int, [_DP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_ffn_gate_up": (ctypes.c_int, [_DP, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_ffn_gate_up_gather": (ctypes.c_int, [_DP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_ffn_down": (ctypes.c_int, [_DP, _P, _P, _P, _P, _P, _P]),
    "moe_combine": (ctypes.c_int, [_DP, _P, _P, _P, _P, _P]),
    "moe_combine_bwd": (ctypes.c_int, [_DP, _P, _P, _P, _P, _P, _P, _P]),
    "moe_route_bwd": (ctypes.c_int, [_DP, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_expert_ffn_bwd": (ctypes.c_int, [_DP] + [_P] * 17 + [_P]),
    "moe_ffn_bwd_dact": (ctypes.c_int, [_DP, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_ffn_bwd_dx": (ctypes.c_int, [_DP, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_ffn_bwd_dw": (ctypes.c_int, [_DP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_permute_bwd": (ctypes.c_int, [_DP, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_permute_bwd_dense": (ctypes.c_int, [_DP, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_aux_loss": (ctypes.c_int, [_DP, _P, _P, _P, _P, _F, _P, _P, _P, _SZ, _P]),
    "moe_route_bwd_aux": (ctypes.c_int, [_DP, _P, _P, _P, _P, _P, _P, _F, _P, _P, _P, _SZ, _P]),
    "moe_shared_ffn": (ctypes.c_int, [_DP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_combine_shared": (ctypes.c_int, [_DP, _P, _P, _P, _P, _P, _P]),
    "moe_shared_ffn_bwd": (ctypes.c_int, [_DP] + [_P] * 15 + [_SZ, _P]),
    "moe_permute_bwd_add": (ctypes.c_int, [_DP, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _SZ, _P]),
    "moe_ffn_bwd_dx_dw": (ctypes.c_int, [_DP] + [_P] * 14 + [_P]),
    "moe_route_meta": (ctypes.c_int, [_DP, _P, _P, _P, _I32] + [_P] * 9 + [_SZ, _P]),
    "moe_route_meta_noalloc": (ctypes.c_int, [_DP, _P, _P, _P, _I32] + [_P] * 8 + [_P]),
    "moe_ffn_bwd_dx_dw_gather": (ctypes.c_int, [_DP] + [_P] * 15 + [_P]),
}

_LIB: Optional[ctypes.CDLL] = None


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().moe_status_str(status).decode() if _LIB is not None else str(status)
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def lib(path: Optional[str] = None) -> ctypes.CDLL:
    """Load (once) and return the HIP library; raises if it is not built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with mixture_experts_layer_sort_amd.build "
                           "(there is no CPU fallback)")
    h = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(h, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = h
    return h


def dims(N: int, H: int, F: int, E: int, K: int, dtype: int, gemm_tiles: int = MOE_TILES_AUTO) -> moe_dims:
    return moe_dims(N, H, F, E, K, dtype, gemm_tiles)


def dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return MOE_BF16
    if t == torch.float32:
        return MOE_F32
    raise ValueError(f"unsupported dtype {t}")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor arguments must be device (cuda) tensors")
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call(name: str, *args):
    st = getattr(lib(), name)(*args)
    if st != MOE_OK:
        raise MoEError(name, st)


def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def moe_max_tiles(d: moe_dims) -> int:
    return lib().moe_max_tiles(ctypes.byref(d))


def moe_workspace_bytes(d: moe_dims, entry: int) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(d), entry)


def moe_route(d, x, w_r, logit_bias, topk_idx, gates, stream=None):
    _call("moe_route", ctypes.byref(d), _ptr(x), _ptr(w_r), _ptr(logit_bias), _ptr(topk_idx), _ptr(gates),
          _stream(stream))


def moe_permute_meta(d, topk_idx, sorted_flat, inv, counts, offsets, tiles, num_tiles, ws, stream=None):
    _call("moe_permute_meta", ctypes.byref(d), _ptr(topk_idx), _ptr(sorted_flat), _ptr(inv), _ptr(counts),
          _ptr(offsets), _ptr(tiles), _ptr(num_tiles), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
          _stream(stream))


def moe_permute_meta_capacity(d, topk_idx, capacity, sorted_flat, inv, counts, offsets, tiles, num_tiles, ws,
                              stream=None):
    _call("moe_permute_meta_capacity", ctypes.byref(d), _ptr(topk_idx), int(capacity), _ptr(sorted_flat), _ptr(inv),
          _ptr(counts), _ptr(offsets), _ptr(tiles), _ptr(num_tiles), _ptr(ws),
          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))


def moe_permute(d, x, sorted_flat, xs, stream=None):
    _call("moe_permute", ctypes.byref(d), _ptr(x), _ptr(sorted_flat), _ptr(xs), _stream(stream))


def moe_expert_ffn(d, xs, w_gate, w_up, w_down, tiles, num_tiles, g_save, u_save, act, ys, stream=None):
    _call("moe_expert_ffn", ctypes.byref(d), _ptr(xs), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(tiles),
          _ptr(num_tiles), _ptr(g_save), _ptr(u_save), _ptr(act), _ptr(ys), _stream(stream))


def moe_ffn_gate_up(d, xs, w_gate, w_up, tiles, num_tiles, g_save, u_save, act, stream=None):
    _call("moe_ffn_gate_up", ctypes.byref(d), _ptr(xs), _ptr(w_gate), _ptr(w_up), _ptr(tiles), _ptr(num_tiles),
          _ptr(g_save), _ptr(u_save), _ptr(act), _stream(stream))

def moe_ffn_gate_up_gather(d, x, sorted_flat, w_gate, w_up, tiles, num_tiles, g_save, u_save, act, stream=None):
    _call("moe_ffn_gate_up_gather", ctypes.byref(d), _ptr(x), _ptr(sorted_flat), _ptr(w_gate), _ptr(w_up),
          _ptr(tiles), _ptr(num_tiles), _ptr(g_save), _ptr(u_save), _ptr(act), _stream(stream))


def moe_ffn_down(d, act, w_down, tiles, num_tiles, ys, stream=None):
    _call("moe_ffn_down", ctypes.byref(d), _ptr(act), _ptr(w_down), _ptr(tiles), _ptr(num_tiles), _ptr(ys),
          _stream(stream))


def moe_combine(d, ys, gates, inv, y, stream=None):
    _call("moe_combine", ctypes.byref(d), _ptr(ys), _ptr(gates), _ptr(inv), _ptr(y), _stream(stream))


def moe_combine_bwd(d, dy, ys, gates, inv, dys, dgates, stream=None):
    _call("moe_combine_bwd", ctypes.byref(d), _ptr(dy), _ptr(ys), _ptr(gates), _ptr(inv), _ptr(dys), _ptr(dgates),
          _stream(stream))


def moe_route_bwd(d, x, topk_idx, gates, dgates, dlogits, dw_r, ws, stream=None):
    _call("moe_route_bwd", ctypes.byref(d), _ptr(x), _ptr(topk_idx), _ptr(gates), _ptr(dgates), _ptr(dlogits),
          _ptr(dw_r), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))


def moe_expert_ffn_bwd(d, dys, xs, w_gate, w_up, w_down, g_save, u_save, act, offsets, tiles, num_tiles, dg, du,
                       dxs, dw_gate, dw_up, dw_down, stream=None):
    _call("moe_expert_ffn_bwd", ctypes.byref(d), _ptr(dys), _ptr(xs), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
          _ptr(g_save), _ptr(u_save), _ptr(act), _ptr(offsets), _ptr(tiles), _ptr(num_tiles), _ptr(dg), _ptr(du),
          _ptr(dxs), _ptr(dw_gate), _ptr(dw_up), _ptr(dw_down), _stream(stream))


def moe_ffn_bwd_dact(d, dys, w_down, g_save, u_save, tiles, num_tiles, dg, du, stream=None):
    _call("moe_ffn_bwd_dact", ctypes.byref(d), _ptr(dys), _ptr(w_down), _ptr(g_save), _ptr(u_save), _ptr(tiles),
          _ptr(num_tiles), _ptr(dg), _ptr(du), _stream(stream))


def moe_ffn_bwd_dx(d, dg, du, w_gate, w_up, tiles, num_tiles, dxs, stream=None):
    _call("moe_ffn_bwd_dx", ctypes.byref(d), _ptr(dg), _ptr(du), _ptr(w_gate), _ptr(w_up), _ptr(tiles),
          _ptr(num_tiles), _ptr(dxs), _stream(stream))


def moe_ffn_bwd_dw(d, xs, act, dys, dg, du, offsets, dw_gate, dw_up, dw_down, stream=None):
    _call("moe_ffn_bwd_dw", ctypes.byref(d), _ptr(xs), _ptr(act), _ptr(dys), _ptr(dg), _ptr(du), _ptr(offsets),
          _ptr(dw_gate), _ptr(dw_up), _ptr(dw_down), _stream(stream))


def moe_permute_bwd(d, dxs, inv, topk_idx, dlogits, w_r, dx, ws, stream=None):
    _call("moe_permute_bwd", ctypes.byref(d), _ptr(dxs), _ptr(inv), _ptr(topk_idx), _ptr(dlogits), _ptr(w_r),
          _ptr(dx), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))


def moe_permute_bwd_dense(d, dxs, inv, topk_idx, dlogits, w_r, dx, ws, stream=None):
    _call("moe_permute_bwd_dense", ctypes.byref(d), _ptr(dxs), _ptr(inv), _ptr(topk_idx), _ptr(dlogits), _ptr(w_r),
          _ptr(dx), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))


def moe_aux_loss(d, x, w_r, logit_bias, counts, alpha, probs, loss, ws, stream=None):
    _call("moe_aux_loss", ctypes.byref(d), _ptr(x), _ptr(w_r), _ptr(logit_bias), _ptr(counts), float(alpha),
          _ptr(probs), _ptr(loss), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))


def moe_route_bwd_aux(d, x, topk_idx, gates, dgates, probs, counts, aux_scale, dlogits, dw_r, ws, stream=None):
    _call("moe_route_bwd_aux", ctypes.byref(d), _ptr(x), _ptr(topk_idx), _ptr(gates), _ptr(dgates), _ptr(probs),
          _ptr(counts), float(aux_scale), _ptr(dlogits), _ptr(dw_r), _ptr(ws),
          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))


def _nbytes(ws) -> int:
    return 0 if ws is None else ws.numel() * ws.element_size()


def moe_shared_ffn(ds, x, w_gate, w_up, w_down, g_save, u_save, act, ys_shared, ws, stream=None):
    _call("moe_shared_ffn", ctypes.byref(ds), _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(g_save),
          _ptr(u_save), _ptr(act), _ptr(ys_shared), _ptr(ws), _nbytes(ws), _stream(stream))


def moe_combine_shared(d, ys, gates, inv, ys_shared, y, stream=None):
    _call("moe_combine_shared", ctypes.byref(d), _ptr(ys), _ptr(gates), _ptr(inv), _ptr(ys_shared), _ptr(y),
          _stream(stream))


def moe_shared_ffn_bwd(ds, x, dy, w_gate, w_up, w_down, g_save, u_save, act, dg, du, dx_shared, dw_gate, dw_up,
                       dw_down, ws, stream=None):
    _call("moe_shared_ffn_bwd", ctypes.byref(ds), _ptr(x), _ptr(dy), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
          _ptr(g_save), _ptr(u_save), _ptr(act), _ptr(dg), _ptr(du), _ptr(dx_shared), _ptr(dw_gate), _ptr(dw_up),
          _ptr(dw_down), _ptr(ws), _nbytes(ws), _stream(stream))


def moe_permute_bwd_add(d, dxs, inv, topk_idx, dlogits, w_r, dense, dx_add, dx, ws, stream=None):
    _call("moe_permute_bwd_add", ctypes.byref(d), _ptr(dxs), _ptr(inv), _ptr(topk_idx), _ptr(dlogits), _ptr(w_r),
          int(dense), _ptr(dx_add), _ptr(dx), _ptr(ws), _nbytes(ws), _stream(stream))


def moe_ffn_bwd_dx_dw(d, dg, du, w_gate, w_up, tiles, num_tiles, dxs, xs, act, dys, offsets, dw_gate, dw_up, dw_down,
                      stream=None):
    _call("moe_ffn_bwd_dx_dw", ctypes.byref(d), _ptr(dg), _ptr(du), _ptr(w_gate), _ptr(w_up), _ptr(tiles),
          _ptr(num_tiles), _ptr(dxs), _ptr(xs), _ptr(act), _ptr(dys), _ptr(offsets), _ptr(dw_gate), _ptr(dw_up),
          _ptr(dw_down), _stream(stream))


def moe_route_meta(d, x, w_r, logit_bias, capacity, topk_idx, gates, sorted_flat, inv, counts, offsets, tiles,
                   num_tiles, ws, stream=None):
    _call("moe_route_meta", ctypes.byref(d), _ptr(x), _ptr(w_r), _ptr(logit_bias), int(capacity), _ptr(topk_idx),
          _ptr(gates), _ptr(sorted_flat), _ptr(inv), _ptr(counts), _ptr(offsets), _ptr(tiles), _ptr(num_tiles),
          _ptr(ws), _nbytes(ws), _stream(stream))


def moe_route_meta_noalloc(d, x, w_r, logit_bias, capacity, topk_idx, gates, sorted_flat, inv, counts, offsets,
                           tiles, num_tiles, stream=None):
    _call("moe_route_meta_noalloc", ctypes.byref(d), _ptr(x), _ptr(w_r), _ptr(logit_bias), int(capacity),
          _ptr(topk_idx), _ptr(gates), _ptr(sorted_flat), _ptr(inv), _ptr(counts), _ptr(offsets), _ptr(tiles),
          _ptr(num_tiles), _stream(stream))


def moe_ffn_bwd_dx_dw_gather(d, dg, du, w_gate, w_up, tiles, num_tiles, dxs, x, sorted_flat, act, dys, offsets,
                             dw_gate, dw_up, dw_down, stream=None):
    _call("moe_ffn_bwd_dx_dw_gather", ctypes.byref(d), _ptr(dg), _ptr(du), _ptr(w_gate), _ptr(w_up), _ptr(tiles),
          _ptr(num_tiles), _ptr(dxs), _ptr(x), _ptr(sorted_flat), _ptr(act), _ptr(dys), _ptr(offsets),
          _ptr(dw_gate), _ptr(dw_up), _ptr(dw_down), _stream(stream))
