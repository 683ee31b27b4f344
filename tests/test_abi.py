"""The C-ABI library loads, exports every entry point declared in
include/moe.h, and rejects bad arguments on the host before any launch
(CPU only: no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

from mixture_experts_layer_sort_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from mixture_experts_layer_sort_amd.build import build
        build()
    return L.lib()


def test_header_declares_the_binding(lib):
    names = header_functions()
    assert len(names) >= 17
    assert sorted(L.SIGNATURES) == names


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_abi_version_matches_header(lib):
    v = int(re.search(r"#define MOE_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert L.moe_abi_version() == v


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4, 7):
        assert isinstance(L.moe_status_str(st), str) and L.moe_status_str(st)


def D(N=64, H=128, F=256, E=4, K=2, dtype=L.MOE_BF16, gemm_tiles=L.MOE_TILES_AUTO):
    return L.dims(N, H, F, E, K, dtype, gemm_tiles)


FAKE = 0x10000  # never dereferenced: every call below fails validation or has N = 0


def route(d, x=FAKE, w=FAKE, b=None, t=FAKE, g=FAKE):
    return L.lib().moe_route(ctypes.byref(d), x, w, b, t, g, None)


@pytest.mark.parametrize("d,status", [
    (D(H=100), L.MOE_EINVAL), (D(F=200), L.MOE_EINVAL), (D(N=-1), L.MOE_EINVAL), (D(E=0), L.MOE_EINVAL),
    (D(K=0), L.MOE_EINVAL), (D(K=5, E=4), L.MOE_EUNSUPPORTED), (D(E=300, K=2), L.MOE_EUNSUPPORTED),
    (D(E=16, K=9), L.MOE_EUNSUPPORTED), (D(dtype=7), L.MOE_EUNSUPPORTED), (D(gemm_tiles=4), L.MOE_EINVAL),
    (D(gemm_tiles=-1), L.MOE_EINVAL),
    (D(N=2 ** 30, K=2), L.MOE_EUNSUPPORTED),
])
def test_bad_dims_rejected(lib, d, status):
    assert route(d) == status
    assert L.moe_max_tiles(d) == -1
    assert L.moe_workspace_bytes(d, L.MOE_ENTRY_ROUTE_BWD) == 2 ** 64 - 1


def test_null_and_misaligned_pointers_rejected(lib):
    assert route(D(), x=None) == L.MOE_EINVAL
    assert route(D(), t=FAKE + 4) == L.MOE_EINVAL
    assert route(D(), b=FAKE + 8) == L.MOE_EINVAL
    assert L.lib().moe_route(None, FAKE, FAKE, None, FAKE, FAKE, None) == L.MOE_EINVAL
    d = D()
    # g_save / u_save must be both set or both NULL
    assert L.lib().moe_ffn_gate_up(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == L.MOE_EINVAL


def test_workspace_checked(lib):
    d = D()
    need = L.moe_workspace_bytes(d, L.MOE_ENTRY_ROUTE_BWD)
    assert need > 0
    st = L.lib().moe_route_bwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None)
    assert st == L.MOE_EWORKSPACE
    st = L.lib().moe_route_bwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, need, None)
    assert st == L.MOE_EWORKSPACE
    need = L.moe_workspace_bytes(d, L.MOE_ENTRY_PERMUTE_BWD)
    st = L.lib().moe_permute_bwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 16, None)
    assert st == L.MOE_EWORKSPACE
    assert L.moe_workspace_bytes(d, 99) == 2 ** 64 - 1


def test_zero_tokens_returns_ok_without_launch(lib):
    d = D(N=0)
    assert route(d) == L.MOE_OK
    assert L.lib().moe_permute_meta(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 0
    assert L.lib().moe_combine(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None) == 0


@pytest.mark.parametrize("N,K,E", [(16384, 2, 8), (16384, 6, 64), (8192, 8, 256), (1, 1, 1), (3, 2, 256)])
def test_max_tiles_bounds_any_routing(lib, N, K, E):
    d = D(N=N, K=K, E=E)
    mt = L.moe_max_tiles(d)
    assert mt == (N * K + E * (L.MOE_TILE_M - 1)) // L.MOE_TILE_M
    # worst case over routings: sum_e ceil(c_e / T) with sum_e c_e = NK
    import math
    NK = N * K
    worst_spread = sum(math.ceil(c / L.MOE_TILE_M) for c in [NK // E + (1 if i < NK % E else 0) for i in range(E)])
    assert worst_spread <= mt


def test_aux_loss_entries_validate_on_the_host(lib):
    d = D(E=8)
    lb = L.lib()
    need = L.moe_workspace_bytes(d, L.MOE_ENTRY_AUX_LOSS)
    assert need > 0 and need != 2 ** 64 - 1
    # bad alpha, null pointers, short workspace
    assert lb.moe_aux_loss(ctypes.byref(d), FAKE, FAKE, None, FAKE, float("nan"), FAKE, FAKE, FAKE, need,
                           None) == L.MOE_EINVAL
    assert lb.moe_aux_loss(ctypes.byref(d), FAKE, FAKE, None, None, 0.01, FAKE, FAKE, FAKE, need, None) == L.MOE_EINVAL
    assert lb.moe_aux_loss(ctypes.byref(d), FAKE, FAKE, None, FAKE, 0.01, FAKE, FAKE, FAKE, need - 4,
                           None) == L.MOE_EWORKSPACE
    need_b = L.moe_workspace_bytes(d, L.MOE_ENTRY_ROUTE_BWD_AUX)
    assert need_b >= L.moe_workspace_bytes(d, L.MOE_ENTRY_ROUTE_BWD) + d.N * 4
    args = [FAKE] * 6
    assert lb.moe_route_bwd_aux(ctypes.byref(d), *args, float("inf"), FAKE, FAKE, FAKE, need_b, None) == L.MOE_EINVAL
    assert lb.moe_route_bwd_aux(ctypes.byref(d), *args, 0.01, FAKE, FAKE, FAKE, need_b - 1,
                                None) == L.MOE_EWORKSPACE
    need_p = L.moe_workspace_bytes(d, L.MOE_ENTRY_PERMUTE_BWD)
    assert lb.moe_permute_bwd_dense(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need_p - 16,
                                    None) == L.MOE_EWORKSPACE
    d0 = D(N=0)
    assert lb.moe_aux_loss(ctypes.byref(d0), FAKE, FAKE, None, FAKE, 0.01, FAKE, FAKE, None, 0, None) == L.MOE_OK


def test_capacity_and_gather_entries_validate_on_the_host(lib):
    d = D(E=8)
    lb = L.lib()
    need = L.moe_workspace_bytes(d, L.MOE_ENTRY_PERMUTE_META)
    args = [FAKE] * 7
    assert lb.moe_permute_meta_capacity(ctypes.byref(d), FAKE, -1, *args, need, None) == L.MOE_EINVAL
    assert lb.moe_permute_meta_capacity(ctypes.byref(d), FAKE, 5, *args, need - 4, None) == L.MOE_EWORKSPACE
    assert lb.moe_permute_meta_capacity(ctypes.byref(d), None, 5, *args, need, None) == L.MOE_EINVAL
    d0 = D(N=0)
    assert lb.moe_permute_meta_capacity(ctypes.byref(d0), FAKE, 0, *([FAKE] * 6), None, 0, None) == L.MOE_OK
    # gathered gate/up: null source rows, one of g/u missing, 32-bit row offsets
    gu = [FAKE] * 4
    assert lb.moe_ffn_gate_up_gather(ctypes.byref(d), FAKE, None, *gu, FAKE, FAKE, FAKE, None) == L.MOE_EINVAL
    assert lb.moe_ffn_gate_up_gather(ctypes.byref(d), FAKE, FAKE, *gu, FAKE, None, FAKE, None) == L.MOE_EINVAL
    big = D(N=2 ** 21, H=1024)
    assert lb.moe_ffn_gate_up_gather(ctypes.byref(big), FAKE, FAKE, *gu, FAKE, FAKE, FAKE,
                                     None) == L.MOE_EUNSUPPORTED
    # gathered weight gradients: null or misaligned x, null sorted_flat; N = 0 launches nothing
    lf = lb.moe_ffn_bwd_dx_dw_gather
    pre = [FAKE] * 7                      # dg, du, w_gate, w_up, tiles, num_tiles, dxs
    post = [FAKE] * 6                     # act, dys, offsets, dw_gate, dw_up, dw_down
    assert lf(ctypes.byref(d), *pre, None, FAKE, *post, None) == L.MOE_EINVAL
    assert lf(ctypes.byref(d), *pre, FAKE, None, *post, None) == L.MOE_EINVAL
    assert lf(ctypes.byref(d), *pre, FAKE + 2, FAKE, *post, None) == L.MOE_EINVAL
    assert lf(ctypes.byref(d0), *pre, FAKE, FAKE, *post, None) == L.MOE_OK


def test_shared_expert_entries_validate_on_the_host(lib):
    lb = L.lib()
    d = D(E=8)
    ds = D(N=64, H=128, F=384, E=1, K=1)
    for e in (L.MOE_ENTRY_SHARED_FFN, L.MOE_ENTRY_SHARED_FFN_BWD):
        assert L.moe_workspace_bytes(d, e) == 2 ** 64 - 1          # only the one-expert dims
    nf = L.moe_workspace_bytes(ds, L.MOE_ENTRY_SHARED_FFN)
    nb = L.moe_workspace_bytes(ds, L.MOE_ENTRY_SHARED_FFN_BWD)
    assert 0 < nf <= nb
    f8 = [FAKE] * 8
    assert lb.moe_shared_ffn(ctypes.byref(d), *f8, FAKE, nf, None) == L.MOE_EINVAL           # E, K != 1
    assert lb.moe_shared_ffn(ctypes.byref(ds), *f8, FAKE, nf - 4, None) == L.MOE_EWORKSPACE
    assert lb.moe_shared_ffn(ctypes.byref(ds), *([FAKE] * 4), None, FAKE, FAKE, FAKE, FAKE, nf,
                             None) == L.MOE_EINVAL                                              # g without u
    assert lb.moe_shared_ffn(ctypes.byref(ds), *([FAKE] * 4), None, None, FAKE, FAKE, FAKE, nf - 4,
                             None) == L.MOE_EWORKSPACE                                          # forward only
    f14 = [FAKE] * 14
    assert lb.moe_shared_ffn_bwd(ctypes.byref(ds), *f14, FAKE, nb - 4, None) == L.MOE_EWORKSPACE
    assert lb.moe_shared_ffn_bwd(ctypes.byref(d), *f14, FAKE, nb, None) == L.MOE_EINVAL
    assert lb.moe_shared_ffn_bwd(ctypes.byref(ds), None, *f14[1:], FAKE, nb, None) == L.MOE_EINVAL
    need_p = L.moe_workspace_bytes(d, L.MOE_ENTRY_PERMUTE_BWD)
    f5 = [FAKE] * 5
    assert lb.moe_permute_bwd_add(ctypes.byref(d), *f5, 2, FAKE, FAKE, FAKE, need_p, None) == L.MOE_EINVAL
    assert lb.moe_permute_bwd_add(ctypes.byref(d), *f5, 0, None, FAKE, FAKE, need_p, None) == L.MOE_EINVAL
    assert lb.moe_permute_bwd_add(ctypes.byref(d), *f5, 1, FAKE, FAKE, FAKE, need_p - 16, None) == L.MOE_EWORKSPACE
    assert lb.moe_combine_shared(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, None) == L.MOE_EINVAL
    d0, ds0 = D(N=0), D(N=0, E=1, K=1)
    assert lb.moe_combine_shared(ctypes.byref(d0), *([FAKE] * 5), None) == L.MOE_OK
    assert lb.moe_shared_ffn(ctypes.byref(ds0), *f8, None, 0, None) == L.MOE_OK


@pytest.mark.parametrize("N,H,Fs,S", [(16384, 512, 1024, 10), (700, 256, 512, 2), (64, 128, 384, 1),
                                      (16384, 4096, 14336, 1), (1500, 256, 768, 3)])
def test_shared_weight_gradient_split(lib, N, H, Fs, S):
    """The shared expert's weight-gradient contraction is cut into S row
    chunks: as many as fill 256 CUs once with 3*ceil(H/256)*ceil(Fs/256)
    output tiles per chunk, each of at least 512 rows (rounded to 64-row
    steps).  The backward workspace holds S+1 chunk bounds and, for S > 1,
    the 3*S*H*Fs float32 partial sums."""
    ds = D(N=N, H=H, F=Fs, E=1, K=1)
    nf = L.moe_workspace_bytes(ds, L.MOE_ENTRY_SHARED_FFN)
    nb = L.moe_workspace_bytes(ds, L.MOE_ENTRY_SHARED_FFN_BWD)
    part = 3 * S * H * Fs * 4 if S > 1 else 0
    assert nb - nf == (S + 1) * 4 + (-(S + 1) * 4) % 16 + part


def test_route_meta_entry_validates_on_the_host(lib):
    lb = L.lib()
    d = D(N=64, E=8)
    need = L.moe_workspace_bytes(d, L.MOE_ENTRY_ROUTE_META)
    assert need == 2 * 8 * 4                      # two 32-token blocks x 8 experts
    f9 = [FAKE] * 8
    assert lb.moe_route_meta(ctypes.byref(d), FAKE, FAKE, None, -1, *f9, FAKE, need, None) == L.MOE_EINVAL
    assert lb.moe_route_meta(ctypes.byref(d), FAKE, FAKE, None, 5, *f9, FAKE, need - 4, None) == L.MOE_EWORKSPACE
    assert lb.moe_route_meta(ctypes.byref(d), FAKE, None, None, 5, *f9, FAKE, need, None) == L.MOE_EINVAL
    assert lb.moe_route_meta(ctypes.byref(d), FAKE, FAKE, FAKE + 4, 5, *f9, FAKE, need, None) == L.MOE_EINVAL
    d0 = D(N=0)
    assert lb.moe_route_meta(ctypes.byref(d0), FAKE, FAKE, None, 0, *f9, None, 0, None) == L.MOE_OK


@pytest.mark.parametrize("N,E,K,fused", [(16384, 8, 2, True), (16384, 64, 6, True), (8192, 256, 8, False),
                                         (16384, 128, 2, False), (32, 1, 1, True)])
def test_route_meta_workspace_follows_the_fusion_rule(lib, N, E, K, fused):
    """Fused while ceil(N/32) * E <= 32768 (the block histograms); else the
    unfused metadata's workspace."""
    d = D(N=N, E=E, K=K)
    got = L.moe_workspace_bytes(d, L.MOE_ENTRY_ROUTE_META)
    blocks = -(-N // 32)
    assert (blocks * E <= 32768) == fused
    if fused:
        assert got == blocks * E * 4
    else:
        assert got == L.moe_workspace_bytes(d, L.MOE_ENTRY_PERMUTE_META)


def test_noalloc_rejects_a_problem_beyond_its_scratch(lib):
    """moe_route_meta_noalloc refuses, on the host and before any launch, a
    problem whose metadata scratch exceeds the library-held array."""
    d = L.dims(600000, 128, 128, 256, 8, L.MOE_BF16)
    assert L.moe_workspace_bytes(d, L.MOE_ENTRY_ROUTE_META) > L.MOE_NOALLOC_SCRATCH_BYTES
    st = lib.moe_route_meta_noalloc(ctypes.byref(d), FAKE, FAKE, None, 2 ** 31 - 1, *([FAKE] * 8), None)
    assert st == L.MOE_ESCRATCH
    assert "scratch" in L.moe_status_str(st)
