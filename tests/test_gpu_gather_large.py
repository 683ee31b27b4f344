"""Gathered gate/up rows past 2 GiB of x, through the C ABI.

gate/up reads its token rows straight from x through sorted_flat, with
32-bit byte offsets into x (x below 4 GiB whenever the gather is used).  Here
x holds N = 2^18 + 1024 tokens of H = 4096 (2.16 GB of bf16), and one
256-row tile gathers the last 256 tokens, all at byte offsets past 2^31.  The
same rows copied to the front of x and gathered from there must give the
same bytes (the same products in the same order), and both must agree with a
float32 product on the host.  Tile lists and row indices are written by hand
(one expert, one tile), so no other stage runs.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

N, H, F = (1 << 18) + 1024, 4096, 256
ROWS = 256


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_sort_amd import _lib
    _lib.lib()


def _gate_up(L, d, x, sorted_flat, wg, wu, tiles, num_tiles):
    NK = d.N * d.K
    g = torch.zeros((NK, F), dtype=torch.bfloat16, device="cuda")
    u = torch.zeros_like(g)
    a = torch.zeros_like(g)
    L.moe_ffn_gate_up_gather(d, x, sorted_flat, wg, wu, tiles, num_tiles, g, u, a)
    torch.cuda.synchronize()
    return g[:ROWS].clone(), u[:ROWS].clone(), a[:ROWS].clone()


def test_gathered_rows_past_2gib_match_front_copy():
    from mixture_experts_layer_sort_amd import _lib as L
    print(f"[gather past 2 GiB] N={N} H={H} F={F}", flush=True)
    assert (1 << 30) < N * H < (1 << 31)
    gen = torch.Generator(device="cpu").manual_seed(5)
    d = L.dims(N, H, F, 1, 1, L.MOE_BF16)
    assert L.moe_max_tiles(d) >= 1
    x = torch.zeros((N, H), dtype=torch.bfloat16, device="cuda")
    tail = torch.randn((ROWS, H), generator=gen).to(torch.bfloat16)
    toks = np.arange(N - ROWS, N)[::-1].copy()          # the last ROWS tokens, in reverse order
    x[torch.from_numpy(toks).cuda()] = tail.cuda()
    assert int(toks.min()) * H * 2 >= (1 << 31)          # every gathered row starts past 2 GiB
    wg = (torch.randn((1, H, F), generator=gen) / 64).to(torch.bfloat16).cuda()
    wu = (torch.randn((1, H, F), generator=gen) / 64).to(torch.bfloat16).cuda()
    tiles = torch.tensor([0, 0, ROWS], dtype=torch.int32, device="cuda")
    num_tiles = torch.tensor([1], dtype=torch.int32, device="cuda")
    sf = torch.zeros((N,), dtype=torch.int32)
    sf[:ROWS] = torch.from_numpy(toks.astype(np.int32))  # K = 1: flat index = token
    far = _gate_up(L, d, x, sf.cuda(), wg, wu, tiles, num_tiles)

    # the same rows at the front of x
    x[:ROWS] = tail.cuda()
    sf_front = torch.zeros((N,), dtype=torch.int32)
    sf_front[:ROWS] = torch.arange(ROWS, dtype=torch.int32)
    near = _gate_up(L, d, x, sf_front.cuda(), wg, wu, tiles, num_tiles)
    for name, t_far, t_near in zip("GUA", far, near):
        assert torch.equal(t_far.view(torch.int16), t_near.view(torch.int16)), name

    # and both against a float32 product on the host
    xs = tail.float()
    g_ref = xs @ wg[0].float().cpu()
    u_ref = xs @ wu[0].float().cpu()
    for name, got, ref in (("G", far[0], g_ref), ("U", far[1], u_ref)):
        err = (got.float().cpu() - ref).abs()
        bound = ref.abs() * 2.0 ** -8 + 1e-3                  # bf16 storage rounding + fp32 order
        assert bool((err <= bound).all()), (name, float(err.max()))
