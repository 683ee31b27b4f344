// Shared expert: one dense SwiGLU expert that every token passes through with
// weight 1, its output added to the routed combine ("MegaBlocks -
// architecture and principles", section 2.1: the layer output plus an
// optional shared-expert MLP over all tokens).
//
// It runs on the grouped-GEMM kernels of the routed experts as a one-expert
// problem (E = K = 1, rows = x in token order, F = its own intermediate
// size), with a tile list built here.  Its weight gradients contract over all
// N tokens but have only ceil(H/256) * ceil(F/256) * 3 output tiles, far too
// few workgroups for 256 CUs; the contraction is therefore split into S row
// chunks (run as S "experts" of the weight-gradient kernel, float32 partials)
// and the partials are summed in chunk order, so the result stays bitwise
// reproducible.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"

namespace {

// tiles: (expert 0, first row, rows) per MOE_TILE_M rows; offs: S + 1 chunk
// bounds (0, chunk, 2 chunk, ..., N).
__global__ __launch_bounds__(256) void k_dense_plan(int32_t* __restrict__ tiles, int32_t* __restrict__ num_tiles,
                                                    int32_t* __restrict__ offs, int N, int nt, int S, int chunk) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < nt) {
    tiles[3 * i] = 0;
    tiles[3 * i + 1] = i * MOE_TILE_M;
    tiles[3 * i + 2] = min(MOE_TILE_M, N - i * MOE_TILE_M);
  }
  if (i == 0) *num_tiles = nt;
  if (offs != nullptr && i <= S) offs[i] = min(N, i * chunk);
}

// out[i] = sum_{s < S} part[s * n + i], s ascending, for the three weight
// gradients (blockIdx.y); n is a multiple of 4.
__global__ __launch_bounds__(256) void k_sum_partials(const float* __restrict__ p0, const float* __restrict__ p1,
                                                      const float* __restrict__ p2, float* __restrict__ o0,
                                                      float* __restrict__ o1, float* __restrict__ o2, int64_t n,
                                                      int S) {
  const float* p = blockIdx.y == 0 ? p0 : (blockIdx.y == 1 ? p1 : p2);
  float* o = blockIdx.y == 0 ? o0 : (blockIdx.y == 1 ? o1 : o2);
  const int64_t n4 = n / 4;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < n4; v += stride) {
    float4 acc = reinterpret_cast<const float4*>(p)[v];
    for (int s = 1; s < S; ++s) {
      const float4 q = reinterpret_cast<const float4*>(p + (int64_t)s * n)[v];
      acc.x += q.x;
      acc.y += q.y;
      acc.z += q.z;
      acc.w += q.w;
    }
    reinterpret_cast<float4*>(o)[v] = acc;
  }
}

struct Split {
  int S;      // row chunks
  int chunk;  // rows per chunk (a multiple of 64; the last one may be short)
};

// One chunk's weight-gradient launch has 3 * ceil(H/256) * ceil(F/256)
// workgroups (256 x 256 output tiles, one workgroup per CU); take as many
// chunks as fill the 256 CUs once, each of at least 512 rows.
Split split_of(const moe_launch::Dims& ds) {
  const int64_t per = 3 * ((ds.H + 255) / 256) * ((ds.F + 255) / 256);
  int64_t S = per >= 256 ? 1 : 256 / per;
  S = std::min<int64_t>(S, std::max<int64_t>(1, (ds.N + 511) / 512));
  const int64_t rows = (ds.N + S - 1) / S;
  const int64_t chunk = std::max<int64_t>(64, (rows + 63) / 64 * 64);
  return Split{int((ds.N + chunk - 1) / chunk), int(chunk)};
}

constexpr size_t align16(size_t b) { return (b + 15) & ~size_t(15); }

struct Layout {
  size_t tiles, num_tiles, offs, part, total;
};

Layout layout_of(const moe_launch::Dims& ds, bool bwd) {
  Layout l{};
  l.tiles = 0;
  l.num_tiles = align16(size_t(moe_launch::max_tiles(ds)) * 3 * sizeof(int32_t));
  l.offs = l.num_tiles + 16;
  l.part = l.offs;
  if (bwd) {
    const Split sp = split_of(ds);
    l.part = l.offs + align16(size_t(sp.S + 1) * sizeof(int32_t));
    l.total = l.part + (sp.S > 1 ? 3 * size_t(sp.S) * size_t(ds.H) * size_t(ds.F) * sizeof(float) : 0);
  } else {
    l.total = l.offs;
  }
  return l;
}

hipError_t plan(const moe_launch::Dims& ds, char* ws, const Layout& l, const Split* sp, hipStream_t s) {
  const int nt = int((ds.N + MOE_TILE_M - 1) / MOE_TILE_M);
  const int S = sp ? sp->S : 0;
  const int n = std::max(nt, S + 1);
  hipLaunchKernelGGL(k_dense_plan, dim3((n + 255) / 256), dim3(256), 0, s, reinterpret_cast<int32_t*>(ws + l.tiles),
                     reinterpret_cast<int32_t*>(ws + l.num_tiles),
                     sp ? reinterpret_cast<int32_t*>(ws + l.offs) : nullptr, int(ds.N), nt, S, sp ? sp->chunk : 0);
  return hipGetLastError();
}

}  // namespace

namespace moe_launch {

size_t shared_ffn_ws(const Dims& ds) { return layout_of(ds, false).total; }
size_t shared_ffn_bwd_ws(const Dims& ds) { return layout_of(ds, true).total; }

hipError_t shared_ffn(const Dims& ds, const void* x, const void* wg, const void* wu, const void* wd, void* g, void* u,
                      void* a, void* ys, void* ws, hipStream_t s) {
  const Layout l = layout_of(ds, false);
  char* w = static_cast<char*>(ws);
  hipError_t err = plan(ds, w, l, nullptr, s);
  if (err != hipSuccess) return err;
  const int32_t* tiles = reinterpret_cast<const int32_t*>(w + l.tiles);
  const int32_t* nt = reinterpret_cast<const int32_t*>(w + l.num_tiles);
  err = ffn_gate_up(ds, x, nullptr, wg, wu, tiles, nt, g, u, a, s);
  if (err != hipSuccess) return err;
  return ffn_down(ds, a, wd, tiles, nt, ys, s);
}

hipError_t shared_ffn_bwd(const Dims& ds, const void* x, const void* dy, const void* wg, const void* wu,
                          const void* wd, const void* g, const void* u, const void* a, void* dg, void* du, void* dxs,
                          float* dwg, float* dwu, float* dwd, void* ws, hipStream_t s) {
  const Layout l = layout_of(ds, true);
  const Split sp = split_of(ds);
  char* w = static_cast<char*>(ws);
  hipError_t err = plan(ds, w, l, &sp, s);
  if (err != hipSuccess) return err;
  const int32_t* tiles = reinterpret_cast<const int32_t*>(w + l.tiles);
  const int32_t* nt = reinterpret_cast<const int32_t*>(w + l.num_tiles);
  const int32_t* offs = reinterpret_cast<const int32_t*>(w + l.offs);
  // the shared expert's upstream gradient is dy itself (weight 1)
  err = ffn_bwd_dact(ds, dy, wd, g, u, tiles, nt, dg, du, s);
  if (err != hipSuccess) return err;
  err = ffn_bwd_dx(ds, dg, du, wg, wu, tiles, nt, dxs, s);
  if (err != hipSuccess) return err;
  Dims dc = ds;
  dc.E = sp.S;
  if (sp.S == 1) return ffn_bwd_dw(dc, x, nullptr, a, dy, dg, du, offs, dwg, dwu, dwd, s);
  const int64_t hf = ds.H * ds.F;
  float* p0 = reinterpret_cast<float*>(w + l.part);
  float* p1 = p0 + sp.S * hf;
  float* p2 = p1 + sp.S * hf;
  err = ffn_bwd_dw(dc, x, nullptr, a, dy, dg, du, offs, p0, p1, p2, s);
  if (err != hipSuccess) return err;
  const int64_t blocks = std::min<int64_t>((hf / 4 + 255) / 256, 2048);
  hipLaunchKernelGGL(k_sum_partials, dim3(unsigned(blocks), 3), dim3(256), 0, s, p0, p1, p2, dwg, dwu, dwd, hf,
                     sp.S);
  return hipGetLastError();
}

}  // namespace moe_launch
