// float32 grouped GEMMs of the SwiGLU experts (the fp32 storage type), and
// the dtype dispatch of the expert entry points.
//
// Same tile list, same tile-to-workgroup mapping and the same epilogue
// arithmetic as the bf16 MFMA path, but plain float32 FMA on the vector ALUs
// with one thread per output element and the contraction in ascending k.
// This path exists for the fp32 storage type (small correctness-sized
// problems); the bf16 path carries the performance.

#include "common.h"

namespace {
using namespace moe;

constexpr int TN = 128;  // output columns per workgroup

// sorted_flat non-null: xs is the token matrix x and row i of the grouped
// order is x[sorted_flat[i] / K] (the permute fused into the loads).
__global__ __launch_bounds__(256) void k_gate_up_f32(const float* __restrict__ xs,
                                                      const int32_t* __restrict__ sorted_flat, int K,
                                                      const float* __restrict__ wg,
                                                      const float* __restrict__ wu, const int32_t* __restrict__ tiles,
                                                      const int32_t* __restrict__ num_tiles, float* __restrict__ g_out,
                                                      float* __restrict__ u_out, float* __restrict__ a_out, int H,
                                                      int F) {
  const int ntn = F / TN;
  const int tile = blockIdx.x / ntn, nt = blockIdx.x % ntn;
  if (tile >= *num_tiles) return;
  const int e = tiles[3 * tile], row0 = tiles[3 * tile + 1], rows = tiles[3 * tile + 2];
  const float* Wg = wg + (int64_t)e * H * F;
  const float* Wu = wu + (int64_t)e * H * F;
  for (int idx = threadIdx.x; idx < rows * TN; idx += 256) {
    const int m = idx / TN, n = nt * TN + idx % TN;
    const int64_t src = sorted_flat ? sorted_flat[row0 + m] / K : row0 + m;
    const float* a = xs + src * H;
    float g = 0.f, u = 0.f;
    for (int k = 0; k < H; ++k) {
      g = fmaf(a[k], Wg[(int64_t)k * F + n], g);
      u = fmaf(a[k], Wu[(int64_t)k * F + n], u);
    }
    const int64_t o = (int64_t)(row0 + m) * F + n;
    if (g_out) g_out[o] = g;
    if (u_out) u_out[o] = u;
    a_out[o] = silu_f32(g) * u;
  }
}

__global__ __launch_bounds__(256) void k_down_f32(const float* __restrict__ act, const float* __restrict__ wd,
                                                   const int32_t* __restrict__ tiles,
                                                   const int32_t* __restrict__ num_tiles, float* __restrict__ ys, int H,
                                                   int F) {
  const int ntn = H / TN;
  const int tile = blockIdx.x / ntn, nt = blockIdx.x % ntn;
  if (tile >= *num_tiles) return;
  const int e = tiles[3 * tile], row0 = tiles[3 * tile + 1], rows = tiles[3 * tile + 2];
  const float* W = wd + (int64_t)e * F * H;
  for (int idx = threadIdx.x; idx < rows * TN; idx += 256) {
    const int m = idx / TN, n = nt * TN + idx % TN;
    const float* a = act + (int64_t)(row0 + m) * F;
    float s = 0.f;
    for (int k = 0; k < F; ++k) s = fmaf(a[k], W[(int64_t)k * H + n], s);
    ys[(int64_t)(row0 + m) * H + n] = s;
  }
}

__global__ __launch_bounds__(256) void k_dact_f32(const float* __restrict__ dys, const float* __restrict__ wd,
                                                   const float* __restrict__ g_in, const float* __restrict__ u_in,
                                                   const int32_t* __restrict__ tiles,
                                                   const int32_t* __restrict__ num_tiles, float* __restrict__ dg,
                                                   float* __restrict__ du, int H, int F) {
  const int ntn = F / TN;
  const int tile = blockIdx.x / ntn, nt = blockIdx.x % ntn;
  if (tile >= *num_tiles) return;
  const int e = tiles[3 * tile], row0 = tiles[3 * tile + 1], rows = tiles[3 * tile + 2];
  const float* W = wd + (int64_t)e * F * H;
  for (int idx = threadIdx.x; idx < rows * TN; idx += 256) {
    const int m = idx / TN, n = nt * TN + idx % TN;
    const float* a = dys + (int64_t)(row0 + m) * H;
    float da = 0.f;
    for (int k = 0; k < H; ++k) da = fmaf(a[k], W[(int64_t)n * H + k], da);
    const int64_t o = (int64_t)(row0 + m) * F + n;
    const float gv = g_in[o], uv = u_in[o];
    const float s = sigmoid_f32(gv);
    dg[o] = da * uv * s * (1.f + gv * (1.f - s));
    du[o] = da * gv * s;
  }
}

__global__ __launch_bounds__(256) void k_dx_f32(const float* __restrict__ dg, const float* __restrict__ du,
                                                 const float* __restrict__ wg, const float* __restrict__ wu,
                                                 const int32_t* __restrict__ tiles,
                                                 const int32_t* __restrict__ num_tiles, float* __restrict__ dxs, int H,
                                                 int F) {
  const int ntn = H / TN;
  const int tile = blockIdx.x / ntn, nt = blockIdx.x % ntn;
  if (tile >= *num_tiles) return;
  const int e = tiles[3 * tile], row0 = tiles[3 * tile + 1], rows = tiles[3 * tile + 2];
  const float* Wg = wg + (int64_t)e * H * F;
  const float* Wu = wu + (int64_t)e * H * F;
  for (int idx = threadIdx.x; idx < rows * TN; idx += 256) {
    const int m = idx / TN, n = nt * TN + idx % TN;
    const float* a = dg + (int64_t)(row0 + m) * F;
    const float* b = du + (int64_t)(row0 + m) * F;
    float s = 0.f;
    for (int k = 0; k < F; ++k) s = fmaf(a[k], Wg[(int64_t)n * F + k], s);
    for (int k = 0; k < F; ++k) s = fmaf(b[k], Wu[(int64_t)n * F + k], s);
    dxs[(int64_t)(row0 + m) * H + n] = s;
  }
}

// gsrc non-null: xs is x and row r of dW_gate / dW_up's rows is x[gsrc[r] / K]
__global__ __launch_bounds__(256) void k_dw_f32(const float* __restrict__ xs, const float* __restrict__ act,
                                                 const float* __restrict__ dys, const float* __restrict__ dg,
                                                 const float* __restrict__ du, const int32_t* __restrict__ offsets,
                                                 float* __restrict__ dwg, float* __restrict__ dwu,
                                                 float* __restrict__ dwd, int H, int F, int E,
                                                 const int32_t* __restrict__ gsrc, int K) {
  const int tpe = (H / TN) * (F / TN);
  const int prob = blockIdx.x / (E * tpe);
  const int rem = blockIdx.x % (E * tpe);
  const int e = rem / tpe, t = rem % tpe;
  const float *L, *R;
  float* out;
  int P, Q;
  if (prob < 2) {
    P = H; Q = F;
    L = xs; R = (prob == 0) ? dg : du;
    out = ((prob == 0) ? dwg : dwu) + (int64_t)e * H * F;
  } else {
    P = F; Q = H;
    L = act; R = dys;
    out = dwd + (int64_t)e * F * H;
  }
  const int mt = t / (Q / TN), nt = t % (Q / TN);
  const int r0 = offsets[e], r1 = offsets[e + 1];
  for (int idx = threadIdx.x; idx < TN * TN; idx += 256) {
    const int p = mt * TN + idx / TN, q = nt * TN + idx % TN;
    float s = 0.f;
    const bool gather = gsrc != nullptr && prob < 2;
    for (int r = r0; r < r1; ++r) {
      const int64_t lr = gather ? (int64_t)(gsrc[r] / K) : r;
      s = fmaf(L[lr * P + p], R[(int64_t)r * Q + q], s);
    }
    out[(int64_t)p * Q + q] = s;
  }
}

}  // namespace

namespace moe_launch {

// bf16 tile shapes: 256 x 256 and 128 x 256 (dA only) LDS-DMA kernels
// (gemm_bf16_big.hip) and 128 x 128 register-staged kernels
// (gemm_bf16_small.hip).
#define MOE_BF16_SHAPE(name, ...)                 \
  hipError_t name##_big(const Dims&, __VA_ARGS__); \
  hipError_t name##_small(const Dims&, __VA_ARGS__);
MOE_BF16_SHAPE(ffn_gate_up, const void*, const int32_t*, const void*, const void*, const int32_t*, const int32_t*, void*,
               void*, void*, hipStream_t)
MOE_BF16_SHAPE(ffn_down, const void*, const void*, const int32_t*, const int32_t*, void*, hipStream_t)
hipError_t ffn_bwd_dact_big(const Dims&, const void*, const void*, const void*, const void*, const int32_t*,
                            const int32_t*, void*, void*, hipStream_t);
hipError_t ffn_bwd_dact_mid(const Dims&, const void*, const void*, const void*, const void*, const int32_t*,
                            const int32_t*, void*, void*, hipStream_t);
hipError_t ffn_gate_up_midr(const Dims&, const void*, const int32_t*, const void*, const void*, const int32_t*,
                            const int32_t*, void*, void*, void*, hipStream_t);
hipError_t ffn_down_midr(const Dims&, const void*, const void*, const int32_t*, const int32_t*, void*, hipStream_t);
hipError_t ffn_gate_up_smallr(const Dims&, const void*, const int32_t*, const void*, const void*, const int32_t*,
                              const int32_t*, void*, void*, void*, hipStream_t);
hipError_t ffn_down_smallr(const Dims&, const void*, const void*, const int32_t*, const int32_t*, void*, hipStream_t);
hipError_t ffn_bwd_dact_midr(const Dims&, const void*, const void*, const void*, const void*, const int32_t*,
                             const int32_t*, void*, void*, hipStream_t);
hipError_t ffn_bwd_dx_midr(const Dims&, const void*, const void*, const void*, const void*, const int32_t*,
                           const int32_t*, void*, hipStream_t);
hipError_t ffn_bwd_dw_midr(const Dims&, const void*, const int32_t*, const void*, const void*, const void*,
                           const void*, const int32_t*, float*, float*, float*, hipStream_t);
MOE_BF16_SHAPE(ffn_bwd_dx, const void*, const void*, const void*, const void*, const int32_t*, const int32_t*, void*,
               hipStream_t)
MOE_BF16_SHAPE(ffn_bwd_dw, const void*, const int32_t*, const void*, const void*, const void*, const void*,
               const int32_t*, float*, float*, float*, hipStream_t)
#undef MOE_BF16_SHAPE
hipError_t ffn_bwd_dx_dw_big(const Dims&, const void*, const void*, const void*, const void*, const int32_t*,
                             const int32_t*, void*, const void*, const int32_t*, const void*, const void*,
                             const int32_t*, float*, float*, float*, hipStream_t);

// Which bf16 tile shape each stage uses.  The 256 x 256 tiles (one workgroup
// per CU: 8 waves of 64 x 128 on the mixed-depth LDS DMA loop) win on long
// contractions; the
// 128 x 128 tiles (2-3 workgroups per CU) hide latency better on short ones,
// where a 256 x 256 tile spends a large share of its time in its prologue and
// epilogue.  Measured on MI355X per stage over the shapes (H, F, rows per
// expert) = (512, 1024, 4096), (2048, 1408, skewed 0..16k), (7168, 2048,
// 256), (4096, 14336, 4096):
//   gate/up (contraction H): 256 x 256 from H = 2048 on, else 128 x 128 on
//   the register-staged loop (SmallR);
//   down (contraction F): 256 x 256 from F = 1280 on, else 128 x 128 on the
//   register-staged loop (SmallR);
//   dA (contraction H): 256 x 256 from H = 2048 on (at H = 2048, F = 1408,
//   E = 64: 0.866-0.869 -> 0.819-0.821 ms on the mixed-depth DMA loop),
//   below that 128 x 256 tiles through the LDS DMA pipeline (two workgroups
//   per CU overlap one's SwiGLU epilogue with the other's loop; at H = 512
//   the 256 x 256 tile takes 0.122 against 0.101 ms);
//   dX (contraction 2F): 256 x 256 from 2F = 2560 on;
//   dW (contraction over an expert's rows): 256 x 256 throughout.
// A forced family in Dims::tiles (moe_dims.gemm_tiles: 256, 128 x 256 or
// 128, the last selecting the 128 x 256 DMA dA tiles) overrides the choice
// for every stage of the call; AUTO keeps the measured choice.  SmallR is
// only ever the measured choice.
enum class Tiles { Small, SmallR, MidR, Big };
static Tiles pick(const Dims& d, Tiles measured) {
  switch (d.tiles) {
    case MOE_TILES_256: return Tiles::Big;
    case MOE_TILES_128X256: return Tiles::MidR;
    case MOE_TILES_128: return Tiles::Small;
    default: return measured;
  }
}
static Tiles tiles_gate_up(const Dims& d) { return pick(d, d.H >= 2048 ? Tiles::Big : Tiles::SmallR); }
static Tiles tiles_down(const Dims& d) { return pick(d, d.F >= 1280 ? Tiles::Big : Tiles::SmallR); }
static Tiles tiles_dact(const Dims& d) { return pick(d, d.H >= 2048 ? Tiles::Big : Tiles::Small); }
static Tiles tiles_dx(const Dims& d) { return pick(d, 2 * d.F >= 2560 ? Tiles::Big : Tiles::Small); }
static Tiles tiles_dw(const Dims& d) { return pick(d, Tiles::Big); }

hipError_t ffn_gate_up(const Dims& d, const void* xs, const int32_t* sorted_flat, const void* wg, const void* wu,
                       const int32_t* tiles, const int32_t* num_tiles, void* g, void* u, void* a, hipStream_t s) {
  if (d.dtype == MOE_BF16)
    switch (tiles_gate_up(d)) {
      case Tiles::Big: return ffn_gate_up_big(d, xs, sorted_flat, wg, wu, tiles, num_tiles, g, u, a, s);
      case Tiles::MidR: return ffn_gate_up_midr(d, xs, sorted_flat, wg, wu, tiles, num_tiles, g, u, a, s);
      case Tiles::SmallR: return ffn_gate_up_smallr(d, xs, sorted_flat, wg, wu, tiles, num_tiles, g, u, a, s);
      default: return ffn_gate_up_small(d, xs, sorted_flat, wg, wu, tiles, num_tiles, g, u, a, s);
    }
  unsigned grid = unsigned(max_tiles(d) * (d.F / TN));
  hipLaunchKernelGGL(k_gate_up_f32, dim3(grid), dim3(256), 0, s, static_cast<const float*>(xs), sorted_flat,
                     int(d.K), static_cast<const float*>(wg), static_cast<const float*>(wu), tiles, num_tiles,
                     static_cast<float*>(g), static_cast<float*>(u), static_cast<float*>(a), int(d.H), int(d.F));
  return hipGetLastError();
}

hipError_t ffn_down(const Dims& d, const void* a, const void* wd, const int32_t* tiles, const int32_t* num_tiles,
                    void* ys, hipStream_t s) {
  if (d.dtype == MOE_BF16)
    switch (tiles_down(d)) {
      case Tiles::Big: return ffn_down_big(d, a, wd, tiles, num_tiles, ys, s);
      case Tiles::MidR: return ffn_down_midr(d, a, wd, tiles, num_tiles, ys, s);
      case Tiles::SmallR: return ffn_down_smallr(d, a, wd, tiles, num_tiles, ys, s);
      default: return ffn_down_small(d, a, wd, tiles, num_tiles, ys, s);
    }
  unsigned grid = unsigned(max_tiles(d) * (d.H / TN));
  hipLaunchKernelGGL(k_down_f32, dim3(grid), dim3(256), 0, s, static_cast<const float*>(a),
                     static_cast<const float*>(wd), tiles, num_tiles, static_cast<float*>(ys), int(d.H), int(d.F));
  return hipGetLastError();
}

hipError_t ffn_bwd_dact(const Dims& d, const void* dys, const void* wd, const void* g, const void* u,
                        const int32_t* tiles, const int32_t* num_tiles, void* dg, void* du, hipStream_t s) {
  if (d.dtype == MOE_BF16)
    switch (tiles_dact(d)) {
      case Tiles::Big: return ffn_bwd_dact_big(d, dys, wd, g, u, tiles, num_tiles, dg, du, s);
      case Tiles::MidR: return ffn_bwd_dact_midr(d, dys, wd, g, u, tiles, num_tiles, dg, du, s);
      default: return ffn_bwd_dact_mid(d, dys, wd, g, u, tiles, num_tiles, dg, du, s);
    }
  unsigned grid = unsigned(max_tiles(d) * (d.F / TN));
  hipLaunchKernelGGL(k_dact_f32, dim3(grid), dim3(256), 0, s, static_cast<const float*>(dys),
                     static_cast<const float*>(wd), static_cast<const float*>(g), static_cast<const float*>(u), tiles,
                     num_tiles, static_cast<float*>(dg), static_cast<float*>(du), int(d.H), int(d.F));
  return hipGetLastError();
}

hipError_t ffn_bwd_dx(const Dims& d, const void* dg, const void* du, const void* wg, const void* wu,
                      const int32_t* tiles, const int32_t* num_tiles, void* dxs, hipStream_t s) {
  if (d.dtype == MOE_BF16)
    switch (tiles_dx(d)) {
      case Tiles::Big: return ffn_bwd_dx_big(d, dg, du, wg, wu, tiles, num_tiles, dxs, s);
      case Tiles::MidR: return ffn_bwd_dx_midr(d, dg, du, wg, wu, tiles, num_tiles, dxs, s);
      default: return ffn_bwd_dx_small(d, dg, du, wg, wu, tiles, num_tiles, dxs, s);
    }
  unsigned grid = unsigned(max_tiles(d) * (d.H / TN));
  hipLaunchKernelGGL(k_dx_f32, dim3(grid), dim3(256), 0, s, static_cast<const float*>(dg),
                     static_cast<const float*>(du), static_cast<const float*>(wg), static_cast<const float*>(wu), tiles,
                     num_tiles, static_cast<float*>(dxs), int(d.H), int(d.F));
  return hipGetLastError();
}

hipError_t ffn_bwd_dw(const Dims& d, const void* xs, const int32_t* sorted_flat, const void* a, const void* dys,
                      const void* dg, const void* du, const int32_t* offsets, float* dwg, float* dwu, float* dwd,
                      hipStream_t s) {
  if (d.dtype == MOE_BF16)
    switch (tiles_dw(d)) {
      case Tiles::Big: return ffn_bwd_dw_big(d, xs, sorted_flat, a, dys, dg, du, offsets, dwg, dwu, dwd, s);
      case Tiles::MidR: return ffn_bwd_dw_midr(d, xs, sorted_flat, a, dys, dg, du, offsets, dwg, dwu, dwd, s);
      default: return ffn_bwd_dw_small(d, xs, sorted_flat, a, dys, dg, du, offsets, dwg, dwu, dwd, s);
    }
  unsigned grid = unsigned(3 * d.E * (d.H / TN) * (d.F / TN));
  hipLaunchKernelGGL(k_dw_f32, dim3(grid), dim3(256), 0, s, static_cast<const float*>(xs),
                     static_cast<const float*>(a), static_cast<const float*>(dys), static_cast<const float*>(dg),
                     static_cast<const float*>(du), offsets, dwg, dwu, dwd, int(d.H), int(d.F), int(d.E), sorted_flat,
                     int(d.K));
  return hipGetLastError();
}

// dX and the weight gradients.  bf16: one launch of 256 x 256 tiles, the
// weight-gradient tiles first and the dX tiles filling the CUs they leave
// idle (at (H, F, E) = (512, 1024, 8) the weight gradients alone have 192
// workgroups for 256 CUs); with a forced tile family the two stages run as
// separate launches of that family.  float32: two launches.
hipError_t ffn_bwd_dx_dw(const Dims& d, const void* dg, const void* du, const void* wg, const void* wu,
                         const int32_t* tiles, const int32_t* num_tiles, void* dxs, const void* xs,
                         const int32_t* sorted_flat, const void* a, const void* dys, const int32_t* offsets,
                         float* dwg, float* dwu, float* dwd, hipStream_t s) {
  if (d.dtype == MOE_BF16 && d.tiles == MOE_TILES_AUTO)
    return ffn_bwd_dx_dw_big(d, dg, du, wg, wu, tiles, num_tiles, dxs, xs, sorted_flat, a, dys, offsets, dwg, dwu,
                             dwd, s);
  hipError_t st = ffn_bwd_dx(d, dg, du, wg, wu, tiles, num_tiles, dxs, s);
  if (st != hipSuccess) return st;
  return ffn_bwd_dw(d, xs, sorted_flat, a, dys, dg, du, offsets, dwg, dwu, dwd, s);
}

}  // namespace moe_launch
