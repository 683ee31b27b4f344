// Device helpers shared by the HIP kernels of the MoE layer (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;

typedef uint16_t bf16_t;  // bfloat16 storage (upper half of a float32)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t v) { return __uint_as_float(uint32_t(v) << 16); }

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// float32 -> bfloat16, round to nearest, ties to even; NaN stays NaN.  gfx950
// converts in hardware (v_cvt_pk_bf16_f32, two values per instruction); it
// agrees bit for bit with the integer formulation (add 0x7fff plus the lowest
// kept bit, keep the upper half; NaN: quiet bit set), denormals included.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f)); }

// Two floats -> two bfloat16 packed in one word (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Element-type traits: loads return float, stores round to the type.
template <typename T> struct Elt;
template <> struct Elt<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float to_f32(float v) { return v; }
  static __device__ __forceinline__ float from_f32(float v) { return v; }
};
template <> struct Elt<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ float to_f32(bf16_t v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

// 16-byte vector of elements of type T, converted to / from float.
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int n = 4;
  static __device__ __forceinline__ void load(const float* p, float* out) {
    float4 v = *reinterpret_cast<const float4*>(p);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* in) {
    *reinterpret_cast<float4*>(p) = make_float4(in[0], in[1], in[2], in[3]);
  }
};
template <> struct Vec16<bf16_t> {
  static constexpr int n = 8;
  static __device__ __forceinline__ void load(const bf16_t* p, float* out) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float* in) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(in[2 * i], in[2 * i + 1]);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};

__device__ __forceinline__ float wave_sum(float v) {
  // fixed butterfly order: bitwise reproducible
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// silu and sigmoid with the hardware exponential and reciprocal (a few ulp of
// float32; the storage rounding to bfloat16 that follows dominates).
__device__ __forceinline__ float sigmoid_f32(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }
__device__ __forceinline__ float silu_f32(float g) { return g * sigmoid_f32(g); }

// Windowed XCD mapping: the hardware deals workgroup b to XCD b % 8.  Within
// each window of 8 * kXcdRun consecutive workgroups, XCD x gets the kXcdRun
// consecutive logical blocks [x * kXcdRun, (x + 1) * kXcdRun), so blocks that
// share operand panels run on one XCD and share its L2, while the logical
// order still advances through all XCDs together.  The launch grid must be a
// multiple of 8 * kXcdRun; returns -1 for blocks past `total`.
constexpr int kXcdRun = 8;
template <int RUN = kXcdRun>
__device__ __forceinline__ int xcd_window_block(int b, int total) {
  const int L = (b / (8 * RUN)) * (8 * RUN) + (b % 8) * RUN + (b / 8) % RUN;
  return L < total ? L : -1;
}
__device__ __forceinline__ int xcd_window_block(int total) { return xcd_window_block<kXcdRun>(blockIdx.x, total); }

// Largest row count of any expert, from offsets [E+1]; computed by each wave
// on its own (the same value in every lane and wave).
__device__ __forceinline__ int max_expert_rows(const int32_t* __restrict__ offsets, int E) {
  int m = 0;
  for (int e = lane_id(); e < E; e += kWave) m = max(m, offsets[e + 1] - offsets[e]);
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) m = max(m, __shfl_xor(m, off, kWave));
  return m;
}

// The expert of rank p when experts are ordered by row count, largest first
// (equal counts: lower id first), from offsets [E+1].  The weight-gradient
// workgroups take their expert in this order, so the longest contractions
// are dispatched first and spread over every XCD instead of forming a tail.
// s: 16-byte aligned LDS scratch of at least MOE_MAX_EXPERTS + 1 ints; the
// call holds two barriers and leaves s free for reuse.
template <int NT>
__device__ __forceinline__ int expert_of_rank(const int32_t* __restrict__ offsets, int E, int p, int* s) {
  const int E4 = (E + 3) & ~3;
  for (int i = threadIdx.x; i < E4; i += NT) s[i] = i < E ? offsets[i + 1] - offsets[i] : -1;
  __syncthreads();
  for (int j = threadIdx.x; j < E; j += NT) {
    const int c = s[j];
    int above = 0;
    for (int i = 0; i < E4; i += 4) {
      const int4 v = *reinterpret_cast<const int4*>(s + i);
      above += (v.x > c || (v.x == c && i < j)) + (v.y > c || (v.y == c && i + 1 < j)) +
               (v.z > c || (v.z == c && i + 2 < j)) + (v.w > c || (v.w == c && i + 3 < j));
    }
    if (above == p) s[MOE_MAX_EXPERTS] = j;
  }
  __syncthreads();
  const int e = s[MOE_MAX_EXPERTS];
  __syncthreads();
  return e;
}

}  // namespace moe

// Host-side launch helpers (defined in the kernel sources).
namespace moe_launch {
struct Dims {
  int64_t N, H, F, E, K;
  int dtype;
  int tiles = 0;  // moe_gemm_tiles: 0 = chosen per stage
  int64_t NK() const { return N * K; }
};
int64_t max_tiles(const Dims& d);
size_t route_bwd_chunks(const Dims& d);

// hist (optional, [ceil(N / 32)][E]): each 32-token block's histogram of
// the chosen experts.
hipError_t route(const Dims& d, const void* x, const void* w_r, const float* bias, int32_t* topk, float* gates,
                 hipStream_t s, int32_t* hist = nullptr);
// route + permute_meta (with a capacity; INT32_MAX: dropless), fused into
// two launches when the block histograms are small enough.
size_t route_meta_ws(const Dims& d);
hipError_t route_meta(const Dims& d, const void* x, const void* w_r, const float* bias, int32_t capacity,
                      int32_t* topk, float* gates, int32_t* sorted_flat, int32_t* inv, int32_t* counts,
                      int32_t* offsets, int32_t* tiles, int32_t* num_tiles, void* ws, hipStream_t s);
hipError_t permute_meta(const Dims& d, const int32_t* topk, int32_t capacity, int32_t* sorted_flat, int32_t* inv,
                        int32_t* counts, int32_t* offsets, int32_t* tiles, int32_t* num_tiles, void* ws,
                        hipStream_t s);
size_t permute_meta_ws(const Dims& d);
hipError_t permute(const Dims& d, const void* x, const int32_t* sorted_flat, void* xs, hipStream_t s);
// add (optional, [N,H], may be null): a row added with weight 1 to each
// token's result (the shared expert's output / input gradient).
hipError_t combine(const Dims& d, const void* ys, const float* gates, const int32_t* inv, const void* add, void* y,
                   hipStream_t s);
hipError_t combine_bwd(const Dims& d, const void* dy, const void* ys, const float* gates, const int32_t* inv,
                       void* dys, float* dgates, hipStream_t s);
hipError_t route_bwd(const Dims& d, const void* x, const int32_t* topk, const float* gates, const float* dgates,
                     float* dlogits, float* dw_r, void* ws, hipStream_t s);
size_t route_bwd_ws(const Dims& d);
size_t aux_loss_ws(const Dims& d);
hipError_t aux_loss(const Dims& d, const void* x, const void* w_r, const float* bias, const int32_t* counts,
                    float alpha, float* probs, float* loss, void* ws, hipStream_t s);
size_t route_bwd_aux_ws(const Dims& d);
hipError_t route_bwd_aux(const Dims& d, const void* x, const int32_t* topk, const float* gates, const float* dgates,
                         const float* probs, const int32_t* counts, float aux_scale, float* dlogits, float* dw_r,
                         void* ws, hipStream_t s);
hipError_t permute_bwd(const Dims& d, const void* dxs, const int32_t* inv, const int32_t* topk, const float* dlogits,
                       const void* w_r, const void* add, void* dx, void* ws, hipStream_t s, bool dense);
size_t permute_bwd_ws(const Dims& d);

// sorted_flat non-null: xs is the token matrix x and the rows are gathered
// on load (row i = x[sorted_flat[i] / K]); null: xs is the grouped matrix.
hipError_t ffn_gate_up(const Dims& d, const void* xs, const int32_t* sorted_flat, const void* wg, const void* wu,
                       const int32_t* tiles, const int32_t* num_tiles, void* g, void* u, void* a, hipStream_t s);
hipError_t ffn_down(const Dims& d, const void* a, const void* wd, const int32_t* tiles, const int32_t* num_tiles,
                    void* ys, hipStream_t s);
hipError_t ffn_bwd_dact(const Dims& d, const void* dys, const void* wd, const void* g, const void* u,
                        const int32_t* tiles, const int32_t* num_tiles, void* dg, void* du, hipStream_t s);
hipError_t ffn_bwd_dx(const Dims& d, const void* dg, const void* du, const void* wg, const void* wu,
                      const int32_t* tiles, const int32_t* num_tiles, void* dxs, hipStream_t s);
// sorted_flat non-null: xs is the token matrix x and dW_gate / dW_up read
// row i of the grouped order as x[sorted_flat[i] / K]; null: xs is the
// grouped matrix.
hipError_t ffn_bwd_dw(const Dims& d, const void* xs, const int32_t* sorted_flat, const void* a, const void* dys,
                      const void* dg, const void* du, const int32_t* offsets, float* dwg, float* dwu, float* dwd,
                      hipStream_t s);
// ffn_bwd_dx and ffn_bwd_dw together (one launch for bf16).
hipError_t ffn_bwd_dx_dw(const Dims& d, const void* dg, const void* du, const void* wg, const void* wu,
                         const int32_t* tiles, const int32_t* num_tiles, void* dxs, const void* xs,
                         const int32_t* sorted_flat, const void* a, const void* dys, const int32_t* offsets,
                         float* dwg, float* dwu, float* dwd, hipStream_t s);

// Shared expert: a dense SwiGLU expert over all N tokens (dims E = K = 1,
// F = its intermediate size).  The workspace holds its tile list, the row
// chunks of its split weight gradient and their float32 partial sums.
size_t shared_ffn_ws(const Dims& ds);
size_t shared_ffn_bwd_ws(const Dims& ds);
hipError_t shared_ffn(const Dims& ds, const void* x, const void* wg, const void* wu, const void* wd, void* g, void* u,
                      void* a, void* ys, void* ws, hipStream_t s);
hipError_t shared_ffn_bwd(const Dims& ds, const void* x, const void* dy, const void* wg, const void* wu,
                          const void* wd, const void* g, const void* u, const void* a, void* dg, void* du, void* dxs,
                          float* dwg, float* dwu, float* dwd, void* ws, hipStream_t s);
}  // namespace moe_launch
