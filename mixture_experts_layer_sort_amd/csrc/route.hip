// Router of the MoE layer: logits x.W_r (+ bias), wavefront top-K and
// renormalised gates; and its backward (dlogits and dW_r).
//
// Forward ("MoE computation principle and execution process", icman.com.cn,
// sections 2.1-2.2; top-k on logits then softmax over the K values,
// "MoE technical analysis: from theory to practice", section 2.3):
//   one workgroup owns 32 tokens; the logits [32, E] are accumulated in
//   float32 registers over H in LDS-staged chunks (h ascending, so the sum
//   order is fixed), parked in LDS, then each wave selects the top-K of 8
//   tokens with K rounds of a wave-wide arg-max under the order (logit desc,
//   expert id asc).
// Backward (icman section 2.2: the gradient reaches the router only through
//   the continuous gate values):
//   dlogits[n, e_k] = g_k (dg_k - sum_j g_j dg_j), zero elsewhere; dW_r is
//   reduced over a fixed partition of the tokens (one LDS accumulator per
//   (expert, h) per chunk, tokens ascending), then the chunk partials are
//   summed in ascending chunk order.
#include "common.h"

namespace {
using namespace moe;

constexpr int kRouteTok = 32;  // tokens per workgroup
constexpr int kRouteHC = 16;   // h per LDS chunk (keeps LDS <= 64 KB at E = 256)

template <typename T, int EPT>
__global__ __launch_bounds__(256) void k_route(const T* __restrict__ x, const T* __restrict__ w_r,
                                               const float* __restrict__ bias, int32_t* __restrict__ topk,
                                               float* __restrict__ gates, int N, int H, int E, int K) {
  constexpr int EP = 8 * EPT;  // padded experts
  extern __shared__ float smem[];
  float* xs_t = smem;                        // [HC][32]   x chunk, transposed
  float* w_l = xs_t + kRouteHC * kRouteTok;  // [HC][EP]   W_r chunk
  float* lg = w_l + kRouteHC * EP;           // [32][EP+1] logits

  const int tid = threadIdx.x;
  const int t = tid & 31;   // token within the block
  const int j = tid >> 5;   // expert group: experts j*EPT .. j*EPT+EPT-1
  const int n0 = blockIdx.x * kRouteTok;

  float acc[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) acc[i] = 0.f;

  for (int h0 = 0; h0 < H; h0 += kRouteHC) {
    // stage x[n0:n0+32, h0:h0+HC] (transposed) and W_r[h0:h0+HC, :]
    for (int idx = tid; idx < kRouteTok * kRouteHC; idx += 256) {
      int tt = idx / kRouteHC, hh = idx % kRouteHC;
      int n = n0 + tt;
      xs_t[hh * kRouteTok + tt] = (n < N) ? Elt<T>::load(x + (int64_t)n * H + h0 + hh) : 0.f;
    }
    for (int idx = tid; idx < kRouteHC * EP; idx += 256) {
      int hh = idx / EP, e = idx % EP;
      w_l[idx] = (e < E) ? Elt<T>::load(w_r + (int64_t)(h0 + hh) * E + e) : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int hh = 0; hh < kRouteHC; ++hh) {
      float xv = xs_t[hh * kRouteTok + t];
      const float* wrow = w_l + hh * EP + j * EPT;
#pragma unroll
      for (int i = 0; i < EPT; ++i) acc[i] = fmaf(xv, wrow[i], acc[i]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    int e = j * EPT + i;
    float v = acc[i];
    if (e < E && bias) v += bias[e];
    lg[t * (EP + 1) + e] = (e < E) ? v : -INFINITY;
  }
  __syncthreads();

  // top-K: wave w handles tokens w*8 .. w*8+7
  const int lane = lane_id();
  const int w = tid >> 6;
  for (int q = 0; q < kRouteTok / 4; ++q) {
    const int tt = w * (kRouteTok / 4) + q;
    const int n = n0 + tt;
    if (n >= N) break;  // uniform across the wave
    // each lane holds experts lane, lane+64, lane+128, lane+192
    float v[4];
    int id[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      int e = lane + 64 * c;
      float val = (e < E) ? lg[tt * (EP + 1) + e] : -INFINITY;
      if (val != val) val = -INFINITY;  // NaN logits rank last
      v[c] = val;
      id[c] = (e < E) ? e : 0x7fffffff;  // sentinel: never beats a real expert
    }
    float sel_v[MOE_MAX_TOPK];
    int sel_e[MOE_MAX_TOPK];
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK; ++k) {
      if (k < K) {
        // lane-local best
        float bv = v[0];
        int be = id[0];
#pragma unroll
        for (int c = 1; c < 4; ++c)
          if (v[c] > bv || (v[c] == bv && id[c] < be)) { bv = v[c]; be = id[c]; }
        // wave arg-max, (value desc, id asc)
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
          float ov = __shfl_xor(bv, off, kWave);
          int oe = __shfl_xor(be, off, kWave);
          if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
        }
        sel_v[k] = bv;
        sel_e[k] = be;
        // remove the winner
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (id[c] == be) { v[c] = -INFINITY; id[c] = 0x7fffffff; }
      }
    }
    // gates: softmax over the selected logits (sel_v[0] is the largest)
    float z[MOE_MAX_TOPK];
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK; ++k) {
      z[k] = (k < K) ? expf(sel_v[k] - sel_v[0]) : 0.f;
      s += z[k];
    }
    if (lane < K) {
      float zk = 0.f;
      int ek = 0;
#pragma unroll
      for (int k = 0; k < MOE_MAX_TOPK; ++k)
        if (k == lane) { zk = z[k]; ek = sel_e[k]; }
      topk[(int64_t)n * K + lane] = ek;
      gates[(int64_t)n * K + lane] = zk / s;
    }
  }
}

// dlogits, dense [N, E]: one thread per element.
__global__ __launch_bounds__(256) void k_route_bwd_dl(const int32_t* __restrict__ topk, const float* __restrict__ gates,
                                                      const float* __restrict__ dgates, float* __restrict__ dl, int N,
                                                      int E, int K) {
  int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)N * E) return;
  int n = int(idx / E), e = int(idx % E);
  const int32_t* tk = topk + (int64_t)n * K;
  const float* g = gates + (int64_t)n * K;
  const float* dg = dgates + (int64_t)n * K;
  float s = 0.f;
  for (int k = 0; k < K; ++k) s = fmaf(g[k], dg[k], s);
  float out = 0.f;
  for (int k = 0; k < K; ++k)
    if (tk[k] == e) out = g[k] * (dg[k] - s);
  dl[idx] = out;
}

constexpr int kRbH = 64;  // h per workgroup in the dW_r partial kernel (LDS E*64 floats <= 64 KB)

// Partial dW_r of one token chunk: part[c][e][h] = sum_{n in chunk} x[n,h] dl[n,e]
// (sparse in e: only the K selected experts of each token contribute).
template <typename T>
__global__ __launch_bounds__(kRbH) void k_route_bwd_partial(const T* __restrict__ x, const int32_t* __restrict__ topk,
                                                            const float* __restrict__ dl, float* __restrict__ part,
                                                            int N, int H, int E, int K, int chunk) {
  extern __shared__ float acc[];  // [E][kRbH]
  const int t = threadIdx.x;
  const int h = blockIdx.x * kRbH + t;
  const int c = blockIdx.y;
  for (int e = 0; e < E; ++e) acc[e * kRbH + t] = 0.f;
  const int nb = c * chunk, ne = min(N, nb + chunk);
  for (int n = nb; n < ne; ++n) {
    float xv = Elt<T>::load(x + (int64_t)n * H + h);
    for (int k = 0; k < K; ++k) {
      int e = topk[(int64_t)n * K + k];
      float d = dl[(int64_t)n * E + e];
      acc[e * kRbH + t] = fmaf(xv, d, acc[e * kRbH + t]);
    }
  }
  float* out = part + (int64_t)c * E * H;
  for (int e = 0; e < E; ++e) out[(int64_t)e * H + h] = acc[e * kRbH + t];
}

// dW_r[h, e] = sum over chunks (ascending) of part[c][e][h].
__global__ __launch_bounds__(256) void k_route_bwd_reduce(const float* __restrict__ part, float* __restrict__ dw_r,
                                                          int H, int E, int nchunks) {
  int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)E * H) return;
  int e = int(idx / H), h = int(idx % H);
  float s = 0.f;
  for (int c = 0; c < nchunks; ++c) s += part[(int64_t)c * E * H + idx];
  dw_r[(int64_t)h * E + e] = s;
}

template <typename T, int EPT>
hipError_t launch_route_t(const moe_launch::Dims& d, const void* x, const void* w_r, const float* bias, int32_t* topk,
                          float* gates, hipStream_t s) {
  constexpr int EP = 8 * EPT;
  size_t lds = sizeof(float) * (kRouteHC * kRouteTok + kRouteHC * EP + kRouteTok * (EP + 1));
  int grid = int((d.N + kRouteTok - 1) / kRouteTok);
  hipLaunchKernelGGL((k_route<T, EPT>), dim3(grid), dim3(256), lds, s, static_cast<const T*>(x),
                     static_cast<const T*>(w_r), bias, topk, gates, int(d.N), int(d.H), int(d.E), int(d.K));
  return hipGetLastError();
}

template <typename T>
hipError_t launch_route(const moe_launch::Dims& d, const void* x, const void* w_r, const float* bias, int32_t* topk,
                        float* gates, hipStream_t s) {
  if (d.E <= 8) return launch_route_t<T, 1>(d, x, w_r, bias, topk, gates, s);
  if (d.E <= 16) return launch_route_t<T, 2>(d, x, w_r, bias, topk, gates, s);
  if (d.E <= 32) return launch_route_t<T, 4>(d, x, w_r, bias, topk, gates, s);
  if (d.E <= 64) return launch_route_t<T, 8>(d, x, w_r, bias, topk, gates, s);
  if (d.E <= 128) return launch_route_t<T, 16>(d, x, w_r, bias, topk, gates, s);
  return launch_route_t<T, 32>(d, x, w_r, bias, topk, gates, s);
}

}  // namespace

namespace moe_launch {

hipError_t route(const Dims& d, const void* x, const void* w_r, const float* bias, int32_t* topk, float* gates,
                 hipStream_t s) {
  if (d.dtype == MOE_BF16) return launch_route<moe::bf16_t>(d, x, w_r, bias, topk, gates, s);
  return launch_route<float>(d, x, w_r, bias, topk, gates, s);
}

size_t route_bwd_chunks(const Dims& d) {
  int64_t c = (d.N + 511) / 512;
  if (c < 1) c = 1;
  if (c > 64) c = 64;
  return size_t(c);
}

size_t route_bwd_ws(const Dims& d) { return route_bwd_chunks(d) * size_t(d.E) * size_t(d.H) * sizeof(float); }

hipError_t route_bwd(const Dims& d, const void* x, const int32_t* topk, const float* gates, const float* dgates,
                     float* dlogits, float* dw_r, void* ws, hipStream_t s) {
  int64_t ne = d.N * d.E;
  hipLaunchKernelGGL(k_route_bwd_dl, dim3(unsigned((ne + 255) / 256)), dim3(256), 0, s, topk, gates, dgates, dlogits,
                     int(d.N), int(d.E), int(d.K));
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  int nch = int(route_bwd_chunks(d));
  int chunk = int((d.N + nch - 1) / nch);
  float* part = static_cast<float*>(ws);
  size_t lds = sizeof(float) * size_t(d.E) * kRbH;
  dim3 grid(unsigned(d.H / kRbH), unsigned(nch));
  if (d.dtype == MOE_BF16)
    hipLaunchKernelGGL(k_route_bwd_partial<moe::bf16_t>, grid, dim3(kRbH), lds, s,
                       static_cast<const moe::bf16_t*>(x), topk, dlogits, part, int(d.N), int(d.H), int(d.E), int(d.K),
                       chunk);
  else
    hipLaunchKernelGGL(k_route_bwd_partial<float>, grid, dim3(kRbH), lds, s, static_cast<const float*>(x), topk,
                       dlogits, part, int(d.N), int(d.H), int(d.E), int(d.K), chunk);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  int64_t nw = d.E * d.H;
  hipLaunchKernelGGL(k_route_bwd_reduce, dim3(unsigned((nw + 255) / 256)), dim3(256), 0, s, part, dw_r, int(d.H),
                     int(d.E), nch);
  return hipGetLastError();
}

}  // namespace moe_launch
