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
#include <type_traits>

#include "common.h"
#include "mma_lds.h"

namespace {
using namespace moe;

constexpr int kRouteTok = 32;  // tokens per workgroup

// h per staged chunk: the W_r chunk [HC][EP] float32 stays within 32 KiB and
// the x chunk [HC][32] within 16 KiB
template <int EPT>
constexpr int route_hc() {
  return (8192 / (8 * EPT)) < 128 ? (8192 / (8 * EPT)) : 128;
}

// Top-K of one token's logits lg[0, E) (+ bias[e] if given) under the order
// (logit desc, expert id asc), and the gates: softmax over the K selected
// logits.  Called by a whole wave; lane k < K writes slot k of token n.
// Each lane holds experts lane, lane+64, lane+128, lane+192; NaN logits rank
// last; K rounds of a wave-wide arg-max pick the winners.
// lhist (LDS, optional): the chosen experts are counted into lhist[e].
__device__ __forceinline__ void wave_topk_gates(const float* __restrict__ lg, const float* __restrict__ bias, int E,
                                                int K, int64_t n, int32_t* __restrict__ topk,
                                                float* __restrict__ gates, int* lhist = nullptr) {
  const int lane = lane_id();
  float v[4];
  int id[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = lane + 64 * c;
    float val = -INFINITY;
    if (e < E) {
      val = lg[e];
      if (bias) val += bias[e];
    }
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
    topk[n * K + lane] = ek;
    gates[n * K + lane] = zk / s;
    if (lhist) atomicAdd(&lhist[ek], 1);
  }
}

// Load-balancing loss, forward part ("MoE computation principle and
// execution process", section 4.2): the full softmax over the E experts of
// each of the block's `rows` tokens, from the logits lg [rows][LP] in LDS
// (+ bias[e] if given), stored to probs [N, E]; and the block's column sums of
// the probabilities (tokens ascending) to part[0, E), summed over the blocks
// in a fixed order afterwards.
template <int NT>
__device__ __forceinline__ void probs_epilogue(float* lg, int LP, int rows, int64_t n0, int E,
                                               const float* __restrict__ bias, float* __restrict__ probs,
                                               float* __restrict__ part) {
  for (int tt = threadIdx.x; tt < rows; tt += NT) {
    float* l = lg + tt * LP;
    float m = -INFINITY;
    for (int e = 0; e < E; ++e) {
      const float v = l[e] + (bias ? bias[e] : 0.f);
      l[e] = v;
      m = fmaxf(m, v);
    }
    float sum = 0.f;
    for (int e = 0; e < E; ++e) {
      const float z = __expf(l[e] - m);
      l[e] = z;
      sum += z;
    }
    const float r = 1.0f / sum;
    for (int e = 0; e < E; ++e) l[e] *= r;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += NT) {
    float c = 0.f;
    for (int tt = 0; tt < rows; ++tt) {
      const float p = lg[tt * LP + e];
      probs[(n0 + tt) * E + e] = p;
      c += p;
    }
    part[e] = c;
  }
}

// hist (optional, [gridDim.x][E]): this block's histogram of the chosen
// experts (integer LDS atomics: the counts do not depend on their order).
template <typename T, int EPT>
__global__ __launch_bounds__(256) void k_route(const T* __restrict__ x, const T* __restrict__ w_r,
                                               const float* __restrict__ bias, int32_t* __restrict__ topk,
                                               float* __restrict__ gates, int N, int H, int E, int K,
                                               float* __restrict__ probs, float* __restrict__ part,
                                               int32_t* __restrict__ hist) {
  constexpr int EP = 8 * EPT;  // padded experts
  constexpr int HC = route_hc<EPT>();
  constexpr int V = Vec16<T>::n;
  constexpr int XV = (kRouteTok * HC / V + 255) / 256;   // x vectors per thread per chunk
  constexpr int WV = (HC * EP / V + 255) / 256;          // W_r vectors per thread per chunk (upper bound)
  extern __shared__ float smem[];
  float* xs_t = smem;                        // [HC][32]   x chunk, transposed
  float* w_l = xs_t + HC * kRouteTok;        // [HC][EP]   W_r chunk
  float* lg = smem;                          // [32][EP+1] logits, reuses the staging space after the h loop
  constexpr int HC_ = HC;
  constexpr int LG_FLOATS = (HC_ * kRouteTok + HC_ * EP) > kRouteTok * (EP + 1) ? (HC_ * kRouteTok + HC_ * EP)
                                                                                 : kRouteTok * (EP + 1);
  int* lhist = reinterpret_cast<int*>(smem + LG_FLOATS);  // [E] past the staging space

  const int tid = threadIdx.x;
  const int t = tid & 31;   // token within the block
  const int j = tid >> 5;   // expert group: experts j*EPT .. j*EPT+EPT-1
  const int n0 = blockIdx.x * kRouteTok;
  const int wvec = HC * E / V;  // vectors in one W_r chunk (rows h0..h0+HC-1 are contiguous)

  float acc[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) acc[i] = 0.f;

  uint4 xr[XV], wr[WV];
  auto fetch = [&](int h0) {
#pragma unroll
    for (int q = 0; q < XV; ++q) {
      const int idx = tid + 256 * q;
      const int tt = idx / (HC / V), hv = idx % (HC / V);
      xr[q] = (idx < kRouteTok * HC / V && n0 + tt < N)
                  ? *reinterpret_cast<const uint4*>(x + (int64_t)(n0 + tt) * H + h0 + hv * V)
                  : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < WV; ++q) {
      const int idx = tid + 256 * q;
      wr[q] = (idx < wvec) ? *reinterpret_cast<const uint4*>(w_r + (int64_t)h0 * E + idx * V)
                           : make_uint4(0, 0, 0, 0);
    }
  };
  auto deposit = [&]() {
#pragma unroll
    for (int q = 0; q < XV; ++q) {
      const int idx = tid + 256 * q;
      if (idx < kRouteTok * HC / V) {
        const int tt = idx / (HC / V), hv = idx % (HC / V);
        float v[V];
        Vec16<T>::load(reinterpret_cast<const T*>(&xr[q]), v);
#pragma unroll
        for (int i = 0; i < V; ++i) xs_t[(hv * V + i) * kRouteTok + tt] = v[i];
      }
    }
#pragma unroll
    for (int q = 0; q < WV; ++q) {
      const int idx = tid + 256 * q;
      if (idx < wvec) {
        float v[V];
        Vec16<T>::load(reinterpret_cast<const T*>(&wr[q]), v);
#pragma unroll
        for (int i = 0; i < V; ++i) {
          const int el = idx * V + i;
          w_l[(el / E) * EP + el % E] = v[i];
        }
      }
    }
  };
  // padded experts of the W_r chunk stay zero
  for (int idx = tid; idx < HC * EP; idx += 256) w_l[idx] = 0.f;
  fetch(0);
  for (int h0 = 0; h0 < H; h0 += HC) {
    __syncthreads();
    deposit();
    __syncthreads();
    if (h0 + HC < H) fetch(h0 + HC);
#pragma unroll 4
    for (int hh = 0; hh < HC; ++hh) {
      const float xv = xs_t[hh * kRouteTok + t];
      const float* wrow = w_l + hh * EP + j * EPT;
#pragma unroll
      for (int i = 0; i < EPT; ++i) acc[i] = fmaf(xv, wrow[i], acc[i]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    int e = j * EPT + i;
    float v = acc[i];
    if (e < E && bias) v += bias[e];
    lg[t * (EP + 1) + e] = (e < E) ? v : -INFINITY;
  }
  __syncthreads();

  if (probs) {  // load-balancing loss: full softmax instead of the top-K
    probs_epilogue<256>(lg, EP + 1, min(kRouteTok, N - n0), n0, E, nullptr, probs, part + (int64_t)blockIdx.x * E);
    return;
  }
  if (hist) {
    for (int e = tid; e < E; e += 256) lhist[e] = 0;
    __syncthreads();
  }
  // top-K: wave w handles tokens w*8 .. w*8+7
  const int w = tid >> 6;
  for (int q = 0; q < kRouteTok / 4; ++q) {
    const int tt = w * (kRouteTok / 4) + q;
    const int n = n0 + tt;
    if (n >= N) break;  // uniform across the wave
    wave_topk_gates(lg + tt * (EP + 1), nullptr, E, K, n, topk, gates, hist ? lhist : nullptr);
  }
  if (hist) {
    __syncthreads();
    for (int e = tid; e < E; e += 256) hist[(int64_t)blockIdx.x * E + e] = lhist[e];
  }
}

// Top-K of one token by a single lane: one pass over the logits lg[0, E)
// (+ bias[e] if given) keeps a sorted list of K (value, id) under the order
// (logit desc, expert id asc); each new logit is pushed down the list by
// predicated swaps.  NaN logits rank last; the sentinel id never beats a real
// expert.  Then the gates (softmax over the K selected logits) and both
// outputs of token n.
__device__ __forceinline__ void lane_topk_gates(const float* __restrict__ lg, const float* __restrict__ bias, int E,
                                                int K, int64_t n, int32_t* __restrict__ topk,
                                                float* __restrict__ gates, int* lhist = nullptr) {
  float tv[MOE_MAX_TOPK];
  int te[MOE_MAX_TOPK];
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK; ++k) {
    tv[k] = -INFINITY;
    te[k] = 0x7fffffff;
  }
  for (int e = 0; e < E; ++e) {
    float cv = lg[e];
    if (bias) cv += bias[e];
    if (cv != cv) cv = -INFINITY;
    int ce = e;
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK; ++k) {
      const bool better = k < K && (cv > tv[k] || (cv == tv[k] && ce < te[k]));
      const float ov = tv[k];
      const int oe = te[k];
      tv[k] = better ? cv : ov;
      te[k] = better ? ce : oe;
      cv = better ? ov : cv;
      ce = better ? oe : ce;
    }
  }
  float z[MOE_MAX_TOPK];
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK; ++k) {
    z[k] = (k < K) ? expf(tv[k] - tv[0]) : 0.f;
    s += z[k];
  }
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK; ++k)
    if (k < K) {
      topk[n * K + k] = te[k];
      gates[n * K + k] = z[k] / s;
      if (lhist) atomicAdd(&lhist[te[k]], 1);
    }
}

// Router logits on the matrix cores (bf16 storage, E a multiple of 8): one
// workgroup owns C::BM tokens and every expert, padded to C::BN columns (the
// padding columns read clamped in-bounds W_r columns and are masked before
// the top-K).  logits = x.W_r with exact bf16 products accumulated in float32
// over h ascending, 64 h per pipeline stage; the logits then go through LDS
// and one lane per token selects its top-K (E <= 64), or one wave per token
// (more experts: a lane's single pass would be long).
template <class C>
__global__ __launch_bounds__(C::NT, C::MINB) void k_route_mma(const bf16_t* __restrict__ x,
                                                             const bf16_t* __restrict__ w_r,
                                                             const float* __restrict__ bias,
                                                             int32_t* __restrict__ topk, float* __restrict__ gates,
                                                             int N, int H, int E, int K, float* __restrict__ probs,
                                                             float* __restrict__ part, int32_t* __restrict__ hist) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int n0 = blockIdx.x * C::BM;
  const int rows = min(C::BM, N - n0);
  const int w = threadIdx.x >> 6, wm = w / C::WN, wn = w % C::WN;
  moe_mma::Acc<C> acc;
  moe_mma::k_loop<C, false, true>(
      lds, acc, H / C::BK,
      [&](int kt, char* st, int j) { moe_mma::dma_kc<C::BM, C::BK, C::NW>(st, x + (int64_t)n0 * H + kt * C::BK, H, rows, j); },
      [&](int kt, char* st, int j) {
        const bf16_t* b = w_r + (int64_t)kt * C::BK * E;
        moe_mma::dma_mn<C::BN, C::BK, C::NW>(st, b, b, C::BN, E, C::BK, E, j);
      },
      wm, wn);
  constexpr int LP = C::BN + 1;  // odd pitch: the column writes of a wave spread over the banks
  float* lg = reinterpret_cast<float*>(lds);
  float* p = lg + moe_mma::lane_row<C>(wm) * LP + moe_mma::lane_col<C>(wn);
#pragma unroll
  for (int mi = 0; mi < C::FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < C::FN; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) p[moe_mma::frag_row(mi, r) * LP + ni * 32] = acc.a[mi][ni][r];
  __syncthreads();
  if (probs) {  // load-balancing loss: full softmax instead of the top-K
    probs_epilogue<C::NT>(lg, LP, rows, n0, E, bias, probs, part + (int64_t)blockIdx.x * E);
    return;
  }
  // block histogram of the chosen experts, past the logits in LDS
  int* lhist = reinterpret_cast<int*>(lds + C::LDS) - MOE_MAX_EXPERTS;
  if (hist) {
    for (int e = threadIdx.x; e < E; e += C::NT) lhist[e] = 0;
    __syncthreads();
  }
  int* lh = hist ? lhist : nullptr;
  if (E <= 64) {
    for (int tt = threadIdx.x; tt < rows; tt += C::NT) lane_topk_gates(lg + tt * LP, bias, E, K, n0 + tt, topk, gates, lh);
  } else {
    for (int tt = w; tt < rows; tt += C::NW) wave_topk_gates(lg + tt * LP, bias, E, K, n0 + tt, topk, gates, lh);
  }
  if (hist) {
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += C::NT) hist[(int64_t)blockIdx.x * E + e] = lhist[e];
  }
}

// Router for few experts and short rows (bf16, E <= 32, H <= 1024).  The
// workgroup's 32 token rows and the whole of W_r, transposed to [expert][h]
// (experts E..31 zero), come into LDS with all of a thread's loads issued
// before its first store; one wave then multiplies them on the matrix cores
// (one 32 x 32 tile, H / 16 k steps, float32 accumulation) and the epilogue
// is k_route_mma's.  The ring-pipelined router above pads W_r to 128
// columns and waits on each 64-deep stage, which leaves it latency-bound
// when E is small.
constexpr int kSmallRouteE = 32, kSmallRouteH = 1024;
constexpr int kSmallRouteLoads = kRouteTok * kSmallRouteH / 8 / 256;  // 16-byte loads per thread, at most

__host__ __device__ constexpr int small_route_pitch(int H) { return H + 8; }  // bf16 per staged row
__host__ __device__ constexpr size_t small_route_lds(int H) {
  return size_t(2) * 32 * small_route_pitch(H) * 2 + size_t(kRouteTok) * (kSmallRouteE + 1) * 4 +
         size_t(MOE_MAX_EXPERTS) * 4;
}

__global__ __launch_bounds__(256) void k_route_small(const bf16_t* __restrict__ x, const bf16_t* __restrict__ w_r,
                                                     const float* __restrict__ bias, int32_t* __restrict__ topk,
                                                     float* __restrict__ gates, int N, int H, int E, int K,
                                                     float* __restrict__ probs, float* __restrict__ part,
                                                     int32_t* __restrict__ hist) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  using moe_mma::u32x4_t;
  const int P = small_route_pitch(H);
  bf16_t* xl = reinterpret_cast<bf16_t*>(lds);                        // [32][P] token rows
  bf16_t* wl = xl + kRouteTok * P;                                    // [32][P] W_r^T
  constexpr int LP = kSmallRouteE + 1;
  float* lg = reinterpret_cast<float*>(wl + kSmallRouteE * P);        // [32][LP] logits
  int* lhist = reinterpret_cast<int*>(lg + kRouteTok * LP);           // [E]
  const int n0 = blockIdx.x * kRouteTok;
  const int rows = min(kRouteTok, N - n0);
  const int tid = threadIdx.x;
  const int cpr = H / 8;  // 16-byte chunks per token row
  {
    u32x4_t v[kSmallRouteLoads];
#pragma unroll
    for (int i = 0; i < kSmallRouteLoads; ++i) {
      const int q = tid + 256 * i, r = q / cpr;
      v[i] = u32x4_t{0u, 0u, 0u, 0u};
      if (q < kRouteTok * cpr && r < rows)
        v[i] = *reinterpret_cast<const u32x4_t*>(x + (int64_t)(n0 + r) * H + (q % cpr) * 8);
    }
#pragma unroll
    for (int i = 0; i < kSmallRouteLoads; ++i) {
      const int q = tid + 256 * i;
      if (q < kRouteTok * cpr) *reinterpret_cast<u32x4_t*>(xl + (q / cpr) * P + (q % cpr) * 8) = v[i];
    }
  }
  {
    // W_r [H][E]: chunk q holds experts 8 (q % cpe) .. +7 of row h = q / cpe
    const int cpe = E / 8;
    u32x4_t v[kSmallRouteLoads];
#pragma unroll
    for (int i = 0; i < kSmallRouteLoads; ++i) {
      const int q = tid + 256 * i;
      v[i] = u32x4_t{0u, 0u, 0u, 0u};
      if (q < H * cpe) v[i] = *reinterpret_cast<const u32x4_t*>(w_r + (int64_t)q * 8);
    }
#pragma unroll
    for (int i = 0; i < kSmallRouteLoads; ++i) {
      const int q = tid + 256 * i;
      if (q < H * cpe) {
        const int h = q / cpe, e0 = (q % cpe) * 8;
        const bf16_t* b = reinterpret_cast<const bf16_t*>(&v[i]);
#pragma unroll
        for (int j = 0; j < 8; ++j) wl[(e0 + j) * P + h] = b[j];
      }
    }
    for (int q = tid; q < (kSmallRouteE - E) * cpr; q += 256)
      *reinterpret_cast<u32x4_t*>(wl + (E + q / cpr) * P + (q % cpr) * 8) = u32x4_t{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  if (tid < 64) {
    // A = the token rows (lane: row l % 32, k 8 (l / 32) ..), B = W_r^T rows
    // (lane: expert l % 32, same k); C[token][expert] in the 32 x 32 layout
    const bf16_t* ap = xl + (tid & 31) * P + 8 * (tid >> 5);
    const bf16_t* bp = wl + (tid & 31) * P + 8 * (tid >> 5);
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    for (int k = 0; k < H; k += 16)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t*>(ap + k),
                                                    *reinterpret_cast<const bf16x8_t*>(bp + k), acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) lg[((r >> 2) * 8 + (tid >> 5) * 4 + (r & 3)) * LP + (tid & 31)] = acc[r];
  }
  __syncthreads();
  if (probs) {  // load-balancing loss: full softmax instead of the top-K
    probs_epilogue<256>(lg, LP, rows, n0, E, bias, probs, part + (int64_t)blockIdx.x * E);
    return;
  }
  if (hist) {
    for (int e = tid; e < E; e += 256) lhist[e] = 0;
    __syncthreads();
  }
  int* lh = hist ? lhist : nullptr;
  for (int tt = tid; tt < rows; tt += 256) lane_topk_gates(lg + tt * LP, bias, E, K, n0 + tt, topk, gates, lh);
  if (hist) {
    __syncthreads();
    for (int e = tid; e < E; e += 256) hist[(int64_t)blockIdx.x * E + e] = lhist[e];
  }
}

// Router tile shapes (tokens x padded experts): the MN-contiguous W_r tile
// needs at least 128 columns for its swizzle.  32 tokens per workgroup
// (against 64 with two workgroups per CU: 9.1 vs 10.7 us at H = 512, E = 8
// and 53.6 vs 56.6 us at H = 2048, E = 64, N = 16384).  Up to 128 experts:
// four-stage rings, two workgroups per CU (160 KB of LDS), which keeps three
// 64-deep stages in flight per workgroup; router + metadata went from 88 to
// 61 us at N = 16384, H = 4096, E = 8 and from 87 to 74 us at H = 2048,
// E = 64 against two-stage rings with four workgroups per CU (eight stages
// per CU with one workgroup: 88 us).  256 experts: four stages, one
// workgroup per CU (no change against two stages at H = 7168, N = 8192,
// where a timing-only copy without the W_r loads saved 70 of about 230 us
// and one without the x loads 19: the rest is the latency of each 64-deep
// step with one 4-wave workgroup per CU).
using RouteCfg128 = moe_mma::TileCfg<32, 128, 1, 4, 2, 64, 4>;
using RouteCfg256 = moe_mma::TileCfg<32, 256, 1, 4, 1, 64, 4>;
static_assert(RouteCfg128::BM * (RouteCfg128::BN + 1) * 4 + MOE_MAX_EXPERTS * 4 <= RouteCfg128::LDS,
              "logits and the block histogram fit the staging space");
static_assert(RouteCfg256::BM * (RouteCfg256::BN + 1) * 4 + MOE_MAX_EXPERTS * 4 <= RouteCfg256::LDS,
              "logits and the block histogram fit the staging space");
static_assert(RouteCfg128::BM == 32 && RouteCfg256::BM == 32 && kRouteTok == 32,
              "every router path has 32-token blocks (the routing metadata reads their histograms)");

// dlogits, dense [N, E]: one thread per element, plus the load-balancing
// loss term when aux.probs is set.  With planes (bf16 path),
// also the exact three-way bf16 split dl = hi + mid + lo of every element into
// planes [3][n_pad][E] (rows N .. n_pad-1 zero), the B operand of the dW_r
// MFMA kernel: hi = bf16(dl), mid = bf16(dl - hi), lo = bf16(dl - hi - mid);
// each difference is exact in float32 and 3 x 8 significant bits cover the
// 24 of a float32.
// Load-balancing loss term of the backward (all null / zero: no term):
// dl[n,e] += coef * p[n,e] * (counts[e] * inv_nk - s[n]) with coef =
// alpha * (upstream gradient) * E / N and s[n] = sum_i f_i p[n,i].
struct AuxGrad {
  const float* probs;
  const int32_t* counts;
  const float* s;
  float coef, inv_nk;
};

__global__ __launch_bounds__(256) void k_route_bwd_dl(const int32_t* __restrict__ topk, const float* __restrict__ gates,
                                                      const float* __restrict__ dgates, float* __restrict__ dl,
                                                      bf16_t* __restrict__ planes, int N, int n_pad, int E, int K,
                                                      AuxGrad aux) {
  int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)(planes ? n_pad : N) * E;
  if (idx >= total) return;
  int n = int(idx / E), e = int(idx % E);
  float out = 0.f;
  if (n < N) {
    const int32_t* tk = topk + (int64_t)n * K;
    const float* g = gates + (int64_t)n * K;
    const float* dg = dgates + (int64_t)n * K;
    float s = 0.f;
    for (int k = 0; k < K; ++k) s = fmaf(g[k], dg[k], s);
    for (int k = 0; k < K; ++k)
      if (tk[k] == e) out = g[k] * (dg[k] - s);
    if (aux.probs) out += aux.coef * aux.probs[idx] * (float(aux.counts[e]) * aux.inv_nk - aux.s[n]);
    dl[idx] = out;
  }
  if (planes) {
    const bf16_t hi = f32_to_bf16(out);
    const float r1 = out - bf16_to_f32(hi);
    const bf16_t mid = f32_to_bf16(r1);
    const bf16_t lo = f32_to_bf16(r1 - bf16_to_f32(mid));
    const int64_t plane = (int64_t)n_pad * E;
    planes[idx] = hi;
    planes[plane + idx] = mid;
    planes[2 * plane + idx] = lo;
  }
}

// Partial dW_r on the matrix cores (bf16 path, E a multiple of 8): workgroup
// (h tile, expert tile, chunk c) computes part[c][h][e] = sum over the chunk's
// tokens n of x[n,h] (hi + mid + lo)[n,e], a contraction over 3 x chunk
// steps: the hi plane over the chunk's tokens in ascending order, then mid,
// then lo.  Both operands are MN-contiguous tiles; chunks are multiples of
// 64 tokens and rows past N are zero in the planes (x rows there read a
// clamped valid row and are multiplied by zero).
template <class C>
__global__ __launch_bounds__(C::NT, C::MINB) void k_route_dwr_mma(const bf16_t* __restrict__ x,
                                                                 const bf16_t* __restrict__ planes,
                                                                 float* __restrict__ part, int N, int n_pad, int H,
                                                                 int E, int chunk) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int h0 = blockIdx.x * C::BM, e0 = blockIdx.y * C::BN, c = blockIdx.z;
  const int nb = c * chunk;
  const int nks = min(chunk, n_pad - nb) / C::BK;  // steps per plane
  const int w = threadIdx.x >> 6, wm = w / C::WN, wn = w % C::WN;
  const int64_t plane = (int64_t)n_pad * E;
  moe_mma::Acc<C> acc;
  moe_mma::k_loop<C, true, true>(
      lds, acc, 3 * nks,
      [&](int kt, char* st, int j) {
        const int n = nb + (kt % nks) * C::BK;
        const bf16_t* a = x + (int64_t)n * H + h0;
        moe_mma::dma_mn<C::BM, C::BK, C::NW>(st, a, a, C::BM, H, N - n, C::BM, j);
      },
      [&](int kt, char* st, int j) {
        const int n = nb + (kt % nks) * C::BK;
        const bf16_t* b = planes + (kt / nks) * plane + (int64_t)n * E + e0;
        moe_mma::dma_mn<C::BN, C::BK, C::NW>(st, b, b, C::BN, E, C::BK, E - e0, j);
      },
      wm, wn);
  const int lr = moe_mma::lane_row<C>(wm), lc = moe_mma::lane_col<C>(wn);
  float* o = part + (int64_t)c * H * E + (int64_t)(h0 + lr) * E + e0 + lc;
#pragma unroll
  for (int mi = 0; mi < C::FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < C::FN; ++ni)
      if (e0 + lc + ni * 32 < E)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[(int64_t)moe_mma::frag_row(mi, r) * E + ni * 32] = acc.a[mi][ni][r];
}

using DwrCfg128 = moe_mma::TileCfg<128, 128, 2, 2, 2, 64, 2>;

constexpr int kRbTok = 128;  // tokens staged in LDS at a time by the dW_r partial kernel

// Partial dW_r of one chunk of tokens and HB hidden units:
// part[c][e][h] = sum_{n in chunk} x[n,h] dl[n,e], sparse in e (only the K
// selected experts of a token contribute) unless DENSE (the load-balancing
// loss gives every logit a gradient: all E experts, ascending, dl read
// straight from its [N, E] rows).  kRbTok tokens at a time, the x slice,
// expert ids and dlogits values are first staged in LDS with independent
// loads; then each thread accumulates its h over the tokens in ascending
// order.
template <typename T, int HB, bool DENSE>
__global__ __launch_bounds__(HB) void k_route_bwd_partial(const T* __restrict__ x, const int32_t* __restrict__ topk,
                                                          const float* __restrict__ dl, float* __restrict__ part,
                                                          int N, int H, int E, int K, int chunk) {
  extern __shared__ float smem[];
  float* acc = smem;                                              // [E][HB]
  float* xs = acc + E * HB;                                       // [kRbTok][HB]
  int* s_e = reinterpret_cast<int*>(xs + kRbTok * HB);            // [kRbTok*K]
  float* s_d = reinterpret_cast<float*>(s_e + kRbTok * K);        // [kRbTok*K]
  const int t = threadIdx.x;
  const int h0 = blockIdx.x * HB;
  const int c = blockIdx.y;
  const int nb = c * chunk, ne = min(N, nb + chunk);
  constexpr int V = Vec16<T>::n;
  constexpr int VPR = HB / V;  // 16-byte vectors per token row of the slice
  for (int e = 0; e < E; ++e) acc[e * HB + t] = 0.f;
  for (int s0 = nb; s0 < ne; s0 += kRbTok) {
    const int nt = min(kRbTok, ne - s0);
    __syncthreads();
    for (int i = t; i < nt * VPR; i += HB) {
      const int tt = i / VPR, v = i % VPR;
      float val[V];
      Vec16<T>::load(x + (int64_t)(s0 + tt) * H + h0 + v * V, val);
#pragma unroll
      for (int q = 0; q < V; ++q) xs[tt * HB + v * V + q] = val[q];
    }
    if (!DENSE)
      for (int i = t; i < nt * K; i += HB) {
        const int64_t f = (int64_t)s0 * K + i;
        const int e = topk[f];
        s_e[i] = e;
        s_d[i] = dl[(f / K) * E + e];
      }
    __syncthreads();
    for (int n = 0; n < nt; ++n) {
      const float xv = xs[n * HB + t];
      if (DENSE) {
        const float* dn = dl + (int64_t)(s0 + n) * E;
        for (int e = 0; e < E; ++e) acc[e * HB + t] = fmaf(xv, dn[e], acc[e * HB + t]);
      } else {
        for (int k = 0; k < K; ++k) {
          const int e = s_e[n * K + k];
          acc[e * HB + t] = fmaf(xv, s_d[n * K + k], acc[e * HB + t]);
        }
      }
    }
  }
  float* out = part + (int64_t)c * E * H;
  for (int e = 0; e < E; ++e) out[(int64_t)e * H + h0 + t] = acc[e * HB + t];
}

// dW_r[h, e] = sum of part[c][e][h] over chunks c: 8 lanes per output each
// sum a fixed stride-8 subset of the chunks in ascending order, then a fixed
// butterfly adds the 8 partial sums.
__global__ __launch_bounds__(256) void k_route_bwd_reduce(const float* __restrict__ part, float* __restrict__ dw_r,
                                                          int H, int E, int nchunks) {
  const int64_t o = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 3;
  const int j = threadIdx.x & 7;
  float sum = 0.f;
  if (o < (int64_t)E * H)
    for (int c = j; c < nchunks; c += 8) sum += part[(int64_t)c * E * H + o];
  sum += __shfl_xor(sum, 1, kWave);
  sum += __shfl_xor(sum, 2, kWave);
  sum += __shfl_xor(sum, 4, kWave);
  if (j == 0 && o < (int64_t)E * H) {
    const int e = int(o / H), h = int(o % H);
    dw_r[(int64_t)h * E + e] = sum;
  }
}

template <typename T, int EPT>
hipError_t launch_route_t(const moe_launch::Dims& d, const void* x, const void* w_r, const float* bias, int32_t* topk,
                          float* gates, hipStream_t s, float* probs, float* part, int32_t* hist) {
  constexpr int EP = 8 * EPT;
  constexpr int HC = route_hc<EPT>();
  constexpr size_t stage = HC * kRouteTok + HC * EP, logits = kRouteTok * (EP + 1);
  size_t lds = sizeof(float) * (stage > logits ? stage : logits) + sizeof(int) * MOE_MAX_EXPERTS;
  int grid = int((d.N + kRouteTok - 1) / kRouteTok);
  hipLaunchKernelGGL((k_route<T, EPT>), dim3(grid), dim3(256), lds, s, static_cast<const T*>(x),
                     static_cast<const T*>(w_r), bias, topk, gates, int(d.N), int(d.H), int(d.E), int(d.K), probs,
                     part, hist);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_route(const moe_launch::Dims& d, const void* x, const void* w_r, const float* bias, int32_t* topk,
                        float* gates, hipStream_t s, float* probs = nullptr, float* part = nullptr,
                        int32_t* hist = nullptr) {
  if (d.E <= 8) return launch_route_t<T, 1>(d, x, w_r, bias, topk, gates, s, probs, part, hist);
  if (d.E <= 16) return launch_route_t<T, 2>(d, x, w_r, bias, topk, gates, s, probs, part, hist);
  if (d.E <= 32) return launch_route_t<T, 4>(d, x, w_r, bias, topk, gates, s, probs, part, hist);
  if (d.E <= 64) return launch_route_t<T, 8>(d, x, w_r, bias, topk, gates, s, probs, part, hist);
  if (d.E <= 128) return launch_route_t<T, 16>(d, x, w_r, bias, topk, gates, s, probs, part, hist);
  return launch_route_t<T, 32>(d, x, w_r, bias, topk, gates, s, probs, part, hist);
}

// Load-balancing loss value: P_e = (sum of the block partials) / N, f_e =
// counts_e / (N K), loss = alpha * E * sum_e f_e P_e.  One workgroup: thread
// t sums the partials of expert t % E over blocks j, j + J, j + 2J, ... (j =
// t / E, J = 256 / E groups; eight independent loads in flight, added in a
// fixed order), the J group sums of each expert are added in ascending j,
// and the E terms by a fixed tree.  The result does not depend on timing.
__global__ __launch_bounds__(256) void k_aux_reduce(const float* __restrict__ part, int nblk,
                                                    const int32_t* __restrict__ counts, int N, int E, int K,
                                                    float alpha, float* __restrict__ loss) {
  __shared__ float g[256];
  __shared__ float t[256];
  const int tid = threadIdx.x;
  const int J = 256 / E;  // groups per expert (E <= 256)
  const int e = tid % E, j = tid / E;
  float acc = 0.f;
  if (j < J) {
    int b = j;
    for (; b + 7 * J < nblk; b += 8 * J) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = part[(int64_t)(b + i * J) * E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += v[i];
    }
    for (; b < nblk; b += J) acc += part[(int64_t)b * E + e];
  }
  g[tid] = acc;
  __syncthreads();
  float term = 0.f;
  if (tid < E) {
    float P = 0.f;
    for (int q = 0; q < J; ++q) P += g[q * E + tid];
    term = (float(counts[tid]) / (float(N) * float(K))) * (P / float(N));
  }
  t[tid] = term;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) t[tid] += t[tid + off];
    __syncthreads();
  }
  if (tid == 0) *loss = alpha * float(E) * t[0];
}

// s[n] = sum_i f_i p[n,i] with f_i = counts_i / (N K), experts ascending.
__global__ __launch_bounds__(256) void k_aux_s(const float* __restrict__ probs, const int32_t* __restrict__ counts,
                                               float* __restrict__ s, int N, int E, float inv_nk) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  float acc = 0.f;
  for (int e = 0; e < E; ++e) acc = fmaf(float(counts[e]) * inv_nk, probs[n * E + e], acc);
  s[n] = acc;
}

}  // namespace

namespace moe_launch {

template <class C>
hipError_t route_mma(const Dims& d, const void* x, const void* w_r, const float* bias, int32_t* topk, float* gates,
                     hipStream_t s, float* probs = nullptr, float* part = nullptr, int32_t* hist = nullptr) {
  hipError_t st = moe_mma::allow_lds<k_route_mma<C>>(C::LDS);
  if (st != hipSuccess) return st;
  const unsigned grid = unsigned((d.N + C::BM - 1) / C::BM);
  hipLaunchKernelGGL(k_route_mma<C>, dim3(grid), dim3(C::NT), C::LDS, s, static_cast<const moe::bf16_t*>(x),
                     static_cast<const moe::bf16_t*>(w_r), bias, topk, gates, int(d.N), int(d.H), int(d.E), int(d.K),
                     probs, part, hist);
  return hipGetLastError();
}

// The matrix-core paths of the router need 16-byte W_r rows (bf16, E % 8 == 0).
static bool router_mma(const Dims& d) { return d.dtype == MOE_BF16 && d.E % 8 == 0; }
// ... and the LDS-resident form takes few experts and short rows.
static bool router_small(const Dims& d) {
  return router_mma(d) && d.E <= kSmallRouteE && d.H <= kSmallRouteH;
}

static hipError_t route_small(const Dims& d, const void* x, const void* w_r, const float* bias, int32_t* topk,
                              float* gates, hipStream_t s, float* probs = nullptr, float* part = nullptr,
                              int32_t* hist = nullptr) {
  const size_t lds = small_route_lds(int(d.H));
  hipError_t st = moe_mma::allow_lds<k_route_small>(int(small_route_lds(kSmallRouteH)));
  if (st != hipSuccess) return st;
  const unsigned grid = unsigned((d.N + kRouteTok - 1) / kRouteTok);
  hipLaunchKernelGGL(k_route_small, dim3(grid), dim3(256), lds, s, static_cast<const moe::bf16_t*>(x),
                     static_cast<const moe::bf16_t*>(w_r), bias, topk, gates, int(d.N), int(d.H), int(d.E), int(d.K),
                     probs, part, hist);
  return hipGetLastError();
}

hipError_t route(const Dims& d, const void* x, const void* w_r, const float* bias, int32_t* topk, float* gates,
                 hipStream_t s, int32_t* hist) {
  if (router_small(d)) return route_small(d, x, w_r, bias, topk, gates, s, nullptr, nullptr, hist);
  if (router_mma(d))
    return d.E <= 128 ? route_mma<RouteCfg128>(d, x, w_r, bias, topk, gates, s, nullptr, nullptr, hist)
                      : route_mma<RouteCfg256>(d, x, w_r, bias, topk, gates, s, nullptr, nullptr, hist);
  if (d.dtype == MOE_BF16) return launch_route<moe::bf16_t>(d, x, w_r, bias, topk, gates, s, nullptr, nullptr, hist);
  return launch_route<float>(d, x, w_r, bias, topk, gates, s, nullptr, nullptr, hist);
}

// Token chunks of the dW_r partial sums: one per kRbTok tokens, fewer when
// the partials (chunks * E * H floats) would exceed 16 MiB.
size_t route_bwd_chunks(const Dims& d) {
  int64_t c = (d.N + kRbTok - 1) / kRbTok;
  const int64_t cap = (int64_t(16) << 20) / (4 * d.E * d.H);
  if (c > cap) c = cap;
  if (c < 1) c = 1;
  return size_t(c);
}

// Matrix-core dW_r: chunks of a multiple of 64 tokens over n_pad = N rounded
// up to 64; the workspace holds the chunk partials, then the bf16 planes.
struct DwrPlan {
  int64_t n_pad, chunk, nch;
  size_t part_bytes, plane_bytes;
};
static DwrPlan dwr_plan(const Dims& d) {
  DwrPlan p;
  p.n_pad = (d.N + 63) / 64 * 64;
  const int64_t target = int64_t(route_bwd_chunks(d));
  p.chunk = ((d.N + target - 1) / target + 63) / 64 * 64;
  p.nch = (p.n_pad + p.chunk - 1) / p.chunk;
  p.part_bytes = (size_t(p.nch) * d.H * d.E * sizeof(float) + 255) / 256 * 256;
  p.plane_bytes = size_t(3) * p.n_pad * d.E * sizeof(moe::bf16_t);
  return p;
}

size_t route_bwd_ws(const Dims& d) {
  const size_t vec = route_bwd_chunks(d) * size_t(d.E) * size_t(d.H) * sizeof(float);
  if (!router_mma(d)) return vec;
  const DwrPlan p = dwr_plan(d);
  return p.part_bytes + p.plane_bytes;
}

// dW_r[h, e] = sum over chunks c of part[c][h][e] (same index as dW_r):
// 8 lanes per output each sum a fixed stride-8 subset of the chunks in
// ascending order, then a fixed butterfly adds the 8 partial sums.
__global__ __launch_bounds__(256) void k_route_dwr_reduce(const float* __restrict__ part, float* __restrict__ dw_r,
                                                          int64_t total, int nchunks) {
  const int64_t o = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 3;
  const int j = threadIdx.x & 7;
  float sum = 0.f;
  if (o < total)
    for (int c = j; c < nchunks; c += 8) sum += part[(int64_t)c * total + o];
  sum += __shfl_xor(sum, 1, moe::kWave);
  sum += __shfl_xor(sum, 2, moe::kWave);
  sum += __shfl_xor(sum, 4, moe::kWave);
  if (j == 0 && o < total) dw_r[o] = sum;
}

hipError_t route_bwd_mma(const Dims& d, const void* x, const int32_t* topk, const float* gates, const float* dgates,
                         float* dlogits, float* dw_r, void* ws, hipStream_t s, AuxGrad aux) {
  using C = DwrCfg128;
  const DwrPlan p = dwr_plan(d);
  float* part = static_cast<float*>(ws);
  moe::bf16_t* planes = reinterpret_cast<moe::bf16_t*>(static_cast<char*>(ws) + p.part_bytes);
  const int64_t ne = p.n_pad * d.E;
  hipLaunchKernelGGL(k_route_bwd_dl, dim3(unsigned((ne + 255) / 256)), dim3(256), 0, s, topk, gates, dgates, dlogits,
                     planes, int(d.N), int(p.n_pad), int(d.E), int(d.K), aux);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  err = moe_mma::allow_lds<k_route_dwr_mma<C>>(C::LDS);
  if (err != hipSuccess) return err;
  dim3 grid(unsigned(d.H / C::BM), unsigned((d.E + C::BN - 1) / C::BN), unsigned(p.nch));
  hipLaunchKernelGGL(k_route_dwr_mma<C>, grid, dim3(C::NT), C::LDS, s, static_cast<const moe::bf16_t*>(x), planes,
                     part, int(d.N), int(p.n_pad), int(d.H), int(d.E), int(p.chunk));
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t total = d.H * d.E;
  hipLaunchKernelGGL(k_route_dwr_reduce, dim3(unsigned((total * 8 + 255) / 256)), dim3(256), 0, s, part, dw_r, total,
                     int(p.nch));
  return hipGetLastError();
}

static hipError_t route_bwd_impl(const Dims& d, const void* x, const int32_t* topk, const float* gates,
                                 const float* dgates, float* dlogits, float* dw_r, void* ws, hipStream_t s,
                                 AuxGrad aux) {
  if (router_mma(d)) return route_bwd_mma(d, x, topk, gates, dgates, dlogits, dw_r, ws, s, aux);
  int64_t ne = d.N * d.E;
  hipLaunchKernelGGL(k_route_bwd_dl, dim3(unsigned((ne + 255) / 256)), dim3(256), 0, s, topk, gates, dgates, dlogits,
                     nullptr, int(d.N), int(d.N), int(d.E), int(d.K), aux);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int nch = int(route_bwd_chunks(d));
  const int chunk = int((d.N + nch - 1) / nch);
  float* part = static_cast<float*>(ws);
  // LDS: E*HB + kRbTok*HB + 2*kRbTok*K floats <= 64 KiB
  auto partial = [&](auto hb, auto dense) {
    constexpr int HB = decltype(hb)::value;
    constexpr bool DENSE = decltype(dense)::value;
    const size_t lds = sizeof(float) * (size_t(d.E) * HB + size_t(kRbTok) * HB + 2 * size_t(kRbTok) * d.K);
    const dim3 grid(unsigned(d.H / HB), unsigned(nch));
    if (d.dtype == MOE_BF16)
      hipLaunchKernelGGL((k_route_bwd_partial<moe::bf16_t, HB, DENSE>), grid, dim3(HB), lds, s,
                         static_cast<const moe::bf16_t*>(x), topk, dlogits, part, int(d.N), int(d.H), int(d.E),
                         int(d.K), chunk);
    else
      hipLaunchKernelGGL((k_route_bwd_partial<float, HB, DENSE>), grid, dim3(HB), lds, s,
                         static_cast<const float*>(x), topk, dlogits, part, int(d.N), int(d.H), int(d.E), int(d.K),
                         chunk);
  };
  using Dense = std::true_type;
  using Sparse = std::false_type;
  const bool dense = aux.probs != nullptr;
  if (d.E <= 64) {
    using HB = std::integral_constant<int, 64>;
    dense ? partial(HB{}, Dense{}) : partial(HB{}, Sparse{});
  } else {
    using HB = std::integral_constant<int, 32>;
    dense ? partial(HB{}, Dense{}) : partial(HB{}, Sparse{});
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t nthreads = d.E * d.H * 8;
  hipLaunchKernelGGL(k_route_bwd_reduce, dim3(unsigned((nthreads + 255) / 256)), dim3(256), 0, s, part, dw_r,
                     int(d.H), int(d.E), nch);
  return hipGetLastError();
}

hipError_t route_bwd(const Dims& d, const void* x, const int32_t* topk, const float* gates, const float* dgates,
                     float* dlogits, float* dw_r, void* ws, hipStream_t s) {
  return route_bwd_impl(d, x, topk, gates, dgates, dlogits, dw_r, ws, s, AuxGrad{nullptr, nullptr, nullptr, 0.f, 0.f});
}

// ---- load-balancing loss

// Token blocks of the probability pass (the router kernel's token tile).
static int64_t probs_blocks(const Dims& d) {
  const int64_t bm = router_mma(d) ? (d.E <= 128 ? RouteCfg128::BM : RouteCfg256::BM) : kRouteTok;
  return (d.N + bm - 1) / bm;
}

size_t aux_loss_ws(const Dims& d) { return size_t(probs_blocks(d)) * size_t(d.E) * sizeof(float); }

hipError_t aux_loss(const Dims& d, const void* x, const void* w_r, const float* bias, const int32_t* counts,
                    float alpha, float* probs, float* loss, void* ws, hipStream_t s) {
  float* part = static_cast<float*>(ws);
  hipError_t err;
  if (router_small(d))
    err = route_small(d, x, w_r, bias, nullptr, nullptr, s, probs, part);
  else if (router_mma(d))
    err = d.E <= 128 ? route_mma<RouteCfg128>(d, x, w_r, bias, nullptr, nullptr, s, probs, part)
                     : route_mma<RouteCfg256>(d, x, w_r, bias, nullptr, nullptr, s, probs, part);
  else if (d.dtype == MOE_BF16)
    err = launch_route<moe::bf16_t>(d, x, w_r, bias, nullptr, nullptr, s, probs, part);
  else
    err = launch_route<float>(d, x, w_r, bias, nullptr, nullptr, s, probs, part);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_aux_reduce, dim3(1), dim3(256), 0, s, part, int(probs_blocks(d)), counts, int(d.N),
                     int(d.E), int(d.K), alpha, loss);
  return hipGetLastError();
}

// route_bwd's workspace, then s[N] of the aux term.
static size_t route_bwd_ws_aligned(const Dims& d) { return (route_bwd_ws(d) + 255) / 256 * 256; }
size_t route_bwd_aux_ws(const Dims& d) { return route_bwd_ws_aligned(d) + size_t(d.N) * sizeof(float); }

hipError_t route_bwd_aux(const Dims& d, const void* x, const int32_t* topk, const float* gates, const float* dgates,
                         const float* probs, const int32_t* counts, float aux_scale, float* dlogits, float* dw_r,
                         void* ws, hipStream_t s) {
  float* sn = reinterpret_cast<float*>(static_cast<char*>(ws) + route_bwd_ws_aligned(d));
  const float inv_nk = 1.0f / (float(d.N) * float(d.K));
  hipLaunchKernelGGL(k_aux_s, dim3(unsigned((d.N + 255) / 256)), dim3(256), 0, s, probs, counts, sn, int(d.N),
                     int(d.E), inv_nk);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const AuxGrad aux{probs, counts, sn, aux_scale * float(d.E) / float(d.N), inv_nk};
  return route_bwd_impl(d, x, topk, gates, dgates, dlogits, dw_r, ws, s, aux);
}

}  // namespace moe_launch
