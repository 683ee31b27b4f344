// Row movement of the MoE layer: the permuting gather, the gate-weighted
// combine, their backward passes, and the router's input-gradient term.
//
// "MegaBlocks - architecture and principles", section 2.1: tokens are
// gathered into expert-grouped order before the expert MLP and scattered back
// with a multiplication by the routing weight and a sum over the top-k after
// it; section 4: the backward of the gather is an (unweighted) scatter and
// vice versa.  Here every output row has exactly one owner: the combine and
// the gather backward read the K rows of a token through inv[] (a gather-sum
// in ascending k) instead of scattering with atomics, so results are bitwise
// reproducible.  All rows move in 16-byte vectors; a row is H elements.
#include <type_traits>

#include "common.h"

namespace {
using namespace moe;

// xs[i] = x[sorted_flat[i] / K], one 16-byte vector per thread, grid-stride;
// dropped rows (sorted_flat < 0, capacity) are skipped.  A per-row form (one
// wave per 2-4 rows, each row's index read once, 32-bit offsets within the
// row, every load of a pass before its stores) measured the same: 80.9 vs
// 79.6 us at N = 16384, K = 2, H = 4096 and 11.5 vs 11.4 us at H = 512, so
// the divide and the index re-reads (L1 hits) are not what bounds this copy.
template <typename T>
__global__ __launch_bounds__(256) void k_permute(const T* __restrict__ x, const int32_t* __restrict__ sorted_flat,
                                                 T* __restrict__ xs, int64_t total_vec, int vpr, int K) {
  constexpr int V = Vec16<T>::n;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < total_vec; v += stride) {
    int64_t row = v / vpr;
    int c = int(v - row * vpr);
    const int32_t f = sorted_flat[row];
    if (f < 0) continue;  // dropped row (capacity): never read
    int64_t tok = f / K;
    const uint4* src = reinterpret_cast<const uint4*>(x + (tok * vpr + c) * V);
    uint4* dst = reinterpret_cast<uint4*>(xs + v * V);
    *dst = *src;
  }
}

// Tokens per wave: two while the row registers of both fit (K <= 4), else one.
__host__ __device__ constexpr int tok_per_wave(int K) { return K <= 4 ? 2 : 1; }

// y[n] = sum_k gates[n,k] * ys[inv[n*K+k]], k ascending, float32 accumulation;
// dropped slots (inv < 0) add nothing.  add (optional, [N,H]): a row added
// with weight 1 after the K terms (the shared expert's output).  One wave per
// tok_per_wave(K) tokens; each lane takes U row vectors at a time (64 apart)
// and issues every row load of them before the first multiply; KT = K.
template <typename T, int KT, int U>
__global__ __launch_bounds__(256) void k_combine(const T* __restrict__ ys, const float* __restrict__ gates,
                                                 const int32_t* __restrict__ inv, const T* __restrict__ add,
                                                 T* __restrict__ y, int N, int vpr) {
  constexpr int V = Vec16<T>::n;
  constexpr int TW = tok_per_wave(KT);
  const int lane = lane_id();
  const int nbase = (blockIdx.x * 4 + (threadIdx.x >> 6)) * TW;
  if (nbase >= N) return;  // uniform across the wave
  int32_t r[TW][KT];
  float g[TW][KT];
  bool valid[TW];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const int n = nbase + t;
    valid[t] = n < N;
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      r[t][k] = valid[t] ? inv[n * KT + k] : -1;
      g[t][k] = valid[t] ? gates[n * KT + k] : 0.f;
    }
  }
  const uint4* ys4 = reinterpret_cast<const uint4*>(ys);
  const uint4* add4 = reinterpret_cast<const uint4*>(add);
  for (int c0 = lane; c0 < vpr; c0 += kWave * U) {
    uint4 raw[U][TW][KT], ra[U][TW];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave;
      if (c >= vpr) break;
#pragma unroll
      for (int t = 0; t < TW; ++t) {
#pragma unroll
        for (int k = 0; k < KT; ++k)
          if (r[t][k] >= 0) raw[u][t][k] = ys4[(int64_t)r[t][k] * vpr + c];
        if (add != nullptr && valid[t]) ra[u][t] = add4[(int64_t)(nbase + t) * vpr + c];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave;
      if (c >= vpr) break;
#pragma unroll
      for (int t = 0; t < TW; ++t) {
        if (!valid[t]) continue;
        float acc[V];
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = 0.f;
#pragma unroll
        for (int k = 0; k < KT; ++k)
          if (r[t][k] >= 0) {
            float val[V];
            Vec16<T>::load(reinterpret_cast<const T*>(&raw[u][t][k]), val);
#pragma unroll
            for (int i = 0; i < V; ++i) acc[i] = fmaf(g[t][k], val[i], acc[i]);
          }
        if (add != nullptr) {
          float val[V];
          Vec16<T>::load(reinterpret_cast<const T*>(&ra[u][t]), val);
#pragma unroll
          for (int i = 0; i < V; ++i) acc[i] += val[i];
        }
        Vec16<T>::store(y + ((int64_t)(nbase + t) * vpr + c) * V, acc);
      }
    }
  }
}

// dys[inv[n,k]] = gates[n,k] dy[n]; dgates[n,k] = <dy[n], ys[inv[n,k]]>
// (fixed lane order, then a butterfly), dropped slots skipped.  Same wave and
// chunk layout as k_combine.
template <typename T, int KT, int U>
__global__ __launch_bounds__(256) void k_combine_bwd(const T* __restrict__ dy, const T* __restrict__ ys,
                                                     const float* __restrict__ gates, const int32_t* __restrict__ inv,
                                                     T* __restrict__ dys, float* __restrict__ dgates, int N, int vpr) {
  constexpr int V = Vec16<T>::n;
  constexpr int TW = tok_per_wave(KT);
  const int lane = lane_id();
  const int nbase = (blockIdx.x * 4 + (threadIdx.x >> 6)) * TW;
  if (nbase >= N) return;  // uniform across the wave
  int32_t r[TW][KT];
  float g[TW][KT];
  bool valid[TW];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const int n = nbase + t;
    valid[t] = n < N;
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      r[t][k] = valid[t] ? inv[n * KT + k] : -1;
      g[t][k] = valid[t] ? gates[n * KT + k] : 0.f;
    }
  }
  float dot[TW][KT];
#pragma unroll
  for (int t = 0; t < TW; ++t)
#pragma unroll
    for (int k = 0; k < KT; ++k) dot[t][k] = 0.f;
  const uint4* dy4 = reinterpret_cast<const uint4*>(dy);
  const uint4* ys4 = reinterpret_cast<const uint4*>(ys);
  for (int c0 = lane; c0 < vpr; c0 += kWave * U) {
    uint4 rd[U][TW], raw[U][TW][KT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave;
      if (c >= vpr) break;
#pragma unroll
      for (int t = 0; t < TW; ++t) {
        if (valid[t]) rd[u][t] = dy4[(int64_t)(nbase + t) * vpr + c];
#pragma unroll
        for (int k = 0; k < KT; ++k)
          if (r[t][k] >= 0) raw[u][t][k] = ys4[(int64_t)r[t][k] * vpr + c];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave;
      if (c >= vpr) break;
#pragma unroll
      for (int t = 0; t < TW; ++t) {
        if (!valid[t]) continue;
        float d[V];
        Vec16<T>::load(reinterpret_cast<const T*>(&rd[u][t]), d);
#pragma unroll
        for (int k = 0; k < KT; ++k) {
          if (r[t][k] < 0) continue;
          float yv[V], o[V];
          Vec16<T>::load(reinterpret_cast<const T*>(&raw[u][t][k]), yv);
          float sdot = dot[t][k];
#pragma unroll
          for (int i = 0; i < V; ++i) {
            sdot = fmaf(d[i], yv[i], sdot);
            o[i] = g[t][k] * d[i];
          }
          dot[t][k] = sdot;
          Vec16<T>::store(dys + ((int64_t)r[t][k] * vpr + c) * V, o);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    if (!valid[t]) continue;  // uniform across the wave
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      const float sum = wave_sum(dot[t][k]);
      if (lane == 0) dgates[(nbase + t) * KT + k] = sum;
    }
  }
}

// W_r [H, E] -> W_r^T [E, H] so the router term of dx reads whole rows.
template <typename T>
__global__ __launch_bounds__(256) void k_transpose_wr(const T* __restrict__ w_r, T* __restrict__ w_rt, int H, int E) {
  int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)H * E) return;
  int e = int(idx / H), h = int(idx % H);
  w_rt[idx] = w_r[(int64_t)h * E + e];
}

// dx[n] = sum_k dxs[inv[n*K+k]] (kept slots, k ascending) + the router
// term sum_k dlogits[n,e_k] * W_r^T[e_k] (k ascending; dlogits of a dropped
// slot is not zero: its gate still takes part in the softmax), float32, one
// rounding.  DENSE: the router term runs over all E experts in ascending
// order (dlogits is dense when the load-balancing loss is on; used for
// E <= 8).  add (optional): one more row added last.  One wave per
// tok_per_wave(K) tokens; each lane takes U row vectors at a time with every
// row load of them issued together; KT = K.
template <typename T, bool DENSE, int KT, int U>
__global__ __launch_bounds__(256) void k_permute_bwd(const T* __restrict__ dxs, const int32_t* __restrict__ inv,
                                                     const int32_t* __restrict__ topk, const float* __restrict__ dl,
                                                     const T* __restrict__ w_rt, const T* __restrict__ add,
                                                     T* __restrict__ dx, int N, int vpr, int E) {
  constexpr int V = Vec16<T>::n;
  constexpr int TW = tok_per_wave(KT);
  const int lane = lane_id();
  const int nbase = (blockIdx.x * 4 + (threadIdx.x >> 6)) * TW;
  if (nbase >= N) return;  // uniform across the wave
  int32_t r[TW][KT], ex[TW][KT];
  float dk[TW][KT];
  bool valid[TW];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const int n = nbase + t;
    valid[t] = n < N;
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      r[t][k] = valid[t] ? inv[n * KT + k] : -1;
      ex[t][k] = valid[t] ? topk[n * KT + k] : 0;
      dk[t][k] = (!DENSE && valid[t]) ? dl[(int64_t)n * E + ex[t][k]] : 0.f;
    }
  }
  const uint4* xs4 = reinterpret_cast<const uint4*>(dxs);
  const uint4* wr4 = reinterpret_cast<const uint4*>(w_rt);
  const uint4* add4 = reinterpret_cast<const uint4*>(add);
  for (int c0 = lane; c0 < vpr; c0 += kWave * U) {
    uint4 rx[U][TW][KT], rw[U][TW][KT], ra[U][TW];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave;
      if (c >= vpr) break;
#pragma unroll
      for (int t = 0; t < TW; ++t) {
#pragma unroll
        for (int k = 0; k < KT; ++k) {
          if (r[t][k] >= 0) rx[u][t][k] = xs4[(int64_t)r[t][k] * vpr + c];
          if (!DENSE && valid[t]) rw[u][t][k] = wr4[(int64_t)ex[t][k] * vpr + c];
        }
        if (add != nullptr && valid[t]) ra[u][t] = add4[(int64_t)(nbase + t) * vpr + c];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave;
      if (c >= vpr) break;
      float acc[TW][V];
#pragma unroll
      for (int t = 0; t < TW; ++t) {
#pragma unroll
        for (int i = 0; i < V; ++i) acc[t][i] = 0.f;
#pragma unroll
        for (int k = 0; k < KT; ++k)
          if (r[t][k] >= 0) {
            float val[V];
            Vec16<T>::load(reinterpret_cast<const T*>(&rx[u][t][k]), val);
#pragma unroll
            for (int i = 0; i < V; ++i) acc[t][i] += val[i];
          }
        if (!DENSE) {
#pragma unroll
          for (int k = 0; k < KT; ++k) {
            float wv[V];
            Vec16<T>::load(reinterpret_cast<const T*>(&rw[u][t][k]), wv);
#pragma unroll
            for (int i = 0; i < V; ++i) acc[t][i] = fmaf(dk[t][k], wv[i], acc[t][i]);
          }
        }
      }
      if (DENSE) {
        // every router logit has a gradient: all E experts, ascending; each
        // W_r^T vector serves the wave's tokens
        for (int e = 0; e < E; ++e) {
          const uint4 raw = wr4[(int64_t)e * vpr + c];
          float wv[V];
          Vec16<T>::load(reinterpret_cast<const T*>(&raw), wv);
#pragma unroll
          for (int t = 0; t < TW; ++t) {
            const float de = valid[t] ? dl[(int64_t)(nbase + t) * E + e] : 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) acc[t][i] = fmaf(de, wv[i], acc[t][i]);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < TW; ++t) {
        if (!valid[t]) continue;
        if (add != nullptr) {
          float val[V];
          Vec16<T>::load(reinterpret_cast<const T*>(&ra[u][t]), val);
#pragma unroll
          for (int i = 0; i < V; ++i) acc[t][i] += val[i];
        }
        Vec16<T>::store(dx + ((int64_t)(nbase + t) * vpr + c) * V, acc[t]);
      }
    }
  }
}

// Dense router term (load-balancing loss on) for many experts: one wave per
// kTokTile tokens, so each W_r^T vector read serves all of them; the tile's
// dlogits rows are staged in LDS (the wave's own slice, read back as
// broadcasts).  Per output element the same order as k_permute_bwd<T, true>:
// dxs rows in ascending k, then dl * W_r^T over ascending e.
constexpr int kTokTile = 8;
template <typename T>
__global__ __launch_bounds__(256) void k_permute_bwd_dense_tiled(const T* __restrict__ dxs,
                                                                 const int32_t* __restrict__ inv,
                                                                 const float* __restrict__ dl,
                                                                 const T* __restrict__ w_rt,
                                                                 const T* __restrict__ add, T* __restrict__ dx,
                                                                 int N, int vpr, int K, int E) {
  constexpr int V = Vec16<T>::n;
  __shared__ float sdl[4][kTokTile * MOE_MAX_EXPERTS];
  const int lane = lane_id(), w = threadIdx.x >> 6;
  const int64_t n0 = ((int64_t)blockIdx.x * 4 + w) * kTokTile;
  if (n0 >= N) return;
  const int nt = int(min<int64_t>(kTokTile, N - n0));
  float* sd = sdl[w];
  for (int i = lane; i < nt * E; i += kWave) sd[i] = dl[n0 * E + i];  // rows n0.. are contiguous
  __builtin_amdgcn_wave_barrier();
  const uint4* wr = reinterpret_cast<const uint4*>(w_rt);
  const uint4* xs4 = reinterpret_cast<const uint4*>(dxs);
  for (int c = lane; c < vpr; c += kWave) {
    float acc[kTokTile][V];
#pragma unroll
    for (int t = 0; t < kTokTile; ++t) {
#pragma unroll
      for (int i = 0; i < V; ++i) acc[t][i] = 0.f;
      if (t < nt) {
        uint4 rx[MOE_MAX_TOPK];
        int32_t rr[MOE_MAX_TOPK];
#pragma unroll
        for (int k = 0; k < MOE_MAX_TOPK; ++k) {
          rr[k] = k < K ? inv[(n0 + t) * K + k] : -1;
          if (rr[k] >= 0) rx[k] = xs4[(int64_t)rr[k] * vpr + c];
        }
#pragma unroll
        for (int k = 0; k < MOE_MAX_TOPK; ++k)
          if (rr[k] >= 0) {
            float val[V];
            Vec16<T>::load(reinterpret_cast<const T*>(&rx[k]), val);
#pragma unroll
            for (int i = 0; i < V; ++i) acc[t][i] += val[i];
          }
      }
    }
    int e = 0;
    for (; e + 4 <= E; e += 4) {
      uint4 raw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) raw[q] = wr[(int64_t)(e + q) * vpr + c];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float wv[V];
        Vec16<T>::load(reinterpret_cast<const T*>(&raw[q]), wv);
#pragma unroll
        for (int t = 0; t < kTokTile; ++t) {
          const float de = sd[t * E + e + q];
#pragma unroll
          for (int i = 0; i < V; ++i) acc[t][i] = fmaf(de, wv[i], acc[t][i]);
        }
      }
    }
    for (; e < E; ++e) {
      const uint4 raw = wr[(int64_t)e * vpr + c];
      float wv[V];
      Vec16<T>::load(reinterpret_cast<const T*>(&raw), wv);
#pragma unroll
      for (int t = 0; t < kTokTile; ++t) {
        const float de = sd[t * E + e];
#pragma unroll
        for (int i = 0; i < V; ++i) acc[t][i] = fmaf(de, wv[i], acc[t][i]);
      }
    }
#pragma unroll
    for (int t = 0; t < kTokTile; ++t)
      if (t < nt) {
        if (add != nullptr) {
          float val[V];
          Vec16<T>::load(add + ((n0 + t) * vpr + c) * V, val);
#pragma unroll
          for (int i = 0; i < V; ++i) acc[t][i] += val[i];
        }
        Vec16<T>::store(dx + ((n0 + t) * vpr + c) * V, acc[t]);
      }
  }
}

// Calls f(std::integral_constant<int, K>) for K in 1..MOE_MAX_TOPK.
template <typename Fn>
hipError_t with_k(int K, Fn&& f) {
  static_assert(MOE_MAX_TOPK == 8, "one case per K");
  switch (K) {
    case 1: return f(std::integral_constant<int, 1>{});
    case 2: return f(std::integral_constant<int, 2>{});
    case 3: return f(std::integral_constant<int, 3>{});
    case 4: return f(std::integral_constant<int, 4>{});
    case 5: return f(std::integral_constant<int, 5>{});
    case 6: return f(std::integral_constant<int, 6>{});
    case 7: return f(std::integral_constant<int, 7>{});
    case 8: return f(std::integral_constant<int, 8>{});
    default: return hipErrorInvalidValue;
  }
}

unsigned grid_for(int64_t total, int64_t cap = 8192) {
  int64_t b = (total + 255) / 256;
  if (b > cap) b = cap;
  if (b < 1) b = 1;
  return unsigned(b);
}

// Workgroups of 4 waves, one wave per row.
unsigned waves4(int64_t rows) { return unsigned((rows + 3) / 4); }

// Row vectors a lane takes at a time in the token-wise row kernels: two once
// a row has at least two vectors per lane (more bytes in flight per wave),
// four once it has eight and K <= 2 (the row registers stay near 64; at
// N = 16384, K = 2, H = 4096 combine_bwd 151.6 -> 140.5 us, gather backward
// 85.2 -> 82.0, combine 81.7 -> 79.6 against two), else one.
template <int KT, typename Fn>
hipError_t with_u(int vpr, Fn&& f) {
  if constexpr (KT <= 2)
    if (vpr >= 8 * kWave) return f(std::integral_constant<int, 4>{});
  return vpr >= 2 * kWave ? f(std::integral_constant<int, 2>{}) : f(std::integral_constant<int, 1>{});
}

template <typename T>
int vpr_of(const moe_launch::Dims& d) {
  return int(d.H * int64_t(sizeof(T)) / 16);
}

}  // namespace

namespace moe_launch {

hipError_t permute(const Dims& d, const void* x, const int32_t* sorted_flat, void* xs, hipStream_t s) {
  if (d.dtype == MOE_BF16) {
    int vpr = vpr_of<moe::bf16_t>(d);
    int64_t tot = d.NK() * vpr;
    hipLaunchKernelGGL(k_permute<moe::bf16_t>, dim3(grid_for(tot)), dim3(256), 0, s,
                       static_cast<const moe::bf16_t*>(x), sorted_flat, static_cast<moe::bf16_t*>(xs), tot, vpr,
                       int(d.K));
  } else {
    int vpr = vpr_of<float>(d);
    int64_t tot = d.NK() * vpr;
    hipLaunchKernelGGL(k_permute<float>, dim3(grid_for(tot)), dim3(256), 0, s, static_cast<const float*>(x),
                       sorted_flat, static_cast<float*>(xs), tot, vpr, int(d.K));
  }
  return hipGetLastError();
}

hipError_t combine(const Dims& d, const void* ys, const float* gates, const int32_t* inv, const void* add, void* y,
                   hipStream_t s) {
  const int tpb = 4 * tok_per_wave(int(d.K));
  const unsigned grid = unsigned((d.N + tpb - 1) / tpb);
  auto run = [&](auto tag) {
    using T = decltype(tag);
    return with_k(int(d.K), [&](auto kt) {
      return with_u<decltype(kt)::value>(vpr_of<T>(d), [&](auto u) {
        hipLaunchKernelGGL((k_combine<T, decltype(kt)::value, decltype(u)::value>), dim3(grid), dim3(256), 0, s,
                           static_cast<const T*>(ys), gates, inv, static_cast<const T*>(add), static_cast<T*>(y),
                           int(d.N), vpr_of<T>(d));
        return hipGetLastError();
      });
    });
  };
  return d.dtype == MOE_BF16 ? run(moe::bf16_t{}) : run(float{});
}

hipError_t combine_bwd(const Dims& d, const void* dy, const void* ys, const float* gates, const int32_t* inv,
                       void* dys, float* dgates, hipStream_t s) {
  const int tpb = 4 * tok_per_wave(int(d.K));
  const unsigned grid = unsigned((d.N + tpb - 1) / tpb);
  auto run = [&](auto tag) {
    using T = decltype(tag);
    return with_k(int(d.K), [&](auto kt) {
      return with_u<decltype(kt)::value>(vpr_of<T>(d), [&](auto u) {
        hipLaunchKernelGGL((k_combine_bwd<T, decltype(kt)::value, decltype(u)::value>), dim3(grid), dim3(256), 0, s,
                           static_cast<const T*>(dy), static_cast<const T*>(ys), gates, inv, static_cast<T*>(dys),
                           dgates, int(d.N), vpr_of<T>(d));
        return hipGetLastError();
      });
    });
  };
  return d.dtype == MOE_BF16 ? run(moe::bf16_t{}) : run(float{});
}

size_t permute_bwd_ws(const Dims& d) {
  return size_t(d.H) * size_t(d.E) * (d.dtype == MOE_BF16 ? 2 : 4);
}

hipError_t permute_bwd(const Dims& d, const void* dxs, const int32_t* inv, const int32_t* topk, const float* dlogits,
                       const void* w_r, const void* add, void* dx, void* ws, hipStream_t s, bool dense) {
  int64_t nw = d.H * d.E;
  unsigned tg = unsigned((nw + 255) / 256);
  const int tpb = 4 * tok_per_wave(int(d.K));
  const unsigned grid = unsigned((d.N + tpb - 1) / tpb);
  auto run = [&](auto tag) -> hipError_t {
    using T = decltype(tag);
    hipLaunchKernelGGL(k_transpose_wr<T>, dim3(tg), dim3(256), 0, s, static_cast<const T*>(w_r), static_cast<T*>(ws),
                       int(d.H), int(d.E));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (dense && d.E > 8) {
      hipLaunchKernelGGL((k_permute_bwd_dense_tiled<T>), dim3(waves4((d.N + kTokTile - 1) / kTokTile)), dim3(256), 0,
                         s, static_cast<const T*>(dxs), inv, dlogits, static_cast<const T*>(ws), static_cast<const T*>(add),
                         static_cast<T*>(dx), int(d.N), vpr_of<T>(d), int(d.K), int(d.E));
      return hipGetLastError();
    }
    return with_k(int(d.K), [&](auto kt) {
      constexpr int KT = decltype(kt)::value;
      return with_u<decltype(kt)::value>(vpr_of<T>(d), [&](auto u) {
        constexpr int UU = decltype(u)::value;
        if (dense)
          hipLaunchKernelGGL((k_permute_bwd<T, true, KT, UU>), dim3(grid), dim3(256), 0, s, static_cast<const T*>(dxs),
                             inv, topk, dlogits, static_cast<const T*>(ws), static_cast<const T*>(add),
                             static_cast<T*>(dx), int(d.N), vpr_of<T>(d), int(d.E));
        else
          hipLaunchKernelGGL((k_permute_bwd<T, false, KT, UU>), dim3(grid), dim3(256), 0, s,
                             static_cast<const T*>(dxs), inv, topk, dlogits, static_cast<const T*>(ws),
                             static_cast<const T*>(add), static_cast<T*>(dx), int(d.N), vpr_of<T>(d), int(d.E));
        return hipGetLastError();
      });
    });
  };
  if (d.dtype == MOE_BF16) return run(moe::bf16_t{});
  return run(float{});
}

}  // namespace moe_launch
