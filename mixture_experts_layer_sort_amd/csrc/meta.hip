// Dropless routing metadata on the device, with no host synchronisation:
// histogram of the flat assignment, exclusive cumsum into expert bins, a
// stable counting sort of the flat indices by expert id, its inverse, and the
// grouped-GEMM tile list ("MegaBlocks - architecture and principles",
// sections 2.1 and 2.3: sort, histogram, cumsum into bins; section 4: the
// sort key is only the expert id, so a counting sort over E <= 256 buckets
// replaces a radix sort).
//
// Three launches over chunks of kChunk flat entries:
//   k_meta_hist  per-chunk expert histogram in LDS (integer atomics: the
//                counts do not depend on their order);
//   k_meta_scan  one workgroup: per-expert totals, exclusive scan over the
//                experts, per-chunk bases, and the tile list;
//   k_meta_rank  stable ranks: each wave walks its sub-chunk in order, 64
//                entries at a time, and ranks equal keys with ballots, so the
//                rank of entry f within its expert is the number of earlier
//                entries with the same expert.
//
// Expert capacity C ("MoE computation principle and execution process",
// section 3.4): an entry whose rank within its expert is C or more is dropped
// (inv = -1); expert e keeps min(count_e, C) rows, the bins (offsets) and the
// tile list cover the kept rows only, and sorted_flat lists the kept rows
// followed by -1 for each dropped one.  counts stays the full histogram.
// With C >= every count nothing is dropped and the result is the dropless one.
#include <algorithm>

#include "common.h"

namespace {
using namespace moe;

constexpr int kChunk = 1024;           // flat entries per workgroup
constexpr int kPerWave = kChunk / 4;   // entries per wave (4 waves)

__global__ __launch_bounds__(256) void k_meta_hist(const int32_t* __restrict__ topk, int32_t* __restrict__ blk_hist,
                                                   int NK, int E) {
  __shared__ int hist[MOE_MAX_EXPERTS];
  const int tid = threadIdx.x;
  hist[tid] = 0;
  __syncthreads();
  const int base = blockIdx.x * kChunk;
  for (int i = tid; i < kChunk; i += 256) {
    int f = base + i;
    if (f < NK) {
      unsigned key = unsigned(topk[f]);
      if (key < unsigned(E)) atomicAdd(&hist[key], 1);  // out-of-range ids are dropped, never written
    }
  }
  __syncthreads();
  if (tid < E) blk_hist[(int64_t)tid * gridDim.x + blockIdx.x] = hist[tid];  // expert-major [E][nblk]
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int t = __shfl_up(v, off, kWave);
    if (lane >= off) v += t;
  }
  return v;
}

// Exclusive prefix sums over the experts of vals[0, E) (E <= 256) by one
// wave: lane l holds experts 4l .. 4l+3.  Writes the prefix to out[e] and
// returns the grand total (in every lane).
__device__ __forceinline__ int wave_excl_scan_experts(const int* vals, int* out, int E) {
  const int lane = lane_id();
  int v[4], ls = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * lane + j;
    v[j] = e < E ? vals[e] : 0;
    ls += v[j];
  }
  const int incl = wave_incl_scan(ls);
  int run = incl - ls;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * lane + j;
    if (e < E) out[e] = run;
    run += v[j];
  }
  return __shfl(incl, kWave - 1, kWave);
}

// One workgroup of 16 waves.  blk [E][nblk] holds the chunk histograms on
// entry and, on exit, the rank within its expert of the first entry of each
// (expert, chunk): the counts of the expert's earlier chunks.  pos [2][E]
// receives, per expert, the first position of its kept rows and of its
// dropped rows (after all kept rows).  Also writes counts (full), offsets
// (kept rows) and the tile list (ceil(kept / tile_m) tiles per expert,
// experts ascending).
constexpr int kScanWaves = 16;
__global__ __launch_bounds__(kScanWaves * 64) void k_meta_scan(int32_t* __restrict__ blk, int32_t* __restrict__ pos,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ tiles,
                                                              int32_t* __restrict__ num_tiles, int nblk, int E,
                                                              int tile_m, int capacity) {
  __shared__ int tot[MOE_MAX_EXPERTS], kept[MOE_MAX_EXPERTS], drop[MOE_MAX_EXPERTS], off[MOE_MAX_EXPERTS],
      doff[MOE_MAX_EXPERTS], ntl[MOE_MAX_EXPERTS], tfirst[MOE_MAX_EXPERTS];
  __shared__ int nkept;
  const int w = threadIdx.x >> 6, lane = lane_id();
  // expert totals (wave per expert; integer sums, order-free)
  for (int e = w; e < E; e += kScanWaves) {
    int sum = 0;
    for (int b = lane; b < nblk; b += kWave) sum += blk[(int64_t)e * nblk + b];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, kWave);
    if (lane == 0) {
      const int k = min(sum, capacity);
      tot[e] = sum;
      kept[e] = k;
      drop[e] = sum - k;
      ntl[e] = (k + tile_m - 1) / tile_m;
    }
  }
  __syncthreads();
  if (w == 0) {
    const int nk = wave_excl_scan_experts(kept, off, E);
    wave_excl_scan_experts(drop, doff, E);
    const int nt = wave_excl_scan_experts(ntl, tfirst, E);
    if (lane == 0) {
      *num_tiles = nt;
      offsets[E] = nk;
      nkept = nk;
    }
  }
  __syncthreads();
  // per-chunk bases: exclusive prefix over the chunks of each expert
  for (int e = w; e < E; e += kScanWaves) {
    int carry = 0;
    for (int b0 = 0; b0 < nblk; b0 += kWave) {
      const int b = b0 + lane;
      const int c = b < nblk ? blk[(int64_t)e * nblk + b] : 0;
      const int incl = wave_incl_scan(c);
      if (b < nblk) blk[(int64_t)e * nblk + b] = carry + incl - c;
      carry += __shfl(incl, kWave - 1, kWave);
    }
  }
  // counts, offsets, first kept / dropped positions and the tiles of expert e
  for (int e = threadIdx.x; e < E; e += kScanWaves * 64) {
    counts[e] = tot[e];
    offsets[e] = off[e];
    pos[e] = off[e];
    pos[E + e] = nkept + doff[e];
    for (int t = 0; t < ntl[e]; ++t) {
      const int64_t o = 3 * (int64_t)(tfirst[e] + t);
      tiles[o + 0] = e;
      tiles[o + 1] = off[e] + t * tile_m;
      tiles[o + 2] = min(tile_m, kept[e] - t * tile_m);
    }
  }
}

__global__ __launch_bounds__(256) void k_meta_rank(const int32_t* __restrict__ topk, const int32_t* __restrict__ blk,
                                                   const int32_t* __restrict__ pos0, int32_t* __restrict__ sorted_flat,
                                                   int32_t* __restrict__ inv, int NK, int E, int key_bits,
                                                   int capacity) {
  const int nblk = gridDim.x;
  __shared__ int wcount[4][MOE_MAX_EXPERTS];
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = lane_id();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int i = tid; i < 4 * MOE_MAX_EXPERTS; i += 256) (&wcount[0][0])[i] = 0;
  __syncthreads();
  const int base = blockIdx.x * kChunk + w * kPerWave;

  // lanes holding the same key as this lane (among valid lanes)
  auto match = [&](int key, bool valid) -> uint64_t {
    uint64_t m = __ballot(valid);
    for (int b = 0; b < key_bits; ++b) {
      bool bit = (key >> b) & 1;
      uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    return m;
  };

  // pass 1: per-wave histogram of the sub-chunk
  for (int p = 0; p < kPerWave; p += kWave) {
    int f = base + p + lane;
    int key = (f < NK) ? topk[f] : -1;
    bool valid = unsigned(key) < unsigned(E);
    if (!valid) key = 0;
    uint64_t m = match(key, valid);
    if (valid && (m & lt_mask) == 0) wcount[w][key] += __popcll(m);
  }
  __syncthreads();
  // per-wave bases: chunk base of the expert + earlier waves of this chunk
  if (tid < E) {
    int run = blk[(int64_t)tid * nblk + blockIdx.x];
    for (int q = 0; q < 4; ++q) {
      int c = wcount[q][tid];
      wcount[q][tid] = run;
      run += c;
    }
  }
  __syncthreads();
  // pass 2: stable ranks, 64 entries at a time in flat order; a kept entry
  // goes to its expert's kept rows, a dropped one marks a dropped row
  for (int p = 0; p < kPerWave; p += kWave) {
    int f = base + p + lane;
    int key = (f < NK) ? topk[f] : -1;
    bool valid = unsigned(key) < unsigned(E);
    if (!valid) key = 0;
    uint64_t m = match(key, valid);
    if (valid) {
      const int g = wcount[w][key] + __popcll(m & lt_mask);
      if (g < capacity) {
        const int pos = pos0[key] + g;
        sorted_flat[pos] = f;
        inv[f] = pos;
      } else {
        sorted_flat[pos0[E + key] + (g - capacity)] = -1;
        inv[f] = -1;
      }
    }
    __builtin_amdgcn_wave_barrier();
    if (valid && (m & lt_mask) == 0) wcount[w][key] += __popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
}

// The metadata from the router's block histograms, in one launch (the
// router and the metadata fused into two launches instead of four).  The
// router's workgroups own kRouteBlockTok tokens each and leave the histogram
// of their chosen experts in rh [nrb][E].  Workgroup c of this kernel owns
// the flat entries of route blocks [c*G, (c+1)*G): it adds up every block
// histogram itself (integer adds, order-free), which gives the expert totals
// and the counts of the blocks before its own without waiting on any other
// workgroup, then ranks its entries as k_meta_rank does (each wave a quarter
// of them, in flat order).  Workgroup 0 also writes counts, offsets and the
// tile list.  Same results as k_meta_hist + k_meta_scan + k_meta_rank.
constexpr int kRouteBlockTok = 32;
__global__ __launch_bounds__(256) void k_meta_fused(const int32_t* __restrict__ topk, const int32_t* __restrict__ rh,
                                                    int nrb, int G, int32_t* __restrict__ sorted_flat,
                                                    int32_t* __restrict__ inv, int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets, int32_t* __restrict__ tiles,
                                                    int32_t* __restrict__ num_tiles, int NK, int E, int K,
                                                    int key_bits, int tile_m, int capacity) {
  __shared__ int tot[MOE_MAX_EXPERTS], pre[MOE_MAX_EXPERTS], kept[MOE_MAX_EXPERTS], drop[MOE_MAX_EXPERTS],
      koff[MOE_MAX_EXPERTS], doff[MOE_MAX_EXPERTS], ntl[MOE_MAX_EXPERTS], tfirst[MOE_MAX_EXPERTS];
  __shared__ int wcount[4][MOE_MAX_EXPERTS];
  __shared__ int nkept;
  const int tid = threadIdx.x, w = tid >> 6, lane = lane_id();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int i = tid; i < MOE_MAX_EXPERTS; i += 256) {
    tot[i] = 0;
    pre[i] = 0;
  }
  for (int i = tid; i < 4 * MOE_MAX_EXPERTS; i += 256) (&wcount[0][0])[i] = 0;
  __syncthreads();
  // expert totals and the counts of the route blocks before this chunk
  const int b0 = blockIdx.x * G;
  const int64_t n_el = (int64_t)nrb * E, pre_el = (int64_t)b0 * E;
  if (256 % E == 0) {
    // every count this thread reads belongs to expert tid % E: private sums,
    // then one add per thread
    int st = 0, sp = 0;
    int64_t i = tid;
    for (; i + 7 * 256 < n_el; i += 8 * 256) {  // eight loads in flight
      int v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = rh[i + j * 256];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        st += v[j];
        sp += i + j * 256 < pre_el ? v[j] : 0;
      }
    }
    for (; i < n_el; i += 256) {
      const int v = rh[i];
      st += v;
      sp += i < pre_el ? v : 0;
    }
    if (st != 0) atomicAdd(&tot[tid % E], st);
    if (sp != 0) atomicAdd(&pre[tid % E], sp);
  } else {
    for (int64_t i = tid; i < n_el; i += 256) {
      const int v = rh[i];
      if (v != 0) {
        const int e = int(i % E);
        atomicAdd(&tot[e], v);
        if (i < pre_el) atomicAdd(&pre[e], v);
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    const int k = min(tot[e], capacity);
    kept[e] = k;
    drop[e] = tot[e] - k;
    ntl[e] = (k + tile_m - 1) / tile_m;
  }
  __syncthreads();
  if (w == 0) {
    const int nk = wave_excl_scan_experts(kept, koff, E);
    wave_excl_scan_experts(drop, doff, E);
    const int nt = wave_excl_scan_experts(ntl, tfirst, E);
    if (lane == 0) {
      nkept = nk;
      if (blockIdx.x == 0) {
        *num_tiles = nt;
        offsets[E] = nk;
      }
    }
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int e = tid; e < E; e += 256) {
      counts[e] = tot[e];
      offsets[e] = koff[e];
      for (int t = 0; t < ntl[e]; ++t) {
        const int64_t o = 3 * (int64_t)(tfirst[e] + t);
        tiles[o + 0] = e;
        tiles[o + 1] = koff[e] + t * tile_m;
        tiles[o + 2] = min(tile_m, kept[e] - t * tile_m);
      }
    }
  }
  // this chunk's entries, a quarter per wave
  const int64_t cbeg = (int64_t)b0 * kRouteBlockTok * K;
  const int64_t cend = min((int64_t)(b0 + G) * kRouteBlockTok * K, (int64_t)NK);
  const int q = int((cend - cbeg + 3) / 4);
  const int64_t wbeg = cbeg + (int64_t)w * q;
  const int64_t wend = min(wbeg + q, cend);
  auto match = [&](int key, bool valid) -> uint64_t {
    uint64_t m = __ballot(valid);
    for (int b = 0; b < key_bits; ++b) {
      bool bit = (key >> b) & 1;
      uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    return m;
  };
  // pass 1: per-wave histogram
  for (int64_t p = wbeg; p < wend; p += kWave) {
    const int64_t f = p + lane;
    int key = (f < wend) ? topk[f] : -1;
    const bool valid = unsigned(key) < unsigned(E);
    if (!valid) key = 0;
    const uint64_t m = match(key, valid);
    if (valid && (m & lt_mask) == 0) wcount[w][key] += __popcll(m);
  }
  __syncthreads();
  // per-wave bases: the counts of the earlier blocks + earlier waves
  if (tid < E) {
    int run = pre[tid];
    for (int qq = 0; qq < 4; ++qq) {
      const int c = wcount[qq][tid];
      wcount[qq][tid] = run;
      run += c;
    }
  }
  __syncthreads();
  // pass 2: stable ranks in flat order; kept entries to their expert's bin,
  // dropped ones (rank >= capacity) mark a dropped row after all kept rows
  for (int64_t p = wbeg; p < wend; p += kWave) {
    const int64_t f = p + lane;
    int key = (f < wend) ? topk[f] : -1;
    const bool valid = unsigned(key) < unsigned(E);
    if (!valid) key = 0;
    const uint64_t m = match(key, valid);
    if (valid) {
      const int g = wcount[w][key] + __popcll(m & lt_mask);
      if (g < capacity) {
        const int pos = koff[key] + g;
        sorted_flat[pos] = int(f);
        inv[f] = pos;
      } else {
        sorted_flat[nkept + doff[key] + (g - capacity)] = -1;
        inv[f] = -1;
      }
    }
    __builtin_amdgcn_wave_barrier();
    if (valid && (m & lt_mask) == 0) wcount[w][key] += __popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

namespace moe_launch {

int64_t max_tiles(const Dims& d) { return (d.NK() + d.E * (MOE_TILE_M - 1)) / MOE_TILE_M; }

// Route blocks and the fused metadata's chunking: each of its workgroups
// re-reads all nrb * E block counts, so the fused path is taken while that
// is at most kFusedMaxCounts (128 KiB); above it the router and the three
// metadata kernels run separately (same results).
constexpr int64_t kFusedMaxCounts = 32768;
static int64_t route_blocks(const Dims& d) { return (d.N + kRouteBlockTok - 1) / kRouteBlockTok; }
static bool route_meta_fused(const Dims& d) { return route_blocks(d) * d.E <= kFusedMaxCounts; }

size_t route_meta_ws(const Dims& d) {
  if (route_meta_fused(d)) return size_t(route_blocks(d) * d.E) * sizeof(int32_t);
  return permute_meta_ws(d);
}

hipError_t route_meta(const Dims& d, const void* x, const void* w_r, const float* bias, int32_t capacity,
                      int32_t* topk, float* gates, int32_t* sorted_flat, int32_t* inv, int32_t* counts,
                      int32_t* offsets, int32_t* tiles, int32_t* num_tiles, void* ws, hipStream_t s) {
  if (!route_meta_fused(d)) {
    hipError_t err = route(d, x, w_r, bias, topk, gates, s);
    if (err != hipSuccess) return err;
    return permute_meta(d, topk, capacity, sorted_flat, inv, counts, offsets, tiles, num_tiles, ws, s);
  }
  int32_t* rh = static_cast<int32_t*>(ws);
  hipError_t err = route(d, x, w_r, bias, topk, gates, s, rh);
  if (err != hipSuccess) return err;
  const int nrb = int(route_blocks(d));
  const int G = std::max(1, kChunk / (kRouteBlockTok * int(d.K)));
  const int nchunks = (nrb + G - 1) / G;
  int key_bits = 0;
  while ((1 << key_bits) < d.E) ++key_bits;
  hipLaunchKernelGGL(k_meta_fused, dim3(nchunks), dim3(256), 0, s, topk, rh, nrb, G, sorted_flat, inv, counts,
                     offsets, tiles, num_tiles, int(d.NK()), int(d.E), int(d.K), key_bits, MOE_TILE_M,
                     int(capacity));
  return hipGetLastError();
}

// [E][nblk] chunk histograms / bases, then [2][E] first kept / dropped positions
size_t permute_meta_ws(const Dims& d) {
  int64_t nblk = (d.NK() + kChunk - 1) / kChunk;
  return (size_t(nblk) * size_t(d.E) + 2 * size_t(d.E)) * sizeof(int32_t);
}

hipError_t permute_meta(const Dims& d, const int32_t* topk, int32_t capacity, int32_t* sorted_flat, int32_t* inv,
                        int32_t* counts, int32_t* offsets, int32_t* tiles, int32_t* num_tiles, void* ws,
                        hipStream_t s) {
  int NK = int(d.NK());
  int E = int(d.E);
  int nblk = (NK + kChunk - 1) / kChunk;
  int32_t* blk = static_cast<int32_t*>(ws);
  int32_t* pos = blk + (int64_t)nblk * E;
  hipLaunchKernelGGL(k_meta_hist, dim3(nblk), dim3(256), 0, s, topk, blk, NK, E);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_meta_scan, dim3(1), dim3(kScanWaves * 64), 0, s, blk, pos, counts, offsets, tiles, num_tiles, nblk,
                     E, MOE_TILE_M, int(capacity));
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  int key_bits = 0;
  while ((1 << key_bits) < E) ++key_bits;
  hipLaunchKernelGGL(k_meta_rank, dim3(nblk), dim3(256), 0, s, topk, blk, pos, sorted_flat, inv, NK, E, key_bits,
                     int(capacity));
  return hipGetLastError();
}

}  // namespace moe_launch
