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
//                position of entry f is its expert's base plus the number of
//                earlier entries with the same expert.
#include "common.h"

namespace {
using namespace moe;

constexpr int kChunk = 4096;           // flat entries per workgroup
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
  if (tid < E) blk_hist[(int64_t)blockIdx.x * E + tid] = hist[tid];
}

// Inclusive scan of one int per thread over the 256 threads of the block.
__device__ int block_inclusive_scan(int v, int* buf) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    int add = (tid >= off) ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  int r = buf[tid];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(256) void k_meta_scan(int32_t* __restrict__ blk, int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets, int32_t* __restrict__ tiles,
                                                   int32_t* __restrict__ num_tiles, int nblk, int E, int NK,
                                                   int tile_m) {
  __shared__ int buf[256];
  const int e = threadIdx.x;
  // per-expert total, and each chunk's exclusive prefix within the expert
  int total = 0;
  if (e < E) {
    for (int b = 0; b < nblk; ++b) {
      int c = blk[(int64_t)b * E + e];
      blk[(int64_t)b * E + e] = total;
      total += c;
    }
  }
  int incl = block_inclusive_scan(e < E ? total : 0, buf);
  int off = incl - (e < E ? total : 0);
  if (e < E) {
    counts[e] = total;
    offsets[e] = off;
    for (int b = 0; b < nblk; ++b) blk[(int64_t)b * E + e] += off;
  }
  if (e == 0) offsets[E] = NK;
  // tile list: ceil(count / tile_m) tiles per expert, experts ascending
  int nt = (e < E) ? (total + tile_m - 1) / tile_m : 0;
  int tincl = block_inclusive_scan(nt, buf);
  int tfirst = tincl - nt;
  for (int t = 0; t < nt; ++t) {
    int64_t o = 3 * (int64_t)(tfirst + t);
    tiles[o + 0] = e;
    tiles[o + 1] = off + t * tile_m;
    tiles[o + 2] = min(tile_m, total - t * tile_m);
  }
  if (e == 255) *num_tiles = tincl;
}

__global__ __launch_bounds__(256) void k_meta_rank(const int32_t* __restrict__ topk, const int32_t* __restrict__ blk,
                                                   int32_t* __restrict__ sorted_flat, int32_t* __restrict__ inv, int NK,
                                                   int E, int key_bits) {
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
    int run = blk[(int64_t)blockIdx.x * E + tid];
    for (int q = 0; q < 4; ++q) {
      int c = wcount[q][tid];
      wcount[q][tid] = run;
      run += c;
    }
  }
  __syncthreads();
  // pass 2: stable positions, 64 entries at a time in flat order
  for (int p = 0; p < kPerWave; p += kWave) {
    int f = base + p + lane;
    int key = (f < NK) ? topk[f] : -1;
    bool valid = unsigned(key) < unsigned(E);
    if (!valid) key = 0;
    uint64_t m = match(key, valid);
    int pos = 0;
    if (valid) {
      pos = wcount[w][key] + __popcll(m & lt_mask);
      sorted_flat[pos] = f;
      inv[f] = pos;
    }
    __builtin_amdgcn_wave_barrier();
    if (valid && (m & lt_mask) == 0) wcount[w][key] += __popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

namespace moe_launch {

int64_t max_tiles(const Dims& d) { return (d.NK() + d.E * (MOE_TILE_M - 1)) / MOE_TILE_M; }

size_t permute_meta_ws(const Dims& d) {
  int64_t nblk = (d.NK() + kChunk - 1) / kChunk;
  return size_t(nblk) * size_t(d.E) * sizeof(int32_t);
}

hipError_t permute_meta(const Dims& d, const int32_t* topk, int32_t* sorted_flat, int32_t* inv, int32_t* counts,
                        int32_t* offsets, int32_t* tiles, int32_t* num_tiles, void* ws, hipStream_t s) {
  int NK = int(d.NK());
  int E = int(d.E);
  int nblk = (NK + kChunk - 1) / kChunk;
  int32_t* blk = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(k_meta_hist, dim3(nblk), dim3(256), 0, s, topk, blk, NK, E);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_meta_scan, dim3(1), dim3(256), 0, s, blk, counts, offsets, tiles, num_tiles, nblk, E, NK,
                     MOE_TILE_M);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  int key_bits = 0;
  while ((1 << key_bits) < E) ++key_bits;
  hipLaunchKernelGGL(k_meta_rank, dim3(nblk), dim3(256), 0, s, topk, blk, sorted_flat, inv, NK, E, key_bits);
  return hipGetLastError();
}

}  // namespace moe_launch
