// bf16 MFMA grouped GEMMs of the SwiGLU experts, forward and backward, for
// CDNA4 (gfx950, v_mfma_f32_32x32x16_bf16, float32 accumulation).
//
// Every expert's rows form one group of a grouped GEMM (one launch covers
// all experts; "MoE computation principle and execution process",
// section 3.4, merges same-expert tokens into one large GEMM; the dropless
// grouped GEMM without padding in memory is the grouped path of "MegaBlocks -
// architecture and principles", sections 2.1 and 2.3).  The row groups are
// read from the device-built tile list (expert, first row, rows), so no host
// synchronisation is needed: the grid is sized for the largest possible tile
// count and workgroups past the real count return at once.
//
// This file holds an older 128 x 128 shape.  The short-contraction forward
// GEMMs now run on the register-staged 128 x 128 tiles of gemm_bf16_big.hip;
// this one serves dX launched on its own below 2F = 2560, and every stage
// when the 128 family is forced.  Workgroup tile 128 x 128,
// K step 64, 256 threads = 4 waves in a 2 x 2 arrangement, 64 x 64 per wave
// (2 x 2 MFMA 32x32x16 per 16-deep k step).  One LDS buffer plus register
// prefetch keeps the LDS footprint near 34 KB, so 3 workgroups share a CU
// and hide each other's latency.  Each workgroup handles half of a 256-row
// list tile.
// Operand tiles live in LDS as [128 rows][64 k] bf16 (128 B per row, eight
// 16-byte chunks) with the chunk index XOR-swizzled by the row, so that both
// the MFMA fragment reads (8 consecutive rows, same chunk) and the staging
// writes are free of bank conflicts.  An operand whose K index is contiguous
// in memory is copied in 16-byte vectors; an operand whose M or N index is
// contiguous (the weights in the forward, both operands of the weight
// gradients) is loaded as 4(k) x 8(mn) blocks and transposed in registers
// before it is written to LDS.  The next K tile is prefetched into registers
// while the current one is multiplied.
//
// Determinism: every output element has exactly one owning workgroup and its
// K loop runs in ascending order.
#include "common.h"

namespace {
using namespace moe;

constexpr int BM = 128, BN = 128, BK = 64, NT = 256;
constexpr int kTileBytes = BM * BK * 2;  // one operand tile in LDS

__device__ __forceinline__ int swz(int row, int chunk) {
  return (row * 8 + (chunk ^ ((row ^ (row >> 3)) & 7))) * 16;
}

// 128 rows x 64 k of a row-major matrix whose k index is contiguous.
struct LoadKC {
  uint4 v[4];
  __device__ __forceinline__ void load(const bf16_t* base, int64_t ld, int rows_valid) {
    const int c = threadIdx.x & 7, r0 = threadIdx.x >> 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int r = r0 + 32 * i;
      if (r < rows_valid)
        v[i] = *reinterpret_cast<const uint4*>(base + (int64_t)r * ld + c * 8);
      else
        v[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
    const int c = threadIdx.x & 7, r0 = threadIdx.x >> 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(lds + swz(r0 + 32 * i, c)) = v[i];
  }
};

// 128 rows x 64 k gathered from the token matrix: tile row r is row
// rows_src[r] / K of x (the permute fused into the loads).  Offsets are
// computed once per tile; rows past the tile load zeros.
struct LoadKCg {
  uint4 v[4];
  int off[4];
  __device__ __forceinline__ void init(const int32_t* rows_src, int K, int64_t ld, int rows_valid) {
    const int c = threadIdx.x & 7, r0 = threadIdx.x >> 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + 32 * i;
      off[i] = r < rows_valid ? int((rows_src[r] / K) * ld) + c * 8 : -1;
    }
  }
  __device__ __forceinline__ void load(const bf16_t* x, int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = off[i] >= 0 ? *reinterpret_cast<const uint4*>(x + off[i] + k0) : make_uint4(0, 0, 0, 0);
  }
  __device__ __forceinline__ void store(char* lds) const {
    const int c = threadIdx.x & 7, r0 = threadIdx.x >> 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(lds + swz(r0 + 32 * i, c)) = v[i];
  }
};

// Thread -> (8-column group mc, 4-row group kg) of the MN loader.  Each
// 16-lane phase of a wave covers 8 column groups x 2 row groups, so its
// 8-byte transposed LDS writes land on 32 distinct banks, while every 8
// consecutive lanes still read one contiguous 128-byte segment of a row.
__device__ __forceinline__ int mn_mc() {
  const int l = threadIdx.x & 63;
  return (l & 7) | (((l >> 4) & 1) << 3);
}
__device__ __forceinline__ int mn_kg() {
  const int l = threadIdx.x & 63;
  return (((l >> 3) & 1) | ((l >> 5) << 1)) + 4 * (threadIdx.x >> 6);
}

// 64 k-rows x 128 mn-columns of a row-major matrix whose mn index is
// contiguous, stored to LDS transposed as [mn][k].
struct LoadMN {
  uint4 v[4];
  __device__ __forceinline__ void load(const bf16_t* base, int64_t ld, int k_valid) {
    const int mc = mn_mc(), kg = mn_kg();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int k = kg * 4 + j;
      if (k < k_valid)
        v[j] = *reinterpret_cast<const uint4*>(base + (int64_t)k * ld + mc * 8);
      else
        v[j] = make_uint4(0, 0, 0, 0);
    }
  }
  // k row k is token row rows_src[k] / K of x (base = x + the tile's column)
  __device__ __forceinline__ void load_gather(const bf16_t* base, const int32_t* rows_src, int K, int64_t ld,
                                              int k_valid) {
    const int mc = mn_mc(), kg = mn_kg();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int k = kg * 4 + j;
      if (k < k_valid)
        v[j] = *reinterpret_cast<const uint4*>(base + (int64_t)(rows_src[k] / K) * ld + mc * 8);
      else
        v[j] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
    const int mc = mn_mc(), kg = mn_kg();
    uint32_t w[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[j][0] = v[j].x; w[j][1] = v[j].y; w[j][2] = v[j].z; w[j][3] = v[j].w;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = i >> 1;
      uint32_t lo, hi;
      if ((i & 1) == 0) {
        lo = (w[0][q] & 0xffffu) | (w[1][q] << 16);
        hi = (w[2][q] & 0xffffu) | (w[3][q] << 16);
      } else {
        lo = (w[0][q] >> 16) | (w[1][q] & 0xffff0000u);
        hi = (w[2][q] >> 16) | (w[3][q] & 0xffff0000u);
      }
      const int row = mc * 8 + i;
      *reinterpret_cast<uint2*>(lds + swz(row, kg >> 1) + (kg & 1) * 8) = make_uint2(lo, hi);
    }
  }
};

// One 64-deep K step of the 64 x 64 wave tile: acc[mi][ni] += A . B^T.
__device__ __forceinline__ void mma_tile(const char* ldsA, const char* ldsB, f32x16_t (&acc)[2][2], int wm, int wn) {
  const int lane = lane_id();
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    const int chunk = kk * 2 + (lane >> 5);
    bf16x8_t a[2], b[2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
      a[mi] = *reinterpret_cast<const bf16x8_t*>(ldsA + swz(wm * 64 + mi * 32 + (lane & 31), chunk));
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
      b[ni] = *reinterpret_cast<const bf16x8_t*>(ldsB + swz(wn * 64 + ni * 32 + (lane & 31), chunk));
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
  }
}

__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[2][2]) {
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
}

// Output coordinates of accumulator element r of fragment (mi, ni) in the
// workgroup tile: MFMA 32x32 result layout (column = lane % 32, rows in groups
// of 4 interleaved across the two lane halves).
__device__ __forceinline__ int acc_row(int wm, int mi, int r) {
  return wm * 64 + mi * 32 + (r >> 2) * 8 + (lane_id() >> 5) * 4 + (r & 3);
}
__device__ __forceinline__ int acc_col(int wn, int ni) { return wn * 64 + ni * 32 + (lane_id() & 31); }

struct TileInfo {
  int e, row0, rows;
};

// The hardware places workgroup b on XCD b % 8 (each XCD has its own L2).
// Logical block L of `total` gets a contiguous range per XCD, so that the
// blocks sharing an operand tile (the n-tiles of one row tile, the output
// tiles of one expert) run on one XCD and share its L2.  The launch grid is
// a multiple of 8 and at least `total`; returns -1 for blocks with no work.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_block(int total) {
  const int b = blockIdx.x;
  const int per = (total + kXcds - 1) / kXcds;
  const int L = (b % kXcds) * per + b / kXcds;
  return (b / kXcds < per && L < total) ? L : -1;
}

// Logical block -> (row tile, n tile) in groups of kGroupM row tiles: inside
// a group the row tile varies fastest, so the workgroups an XCD runs at once
// cover a patch of row tiles x n tiles and share operand tiles in its L2.
constexpr int kGroupM = 8;
__device__ __forceinline__ void grouped(int L, int nrow, int ncol, int& row, int& col) {
  const int per_group = kGroupM * ncol;
  const int g = L / per_group, r = L % per_group;
  const int first = g * kGroupM;
  const int gm = min(kGroupM, nrow - first);
  row = first + r % gm;
  col = r / gm;
}

// Half `h` of the 256-row list tiles (two 128-row workgroup tiles per list
// tile); rows <= 0 when the list tile is shorter.
constexpr int kSub = MOE_TILE_M / BM;
__device__ __forceinline__ TileInfo half_tile(const int32_t* tiles, int h) {
  const int t = h / kSub, part = h % kSub;
  return TileInfo{tiles[3 * t], tiles[3 * t + 1] + part * BM, min(BM, tiles[3 * t + 2] - part * BM)};
}

// Output tiles leave through LDS: each lane deposits its accumulator elements
// (MFMA layout) into a [128][kEpiPitch] bf16 tile, then the workgroup writes
// whole rows with 16-byte stores.  The 8-element row padding puts the two
// lane halves of a fragment store (rows r and r+4) on different banks.
constexpr int kEpiPitch = BN + 8;
constexpr int kEpiBytes = BM * kEpiPitch * 2;
constexpr int kLds2 = (2 * kTileBytes > kEpiBytes) ? 2 * kTileBytes : kEpiBytes;

__device__ __forceinline__ int epi_off(int wm, int wn, int mi, int ni, int r) {
  return acc_row(wm, mi, r) * kEpiPitch + acc_col(wn, ni);
}

// rows [0, rows) of the staged tile -> out (leading dimension ld)
__device__ __forceinline__ void epi_store(const bf16_t* tile, bf16_t* out, int64_t ld, int rows) {
  const int c = threadIdx.x & 15;
#pragma unroll 4
  for (int r = threadIdx.x >> 4; r < rows; r += NT / 16)
    *reinterpret_cast<uint4*>(out + (int64_t)r * ld + c * 8) =
        *reinterpret_cast<const uint4*>(tile + r * kEpiPitch + c * 8);
}

// staged tile <- bf16(acc)
__device__ __forceinline__ void epi_put_acc(bf16_t* tile, const f32x16_t (&acc)[2][2], int wm, int wn) {
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) tile[epi_off(wm, wn, mi, ni, r)] = f32_to_bf16(acc[mi][ni][r]);
}

// ---------------------------------------------------------------- forward

// G = xs.W_gate[e], U = xs.W_up[e] (both rounded to bf16), A = silu(G)*U.
// The B tile interleaves 64 columns of W_gate[e] (tile columns 0..63) with
// the same 64 columns of W_up[e] (tile columns 64..127), so waves wn = 0
// hold G and waves wn = 1 hold U; the epilogue pairs them through LDS.
// GATHER: `xs` is the token matrix x and row i of the grouped order is read
// as x[sorted_flat[i] / K].
template <bool GATHER>
__global__ __launch_bounds__(NT, 2) void k_gate_up(const bf16_t* __restrict__ xs,
                                                    const int32_t* __restrict__ sorted_flat, int K,
                                                    const bf16_t* __restrict__ wg,
                                                    const bf16_t* __restrict__ wu, const int32_t* __restrict__ tiles,
                                                    const int32_t* __restrict__ num_tiles, bf16_t* __restrict__ g_out,
                                                    bf16_t* __restrict__ u_out, bf16_t* __restrict__ a_out, int H,
                                                    int F) {
  __shared__ __attribute__((aligned(16))) char lds[kLds2];
  constexpr int HALF = BN / 2;
  const int ntn = F / HALF;
  const int nrow = *num_tiles * kSub;
  const int L = xcd_block(nrow * ntn);
  if (L < 0) return;
  int ht, nt;
  grouped(L, nrow, ntn, ht, nt);
  const TileInfo ti = half_tile(tiles, ht);
  if (ti.rows <= 0) return;
  const int w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
  const bf16_t* a_base = xs + (int64_t)ti.row0 * H;
  // this thread's 8-column group of the B tile comes from W_gate or W_up
  const int mc = mn_mc();
  const bf16_t* b_base = ((mc < 8) ? wg : wu) + (int64_t)ti.e * H * F + nt * HALF - (mc < 8 ? 0 : HALF);

  f32x16_t acc[2][2];
  zero_acc(acc);
  LoadKC la;
  LoadKCg lg;
  LoadMN lb;
  const int nk = H / BK;
  if (GATHER) {
    lg.init(sorted_flat + ti.row0, K, H, ti.rows);
    lg.load(xs, 0);
  } else {
    la.load(a_base, H, ti.rows);
  }
  lb.load(b_base, F, BK);
  for (int kt = 0; kt < nk; ++kt) {
    if (GATHER)
      lg.store(lds);
    else
      la.store(lds);
    lb.store(lds + kTileBytes);
    __syncthreads();
    if (kt + 1 < nk) {
      if (GATHER)
        lg.load(xs, (kt + 1) * BK);
      else
        la.load(a_base + (kt + 1) * BK, H, ti.rows);
      lb.load(b_base + (int64_t)(kt + 1) * BK * F, F, BK);
    }
    mma_tile(lds, lds + kTileBytes, acc, wm, wn);
    __syncthreads();
  }
  // staged tile: columns 0..63 = G, 64..127 = U (bf16)
  bf16_t* stg = reinterpret_cast<bf16_t*>(lds);
  epi_put_acc(stg, acc, wm, wn);
  __syncthreads();
  const int64_t obase = (int64_t)ti.row0 * F + nt * HALF;
  const int c = threadIdx.x & 7;
#pragma unroll 4
  for (int r = threadIdx.x >> 3; r < ti.rows; r += NT / 8) {
    const uint4 gq = *reinterpret_cast<const uint4*>(stg + r * kEpiPitch + c * 8);
    const uint4 uq = *reinterpret_cast<const uint4*>(stg + r * kEpiPitch + HALF + c * 8);
    const int64_t o = obase + (int64_t)r * F + c * 8;
    if (g_out) {
      *reinterpret_cast<uint4*>(g_out + o) = gq;
      *reinterpret_cast<uint4*>(u_out + o) = uq;
    }
    const uint32_t gw[4] = {gq.x, gq.y, gq.z, gq.w}, uw[4] = {uq.x, uq.y, uq.z, uq.w};
    uint32_t aw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float g0 = __uint_as_float(gw[i] << 16), g1 = __uint_as_float(gw[i] & 0xffff0000u);
      const float u0 = __uint_as_float(uw[i] << 16), u1 = __uint_as_float(uw[i] & 0xffff0000u);
      aw[i] = pack_bf16x2(silu_f32(g0) * u0, silu_f32(g1) * u1);
    }
    *reinterpret_cast<uint4*>(a_out + o) = make_uint4(aw[0], aw[1], aw[2], aw[3]);
  }
}

// ys = A.W_down[e]
__global__ __launch_bounds__(NT, 2) void k_down(const bf16_t* __restrict__ act, const bf16_t* __restrict__ wd,
                                                 const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles,
                                                 bf16_t* __restrict__ ys, int H, int F) {
  __shared__ __attribute__((aligned(16))) char lds[kLds2];
  const int ntn = H / BN;
  const int nrow = *num_tiles * kSub;
  const int L = xcd_block(nrow * ntn);
  if (L < 0) return;
  int ht, nt;
  grouped(L, nrow, ntn, ht, nt);
  const TileInfo ti = half_tile(tiles, ht);
  if (ti.rows <= 0) return;
  const int w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
  const bf16_t* a_base = act + (int64_t)ti.row0 * F;
  const bf16_t* b_base = wd + (int64_t)ti.e * F * H + nt * BN;
  f32x16_t acc[2][2];
  zero_acc(acc);
  LoadKC la;
  LoadMN lb;
  const int nk = F / BK;
  la.load(a_base, F, ti.rows);
  lb.load(b_base, H, BK);
  for (int kt = 0; kt < nk; ++kt) {
    la.store(lds);
    lb.store(lds + kTileBytes);
    __syncthreads();
    if (kt + 1 < nk) {
      la.load(a_base + (kt + 1) * BK, F, ti.rows);
      lb.load(b_base + (int64_t)(kt + 1) * BK * H, H, BK);
    }
    mma_tile(lds, lds + kTileBytes, acc, wm, wn);
    __syncthreads();
  }
  bf16_t* stg = reinterpret_cast<bf16_t*>(lds);
  epi_put_acc(stg, acc, wm, wn);
  __syncthreads();
  epi_store(stg, ys + (int64_t)ti.row0 * H + nt * BN, H, ti.rows);
}

// --------------------------------------------------------------- backward

// dxs = dG.W_gate[e]^T + dU.W_up[e]^T  (one K loop over 2F)
__global__ __launch_bounds__(NT, 2) void k_dx(const bf16_t* __restrict__ dg, const bf16_t* __restrict__ du,
                                               const bf16_t* __restrict__ wg, const bf16_t* __restrict__ wu,
                                               const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles,
                                               bf16_t* __restrict__ dxs, int H, int F) {
  __shared__ __attribute__((aligned(16))) char lds[kLds2];
  const int ntn = H / BN;
  const int nrow = *num_tiles * kSub;
  const int L = xcd_block(nrow * ntn);
  if (L < 0) return;
  int ht, nt;
  grouped(L, nrow, ntn, ht, nt);
  const TileInfo ti = half_tile(tiles, ht);
  if (ti.rows <= 0) return;
  const int w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
  // B[k = f][n = h] = W[e][h][f]: rows h of W[e] are k-contiguous
  const int64_t woff = (int64_t)ti.e * H * F + (int64_t)nt * BN * F;
  f32x16_t acc[2][2];
  zero_acc(acc);
  LoadKC la, lb;
  const int nkf = F / BK, nk = 2 * nkf;
  auto load = [&](int kt) {
    const bool second = kt >= nkf;
    const int k0 = (second ? kt - nkf : kt) * BK;
    la.load((second ? du : dg) + (int64_t)ti.row0 * F + k0, F, ti.rows);
    lb.load((second ? wu : wg) + woff + k0, F, BN);
  };
  load(0);
  for (int kt = 0; kt < nk; ++kt) {
    la.store(lds);
    lb.store(lds + kTileBytes);
    __syncthreads();
    if (kt + 1 < nk) load(kt + 1);
    mma_tile(lds, lds + kTileBytes, acc, wm, wn);
    __syncthreads();
  }
  bf16_t* stg = reinterpret_cast<bf16_t*>(lds);
  epi_put_acc(stg, acc, wm, wn);
  __syncthreads();
  epi_store(stg, dxs + (int64_t)ti.row0 * H + nt * BN, H, ti.rows);
}

// Weight gradients, one workgroup per 128 x 128 output tile of one expert:
//   problem 0: dW_gate[e] = xs_e^T . dG_e   [H, F]
//   problem 1: dW_up[e]   = xs_e^T . dU_e   [H, F]
//   problem 2: dW_down[e] = A_e^T  . dys_e  [F, H]
// The contraction runs over the expert's rows in ascending 64-row steps.
// gsrc non-null: xs is x and the rows of dW_gate / dW_up are x[gsrc[i] / K]
__global__ __launch_bounds__(NT, 2) void k_dw(const bf16_t* __restrict__ xs, const bf16_t* __restrict__ act,
                                               const bf16_t* __restrict__ dys, const bf16_t* __restrict__ dg,
                                               const bf16_t* __restrict__ du, const int32_t* __restrict__ offsets,
                                               float* __restrict__ dwg, float* __restrict__ dwu,
                                               float* __restrict__ dwd, int H, int F, int E,
                                               const int32_t* __restrict__ gsrc, int K) {
  __shared__ __attribute__((aligned(16))) char lds[kLds2];
  const int tpe = (H / BM) * (F / BN);  // output tiles per expert and problem
  // experts largest first, each expert's 3 * tpe tiles consecutive, dealt to
  // the XCDs in runs of kXcdRun
  const int blk = xcd_window_block(3 * E * tpe);
  if (blk < 0) return;
  const int e = expert_of_rank<NT>(offsets, E, blk / (3 * tpe), reinterpret_cast<int*>(lds));
  const int prob = (blk % (3 * tpe)) / tpe, t = blk % tpe;
  const bf16_t *L, *R;
  float* out;
  int P, Q, mt, nt;
  if (prob < 2) {
    P = H; Q = F;
    L = xs; R = (prob == 0) ? dg : du;
    out = ((prob == 0) ? dwg : dwu) + (int64_t)e * H * F;
  } else {
    P = F; Q = H;
    L = act; R = dys;
    out = dwd + (int64_t)e * F * H;
  }
  mt = t / (Q / BN);
  nt = t % (Q / BN);
  const int w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
  const int r0 = offsets[e], cnt = offsets[e + 1] - r0;
  const bf16_t* l_base = L + (int64_t)r0 * P + mt * BM;
  const bf16_t* r_base = R + (int64_t)r0 * Q + nt * BN;
  f32x16_t acc[2][2];
  zero_acc(acc);
  LoadMN la, lb;
  const bool gather = gsrc != nullptr && prob < 2;
  const bf16_t* x_cols = xs + mt * BM;
  auto load_l = [&](int kt, int kv) {
    if (gather)
      la.load_gather(x_cols, gsrc + r0 + kt * BK, K, P, kv);
    else
      la.load(l_base + (int64_t)kt * BK * P, P, kv);
  };
  const int nk = (cnt + BK - 1) / BK;
  if (nk > 0) {
    load_l(0, cnt);
    lb.load(r_base, Q, cnt);
  }
  for (int kt = 0; kt < nk; ++kt) {
    la.store(lds);
    lb.store(lds + kTileBytes);
    __syncthreads();
    if (kt + 1 < nk) {
      const int kv = cnt - (kt + 1) * BK;
      load_l(kt + 1, kv);
      lb.load(r_base + (int64_t)(kt + 1) * BK * Q, Q, kv);
    }
    mma_tile(lds, lds + kTileBytes, acc, wm, wn);
    __syncthreads();
  }
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        out[(int64_t)(mt * BM + acc_row(wm, mi, r)) * Q + nt * BN + acc_col(wn, ni)] = acc[mi][ni][r];
}

}  // namespace

namespace moe_launch {

// grid size rounded up to whole XCD rounds
static unsigned grid8(int64_t n) { return unsigned((n + kXcds - 1) / kXcds * kXcds); }

// sorted_flat non-null: xs is x and the rows are gathered on load
hipError_t ffn_gate_up_small(const Dims& d, const void* xs, const int32_t* sorted_flat, const void* wg,
                             const void* wu, const int32_t* tiles, const int32_t* num_tiles, void* g, void* u,
                             void* a, hipStream_t s) {
  unsigned grid = grid8(max_tiles(d) * kSub * (d.F / (BN / 2)));
  if (sorted_flat)
    hipLaunchKernelGGL(k_gate_up<true>, dim3(grid), dim3(NT), 0, s, static_cast<const bf16_t*>(xs), sorted_flat,
                       int(d.K), static_cast<const bf16_t*>(wg), static_cast<const bf16_t*>(wu), tiles, num_tiles,
                       static_cast<bf16_t*>(g), static_cast<bf16_t*>(u), static_cast<bf16_t*>(a), int(d.H), int(d.F));
  else
    hipLaunchKernelGGL(k_gate_up<false>, dim3(grid), dim3(NT), 0, s, static_cast<const bf16_t*>(xs), nullptr,
                       int(d.K), static_cast<const bf16_t*>(wg), static_cast<const bf16_t*>(wu), tiles, num_tiles,
                       static_cast<bf16_t*>(g), static_cast<bf16_t*>(u), static_cast<bf16_t*>(a), int(d.H), int(d.F));
  return hipGetLastError();
}

hipError_t ffn_down_small(const Dims& d, const void* a, const void* wd, const int32_t* tiles, const int32_t* num_tiles,
                         void* ys, hipStream_t s) {
  unsigned grid = grid8(max_tiles(d) * kSub * (d.H / BN));
  hipLaunchKernelGGL(k_down, dim3(grid), dim3(NT), 0, s, static_cast<const bf16_t*>(a),
                     static_cast<const bf16_t*>(wd), tiles, num_tiles, static_cast<bf16_t*>(ys), int(d.H), int(d.F));
  return hipGetLastError();
}

hipError_t ffn_bwd_dx_small(const Dims& d, const void* dg, const void* du, const void* wg, const void* wu,
                           const int32_t* tiles, const int32_t* num_tiles, void* dxs, hipStream_t s) {
  unsigned grid = grid8(max_tiles(d) * kSub * (d.H / BN));
  hipLaunchKernelGGL(k_dx, dim3(grid), dim3(NT), 0, s, static_cast<const bf16_t*>(dg), static_cast<const bf16_t*>(du),
                     static_cast<const bf16_t*>(wg), static_cast<const bf16_t*>(wu), tiles, num_tiles,
                     static_cast<bf16_t*>(dxs), int(d.H), int(d.F));
  return hipGetLastError();
}

// sorted_flat non-null: xs is x and dW_gate / dW_up gather their rows
hipError_t ffn_bwd_dw_small(const Dims& d, const void* xs, const int32_t* sorted_flat, const void* a, const void* dys,
                            const void* dg, const void* du, const int32_t* offsets, float* dwg, float* dwu,
                            float* dwd, hipStream_t s) {
  const int64_t total = 3 * d.E * (d.H / BM) * (d.F / BN);
  const int64_t win = 8 * kXcdRun;
  unsigned grid = unsigned((total + win - 1) / win * win);
  hipLaunchKernelGGL(k_dw, dim3(grid), dim3(NT), 0, s, static_cast<const bf16_t*>(xs), static_cast<const bf16_t*>(a),
                     static_cast<const bf16_t*>(dys), static_cast<const bf16_t*>(dg), static_cast<const bf16_t*>(du),
                     offsets, dwg, dwu, dwd, int(d.H), int(d.F), int(d.E), sorted_flat, int(d.K));
  return hipGetLastError();
}

}  // namespace moe_launch
