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
// Workgroup tile 256 x 256, K step 64.  A 256 x 256 x 64 step moves 64 KB
// from L2 for 8.4 MFLOP.  Used for the long contractions;
// gemm_bf16_small.hip holds the 128 x 128 shape for short ones.
//
// Main configuration (Big8): 8 waves in a 4 x 2 arrangement, 64 x 128 per
// wave (128 accumulator registers each, two waves per SIMD, one workgroup
// per CU), on the mixed-depth LDS DMA loop of mma_lds.h (k_loop_dma2):
// operand A one K tile ahead in two LDS slots, operand B two K tiles ahead in
// three, both moved by buffer-resource LDS DMA, so 96 KB per CU are in flight
// and none of it occupies registers.  Every GEMM stage on this tile runs it
// (gate/up with its W_gate and W_up columns as two B sub-tiles, one per wave
// column).  The register-staged loop (k_loop_reg: each thread's 16-byte
// chunks of the next K tile requested into registers between the MFMAs and
// stored into the other LDS stage) remains for the 128-row tiles.
//
// A K-contiguous operand (token rows; weight rows in the backward) sits in
// LDS as [rows][64 k] and is read with 16-byte fragment loads; an
// MN-contiguous operand (the weights in the forward, both operands of the
// weight gradients) sits as [64 k][columns] and is read with the transposing
// LDS load (ds_read_b64_tr_b16), so no operand is ever transposed in
// registers.  Both layouts XOR-swizzle 16-byte chunks by row so the fragment
// reads are free of bank conflicts.  Output tiles leave through LDS with
// 16-byte row stores.
//
// Tails: N (and, for the weight gradients, M) may end on a 128 boundary
// inside a tile; loads past the end read clamped in-bounds positions whose
// results are never stored, and the ragged contraction tail of the weight
// gradients is zeroed in LDS.
//
// Determinism: every output element has exactly one owning workgroup and its
// K loop runs in ascending order.
#include <type_traits>

#include "common.h"

#include "mma_lds.h"


namespace {
using namespace moe;

using namespace moe_mma;

// 256 x 256 tiles with 8 waves of 64 x 128 (two per SIMD, each covering the
// other's issue stalls).  On the register-staged loop 8 waves measured faster
// than 4 waves of 128 x 128 for dX, the weight gradients, down and dA (merged
// dX/dW 866-870 -> 891-896 TFLOP/s at H = 512, F = 1024, E = 8; 846-851 ->
// 881 at the skewed H = 2048, E = 64 workload) and equal for gate/up (7.22 vs
// 7.20 ms at H = 4096, F = 14336).  On k_loop_dma2, which the Big8 kernels
// run (160 KiB of LDS slots, requested by the launches), gate/up gained
// further against its 4-wave register-staged tile: 7.11-7.13 -> 6.92-6.95 ms
// there, 5.12-5.18 -> 4.71 ms at H = 7168, E = 256 and 1.27-1.28 -> 1.19-1.20
// ms at the skewed workload (interleaved runs, one box).
using Big8 = TileCfg<256, 256, 4, 2, 1, 64, 2, true>;
// 128 x 256 tiles through the same DMA pipeline, 32 k per stage, three stages
// (72 KiB of LDS, two workgroups per CU): used by the SwiGLU backward on
// short contractions, where its two workgroups per CU overlap one's SwiGLU
// epilogue with the other's main loop better than the register-staged
// kernels do.
using Mid = TileCfg<128, 256, 2, 4, 2, 32, 3>;
// 128 x 256 tiles on the register-staged loop: 4 waves of 64 x 128, 32 k per
// stage, two stages (48 KiB of operands, 65 KiB with the staged dA),
// two workgroups per CU so one's epilogue overlaps the other's main loop.
using MidR = TileCfg<128, 256, 2, 2, 2, 32, 2, true>;
// 128 x 128 tiles on the register-staged loop for the short-contraction
// forward GEMMs (H or F below the 256 x 256 thresholds): 4 waves of 64 x 64.
// gate/up takes 32 k per stage (32 KiB of operands, four workgroups per CU);
// down takes 64 k per stage (64 KiB, two per CU).  At H = 512, F = 1024
// they measured 121-123 against 125-129 us (gate/up) and 61 against 68 us
// (down) for the 128 x 128 kernels of gemm_bf16_small.hip.
using SmallR32 = TileCfg<128, 128, 2, 2, 4, 32, 2, true>;
using SmallR64 = TileCfg<128, 128, 2, 2, 2, 64, 2, true>;
// dX tiles inside the merged dX / weight-gradient launch.  128 x 256 tiles
// would balance that launch better (at H = 512, F = 1024, E = 8 its 192
// weight-gradient tiles take 64 k steps and the dX tiles 32), but measured
// slower on every workload (221 -> 238 us there with 64 k per stage, 260 with
// 32): the smaller tile's operand traffic per flop outweighs the balance.
using DxInMerged = Big8;
static_assert(MOE_TILE_M % Big8::BM == 0 && MOE_TILE_M % Mid::BM == 0 &&
                  MOE_TILE_M % MidR::BM == 0 && MOE_TILE_M % SmallR32::BM == 0 && MOE_TILE_M % SmallR64::BM == 0,
              "list tiles split into row tiles");

// staged tile <- bf16(acc), as 32-bit pairs of neighbouring columns: lanes
// 2j and 2j+1 hold columns c and c+1 of the same rows, and element pairs
// (r, r+1) are rows R and R+1.  Each lane packs its own pair, swaps it with
// its neighbour (DPP quad permutation 1,0,3,2), and keeps row R of both
// columns (even lane) or row R+1 of both (odd lane): one 4-byte LDS store per
// two elements instead of two 2-byte ones, the same bytes (gate/up 111.4 ->
// 109.7 us and down 62.0 -> 60.9 us at H = 512, F = 1024; within noise at
// H = 4096, F = 14336, where a timing-only copy without the epilogues put
// them at 0.49 ms of gate/up's 7.24 and 0.30 ms of down's 3.61).
template <class C>
__device__ __forceinline__ void epi_put(bf16_t* stg, const Acc<C>& acc, int wm, int wn) {
  const int odd = lane_id() & 1;
  bf16_t* p = stg + (lane_row<C>(wm) + odd) * C::PITCH + lane_col<C>(wn) - odd;
  // bytes 0-3 = own pair, 4-7 = neighbour's: even keeps (own lo, its lo), odd (its hi, own hi)
  const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
#pragma unroll
  for (int mi = 0; mi < C::FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < C::FN; ++ni)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const uint32_t w = pack_bf16x2(acc.a[mi][ni][r], acc.a[mi][ni][r + 1]);
        const uint32_t y = uint32_t(__builtin_amdgcn_mov_dpp(int(w), 0xB1, 0xF, 0xF, false));
        *reinterpret_cast<uint32_t*>(p + frag_row(mi, r) * C::PITCH + ni * 32) = __builtin_amdgcn_perm(y, w, sel);
      }
}

// rows [0, rows) x columns [0, cols) of the staged tile -> out (leading dim ld)
template <class C>
__device__ __forceinline__ void epi_store(const bf16_t* stg, bf16_t* out, int64_t ld, int rows, int cols) {
  constexpr int CPR = C::BN / 8;  // 16-byte chunks per row
  const int c = threadIdx.x % CPR;
  if (c * 8 >= cols) return;
#pragma unroll 4
  for (int r = threadIdx.x / CPR; r < rows; r += C::NT / CPR)
    *reinterpret_cast<uint4*>(out + (int64_t)r * ld + c * 8) =
        *reinterpret_cast<const uint4*>(stg + r * C::PITCH + c * 8);
}

// rows [0, rows) x columns [0, cols) of a global bf16 tile -> staged tile
template <class C>
__device__ __forceinline__ void epi_load(bf16_t* stg, const bf16_t* in, int64_t ld, int rows, int cols) {
  constexpr int CPR = C::BN / 8;
  const int c = threadIdx.x % CPR;
  if (c * 8 >= cols) return;
#pragma unroll 4
  for (int r = threadIdx.x / CPR; r < rows; r += C::NT / CPR)
    *reinterpret_cast<uint4*>(stg + r * C::PITCH + c * 8) =
        *reinterpret_cast<const uint4*>(in + (int64_t)r * ld + c * 8);
}

constexpr int kNoSplit = 1 << 30;  // single-source K-contiguous operand

struct TileInfo {
  int e, row0, rows;
};

// The hardware places workgroup b on XCD b % 8 (each XCD has its own L2).
// Logical block L of `total` gets a contiguous range per XCD, so that the
// blocks sharing an operand tile (the n-tiles of one row tile, the output
// tiles of one expert) run on one XCD and share its L2.  The launch grid is
// a multiple of 8 and at least `total`; returns -1 for blocks with no work.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_block(int b, int total) {
  const int per = (total + kXcds - 1) / kXcds;
  const int L = (b % kXcds) * per + b / kXcds;
  return (b / kXcds < per && L < total) ? L : -1;
}
__device__ __forceinline__ int xcd_block(int total) { return xcd_block(blockIdx.x, total); }

// Logical block -> (row tile, n tile) in groups of gmax row tiles: inside
// a group the row tile varies fastest, so the ~32 workgroups an XCD runs at
// once cover a patch of gmax row tiles x 32/gmax n tiles and each weight
// tile and each activation tile is fetched from HBM once per patch.
constexpr int kGroupM = 8;
__device__ __forceinline__ void grouped(int L, int nrow, int ncol, int& row, int& col, int gmax) {
  const int per_group = gmax * ncol;
  const int g = L / per_group, r = L % per_group;
  const int first = g * gmax;
  const int gm = min(gmax, nrow - first);
  row = first + r % gm;
  col = r / gm;
}

// Weight-gradient tiles in patches: one XCD runs 32 workgroups at a time,
// and a patch of kPatchM x kPatchN output tiles of one problem shares
// kPatchM left panels and kPatchN right panels, each K step of which is
// fetched into the XCD's L2 once for the patch (a 1 x 8 run of tiles shares
// one left panel and fetches eight right panels).  Tile t of an mtiles x
// ntiles problem, patch-major: row groups of kPatchM row tiles; inside a
// group, column chunks of kPatchN; inside a chunk, the row tile fastest.
constexpr int kPatchM = 4, kPatchN = 8, kDwRun = kPatchM * kPatchN;

// Run length of the weight-gradient tiles per XCD window: one patch when
// there are at least that many tiles per XCD, else an even eighth of them
// (at H = 512, F = 1024, E = 8 the 192 tiles in runs of 32 would leave two
// XCDs without any: 201 -> 245 us for the merged dX/dW launch), at least 8.
__host__ __device__ __forceinline__ int dw_run(int64_t total) {
  const int64_t per_xcd = (total + 7) / 8;
  return int(per_xcd >= kDwRun ? kDwRun : (per_xcd < 8 ? 8 : per_xcd));
}

// xcd_window_block with a run length known at launch time.
__device__ __forceinline__ int xcd_window_block_rt(int b, int total, int run) {
  const int L = (b / (8 * run)) * (8 * run) + (b % 8) * run + (b / 8) % run;
  return L < total ? L : -1;
}
__device__ __forceinline__ void patch_tile(int t, int mtiles, int ntiles, int& mt, int& nt) {
  const int per_group = kPatchM * ntiles;
  const int g = t / per_group, r = t % per_group;
  const int gm = min(kPatchM, mtiles - g * kPatchM);
  const int chunk = r / (gm * kPatchN), rc = r % (gm * kPatchN);
  mt = g * kPatchM + rc % gm;
  nt = chunk * kPatchN + rc / gm;
}

// Row tile `sub` of the list tiles (C::SUB row tiles per list tile); rows <= 0
// when the list tile is shorter.
template <class C>
__device__ __forceinline__ TileInfo row_tile(const int32_t* tiles, int sub) {
  const int t = sub / C::SUB, part = sub % C::SUB;
  TileInfo ti{tiles[3 * t], tiles[3 * t + 1] + part * C::BM, min(C::BM, tiles[3 * t + 2] - part * C::BM)};
  return ti;
}

// ---------------------------------------------------------------- forward

// G = xs.W_gate[e], U = xs.W_up[e] (both rounded to bf16), A = silu(G)*U.
// The B tile interleaves BN/2 columns of W_gate[e] (tile columns 0..BN/2-1)
// with the same columns of W_up[e] (tile columns BN/2..BN-1): waves wn = 0
// hold G and waves wn = 1 hold U; the epilogue pairs them through LDS.
// GATHER: `xs` is the token matrix x and row i of the grouped order is read
// as x[sorted_flat[i] / K] (the permute fused into the A-tile loads).
template <class C, bool GATHER = false>
__global__ __launch_bounds__(C::NT, C::MINB) void k_gate_up(const bf16_t* __restrict__ xs,
                                                   const int32_t* __restrict__ sorted_flat, int K,
                                                   const bf16_t* __restrict__ wg,
                                                   const bf16_t* __restrict__ wu, const int32_t* __restrict__ tiles,
                                                   const int32_t* __restrict__ num_tiles, bf16_t* __restrict__ g_out,
                                                   bf16_t* __restrict__ u_out, bf16_t* __restrict__ a_out, int H,
                                                   int F, int gm) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr int HALF = C::BN / 2;
  const int ntn = F / HALF;
  const int nrow = *num_tiles * C::SUB;
  const int L = xcd_block(nrow * ntn);
  if (L < 0) return;
  int rt, nt;
  grouped(L, nrow, ntn, rt, nt, gm);
  const TileInfo ti = row_tile<C>(tiles, rt);
  if (ti.rows <= 0) return;
  const int w = threadIdx.x >> 6, wm = w / C::WN, wn = w % C::WN;
  const bf16_t* a_base = xs + (int64_t)ti.row0 * H;
  const int64_t eoff = (int64_t)ti.e * H * F + nt * HALF;
  // 8-column groups mc < BN/16 come from W_gate, the rest from W_up (tile
  // columns HALF.. map to the same F columns)
  const bf16_t* b_g = wg + eoff;
  const bf16_t* b_u = wu + eoff - HALF;

  Acc<C> acc;
  if constexpr (C::REG && C::NW >= 8) {
    // mixed-depth DMA loop; W_gate and W_up as two B sub-tiles, one per wave column
    const MnDma2<C::BN, C::BK, C::NW> wdma(b_g, b_u + HALF, F);
    if constexpr (GATHER)
      k_loop_dma2<C, false, true, KcGatherDma<C::BM, C::BK, C::NW>, MnDma2<C::BN, C::BK, C::NW>, true, true>(
          lds, acc, H / C::BK, KcGatherDma<C::BM, C::BK, C::NW>(xs, sorted_flat + ti.row0, K, H, ti.rows), wdma, wm,
          wn, wm * C::TM < ti.rows);
    else
      k_loop_dma2<C, false, true, KcDma<C::BM, C::BK, C::NW>, MnDma2<C::BN, C::BK, C::NW>, true, true>(
          lds, acc, H / C::BK, KcDma<C::BM, C::BK, C::NW>(a_base, H, ti.rows), wdma, wm, wn, wm * C::TM < ti.rows);
  } else if constexpr (GATHER) {
    static_assert(C::REG, "the gathered A tile uses the register-staged loop");
    k_loop_reg<C, false, true>(lds, acc, H / C::BK,
                               KcGather<C::BM, C::BK, C::NT>(xs, sorted_flat + ti.row0, K, H, ti.rows),
                               MnOp<C::BN, C::BK, C::NT>(b_g, b_u, HALF, F, C::BN), wm, wn, C::BK,
                               wm * C::TM < ti.rows);
  } else if constexpr (C::REG) {
    k_loop_reg<C, false, true>(lds, acc, H / C::BK, KcOp<C::BM, C::BK, C::NT>(a_base, a_base, kNoSplit, H, ti.rows),
                               MnOp<C::BN, C::BK, C::NT>(b_g, b_u, HALF, F, C::BN), wm, wn, C::BK,
                               wm * C::TM < ti.rows);
  } else {
    k_loop<C, false, true>(
        lds, acc, H / C::BK,
        [&](int kt, char* st, int j) { dma_kc<C::BM, C::BK, C::NW>(st, a_base + kt * C::BK, H, ti.rows, j); },
        [&](int kt, char* st, int j) {
          dma_mn<C::BN, C::BK, C::NW>(st, b_g + (int64_t)kt * C::BK * F, b_u + (int64_t)kt * C::BK * F, HALF, F,
                                      C::BK, C::BN, j);
        },
        wm, wn);
  }

  // staged tile: columns 0..HALF-1 = G, HALF..BN-1 = U (bf16)
  bf16_t* stg = reinterpret_cast<bf16_t*>(lds);
  epi_put<C>(stg, acc, wm, wn);
  __syncthreads();
  const int64_t obase = (int64_t)ti.row0 * F + nt * HALF;
  constexpr int CPR = HALF / 8;
  const int c = threadIdx.x % CPR;
#pragma unroll 4
  for (int r = threadIdx.x / CPR; r < ti.rows; r += C::NT / CPR) {
    const uint4 gq = *reinterpret_cast<const uint4*>(stg + r * C::PITCH + c * 8);
    const uint4 uq = *reinterpret_cast<const uint4*>(stg + r * C::PITCH + HALF + c * 8);
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
template <class C>
__global__ __launch_bounds__(C::NT, C::MINB) void k_down(const bf16_t* __restrict__ act, const bf16_t* __restrict__ wd,
                                                const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles,
                                                bf16_t* __restrict__ ys, int H, int F, int gm) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int ntn = (H + C::BN - 1) / C::BN;
  const int nrow = *num_tiles * C::SUB;
  const int L = xcd_block(nrow * ntn);
  if (L < 0) return;
  int rt, nt;
  grouped(L, nrow, ntn, rt, nt, gm);
  const TileInfo ti = row_tile<C>(tiles, rt);
  if (ti.rows <= 0) return;
  const int ncols = min(C::BN, H - nt * C::BN);
  const int w = threadIdx.x >> 6, wm = w / C::WN, wn = w % C::WN;
  const bf16_t* a_base = act + (int64_t)ti.row0 * F;
  const bf16_t* b_base = wd + (int64_t)ti.e * F * H + nt * C::BN;
  Acc<C> acc;
  if constexpr (C::REG && C::NW >= 8) {
    k_loop_dma2<C, false, true, KcDma<C::BM, C::BK, C::NW>, MnDma<C::BN, C::BK, C::NW>, false, true>(
        lds, acc, F / C::BK, KcDma<C::BM, C::BK, C::NW>(a_base, F, ti.rows), MnDma<C::BN, C::BK, C::NW>(b_base, H, ncols),
        wm, wn, wm * C::TM < ti.rows);
  } else if constexpr (C::REG) {
    k_loop_reg<C, false, true>(lds, acc, F / C::BK, KcOp<C::BM, C::BK, C::NT>(a_base, a_base, kNoSplit, F, ti.rows),
                               MnBuf<C::BN, C::BK, C::NT>(b_base, H, ncols, F), wm, wn, C::BK,
                               wm * C::TM < ti.rows);
  } else {
    k_loop<C, false, true>(
        lds, acc, F / C::BK,
        [&](int kt, char* st, int j) { dma_kc<C::BM, C::BK, C::NW>(st, a_base + kt * C::BK, F, ti.rows, j); },
        [&](int kt, char* st, int j) {
          const bf16_t* b = b_base + (int64_t)kt * C::BK * H;
          dma_mn<C::BN, C::BK, C::NW>(st, b, b, C::BN, H, C::BK, ncols, j);
        },
        wm, wn);
  }
  bf16_t* stg = reinterpret_cast<bf16_t*>(lds);
  epi_put<C>(stg, acc, wm, wn);
  __syncthreads();
  epi_store<C>(stg, ys + (int64_t)ti.row0 * H + nt * C::BN, H, ti.rows, ncols);
}

// --------------------------------------------------------------- backward

// Thread layout of the SwiGLU backward epilogue: 16-byte chunks (8 bf16)
// of a TM x BN part, CPR per row, RPP rows per pass of the workgroup, CH
// chunks per thread; NB register buffers of G and U (two: the next part's
// loads are in flight while this part computes; one where the second would
// not fit the registers of MINB workgroups per CU); dA staged in float32
// with pitch FP.
template <class C>
struct DactEpi {
  static constexpr int CPR = C::BN / 8;
  static constexpr int RPP = C::NT / CPR;
  static constexpr int CH = C::TM / RPP;
  static constexpr int NB = CH <= 4 && C::MINB * C::NW <= 8 ? 2 : 1;
  static constexpr int FP = C::BN + 4;
  static_assert(C::NT % CPR == 0 && C::TM % RPP == 0, "whole rows per pass, whole passes per part");
  static_assert(C::TM * FP * 4 <= C::LDS, "the staged dA of one part fits the LDS");
};

// dA = dys.W_down[e]^T; dG = dA*U*s*(1+G*(1-s)), dU = dA*G*s with s = sigmoid(G).
template <class C>
__global__ __launch_bounds__(C::NT, C::MINB) void k_dact(const bf16_t* __restrict__ dys, const bf16_t* __restrict__ wd,
                                                const bf16_t* __restrict__ g_in, const bf16_t* __restrict__ u_in,
                                                const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles,
                                                bf16_t* __restrict__ dg, bf16_t* __restrict__ du, int H, int F,
                                                int gm) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int ntn = (F + C::BN - 1) / C::BN;
  const int nrow = *num_tiles * C::SUB;
  const int L = xcd_block(nrow * ntn);
  if (L < 0) return;
  int rt, nt;
  grouped(L, nrow, ntn, rt, nt, gm);
  const TileInfo ti = row_tile<C>(tiles, rt);
  if (ti.rows <= 0) return;
  const int ncols = min(C::BN, F - nt * C::BN);
  const int w = threadIdx.x >> 6, wm = w / C::WN, wn = w % C::WN;
  const bf16_t* a_base = dys + (int64_t)ti.row0 * H;
  // B[k = h][n = f] = W_down[e][f][h]: rows f of W_down[e] are k-contiguous
  const bf16_t* b_base = wd + (int64_t)ti.e * F * H + (int64_t)nt * C::BN * H;
  Acc<C> acc;
  if constexpr (C::REG && C::NW >= 8) {
    k_loop_dma2<C, false, false>(lds, acc, H / C::BK, KcDma<C::BM, C::BK, C::NW>(a_base, H, ti.rows),
                             KcDma<C::BN, C::BK, C::NW>(b_base, H, ncols), wm, wn, wm * C::TM < ti.rows);
  } else if constexpr (C::REG) {
    k_loop_reg<C, false, false>(lds, acc, H / C::BK, KcOp<C::BM, C::BK, C::NT>(a_base, a_base, kNoSplit, H, ti.rows),
                                KcOp<C::BN, C::BK, C::NT>(b_base, b_base, kNoSplit, H, ncols), wm, wn, C::BK,
                                wm * C::TM < ti.rows);
  } else {
    k_loop<C, false, false>(
        lds, acc, H / C::BK,
        [&](int kt, char* st, int j) { dma_kc<C::BM, C::BK, C::NW>(st, a_base + kt * C::BK, H, ti.rows, j); },
        [&](int kt, char* st, int j) { dma_kc<C::BN, C::BK, C::NW>(st, b_base + kt * C::BK, H, ncols, j); }, wm, wn);
  }

  // Epilogue, one wave row (TM rows) per part: the waves owning the part
  // write its float32 dA to LDS; then every thread takes 16-byte column
  // chunks of G and U straight from global memory (loaded one part ahead
  // when the registers allow), reads the matching dA, and stores its dG and
  // dU chunks straight to global memory.  All waves share the SwiGLU
  // arithmetic, which dominates the epilogue (against G and U staged in LDS
  // and only the owning waves computing: dA 4.56 -> 4.05 ms at H = 4096,
  // F = 14336, 112 -> 103 us at H = 512, F = 1024, bit-identical outputs).
  using EP = DactEpi<C>;
  float* sda = reinterpret_cast<float*>(lds);
  const int64_t obase = (int64_t)ti.row0 * F + nt * C::BN;
  const int c = threadIdx.x % EP::CPR, r0 = threadIdx.x / EP::CPR;
  const bool cok = c * 8 < ncols;
  uint4 gq[EP::NB][EP::CH], uq[EP::NB][EP::CH];
  auto load_part = [&](int part, uint4(&g)[EP::CH], uint4(&u)[EP::CH]) {
#pragma unroll
    for (int i = 0; i < EP::CH; ++i) {
      const int row = part * C::TM + r0 + i * EP::RPP;
      if (cok && row < ti.rows) {
        const int64_t o = obase + (int64_t)row * F + c * 8;
        g[i] = *reinterpret_cast<const uint4*>(g_in + o);
        u[i] = *reinterpret_cast<const uint4*>(u_in + o);
      }
    }
  };
  if constexpr (EP::NB == 2) load_part(0, gq[0], uq[0]);
  float* wsda = sda + ((lane_id() >> 5) * 4) * EP::FP + lane_col<C>(wn);
#pragma unroll
  for (int part = 0; part < C::WM; ++part) {
    const int rb = part * C::TM;
    const int nr = min(C::TM, ti.rows - rb);
    if (nr <= 0) break;
    const int cb = EP::NB == 2 ? (part & 1) : 0;
    if constexpr (EP::NB == 1) load_part(part, gq[0], uq[0]);
    if (wm == part) {
#pragma unroll
      for (int mi = 0; mi < C::FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::FN; ++ni)
#pragma unroll
          for (int r = 0; r < 16; ++r) wsda[frag_row(mi, r) * EP::FP + ni * 32] = acc.a[mi][ni][r];
    }
    __syncthreads();
    if constexpr (EP::NB == 2)
      if (part + 1 < C::WM) load_part(part + 1, gq[cb ^ 1], uq[cb ^ 1]);
#pragma unroll
    for (int i = 0; i < EP::CH; ++i) {
      const int row = r0 + i * EP::RPP;
      if (!cok || row >= nr) continue;
      const float4* pa = reinterpret_cast<const float4*>(sda + row * EP::FP + c * 8);
      const float4 a0 = pa[0], a1 = pa[1];
      const float da[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const uint32_t gw[4] = {gq[cb][i].x, gq[cb][i].y, gq[cb][i].z, gq[cb][i].w};
      const uint32_t uw[4] = {uq[cb][i].x, uq[cb][i].y, uq[cb][i].z, uq[cb][i].w};
      uint32_t dgw[4], duw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float dgv[2], duv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float gv = __uint_as_float(h ? (gw[j] & 0xffff0000u) : (gw[j] << 16));
          const float uv = __uint_as_float(h ? (uw[j] & 0xffff0000u) : (uw[j] << 16));
          const float sg = sigmoid_f32(gv);
          const float a = da[2 * j + h];
          dgv[h] = a * uv * sg * (1.f + gv * (1.f - sg));
          duv[h] = a * gv * sg;
        }
        dgw[j] = pack_bf16x2(dgv[0], dgv[1]);
        duw[j] = pack_bf16x2(duv[0], duv[1]);
      }
      const int64_t o = obase + (int64_t)(rb + row) * F + c * 8;
      *reinterpret_cast<uint4*>(dg + o) = make_uint4(dgw[0], dgw[1], dgw[2], dgw[3]);
      *reinterpret_cast<uint4*>(du + o) = make_uint4(duw[0], duw[1], duw[2], duw[3]);
    }
    __syncthreads();
  }
}

// dxs = dG.W_gate[e]^T + dU.W_up[e]^T  (one K loop over 2F); b: this
// workgroup's block index within the dX part of the launch.
template <class C>
__device__ __forceinline__ void dx_tile(char* lds, int b, const bf16_t* __restrict__ dg,
                                        const bf16_t* __restrict__ du, const bf16_t* __restrict__ wg,
                                        const bf16_t* __restrict__ wu, const int32_t* __restrict__ tiles,
                                        const int32_t* __restrict__ num_tiles, bf16_t* __restrict__ dxs, int H,
                                        int F, int gm) {
  const int ntn = (H + C::BN - 1) / C::BN;
  const int nrow = *num_tiles * C::SUB;
  const int L = xcd_block(b, nrow * ntn);
  if (L < 0) return;
  int rt, nt;
  grouped(L, nrow, ntn, rt, nt, gm);
  const TileInfo ti = row_tile<C>(tiles, rt);
  if (ti.rows <= 0) return;
  const int ncols = min(C::BN, H - nt * C::BN);
  const int w = threadIdx.x >> 6, wm = w / C::WN, wn = w % C::WN;
  // B[k = f][n = h] = W[e][h][f]: rows h of W[e] are k-contiguous
  const int64_t woff = (int64_t)ti.e * H * F + (int64_t)nt * C::BN * F;
  const int nkf = F / C::BK;
  Acc<C> acc;
  if constexpr (C::REG && C::NW >= 8) {
    const int64_t aoff = (int64_t)ti.row0 * F;
    k_loop_dma2<C, false, false>(lds, acc, 2 * nkf, KcDma<C::BM, C::BK, C::NW>(dg + aoff, du + aoff, nkf, F, ti.rows),
                             KcDma<C::BN, C::BK, C::NW>(wg + woff, wu + woff, nkf, F, ncols), wm, wn,
                             wm * C::TM < ti.rows);
  } else if constexpr (C::REG) {
    const int64_t aoff = (int64_t)ti.row0 * F;
    k_loop_reg<C, false, false>(lds, acc, 2 * nkf,
                                KcOp<C::BM, C::BK, C::NT>(dg + aoff, du + aoff, nkf, F, ti.rows),
                                KcOp<C::BN, C::BK, C::NT>(wg + woff, wu + woff, nkf, F, ncols), wm, wn, C::BK,
                                wm * C::TM < ti.rows);
  } else {
  k_loop<C, false, false>(
      lds, acc, 2 * nkf,
      [&](int kt, char* st, int j) {
        const bool second = kt >= nkf;
        dma_kc<C::BM, C::BK, C::NW>(st, (second ? du : dg) + (int64_t)ti.row0 * F + (second ? kt - nkf : kt) * C::BK, F,
                             ti.rows, j);
      },
      [&](int kt, char* st, int j) {
        const bool second = kt >= nkf;
        dma_kc<C::BN, C::BK, C::NW>(st, (second ? wu : wg) + woff + (second ? kt - nkf : kt) * C::BK, F, ncols, j);
      },
      wm, wn);
  }
  bf16_t* stg = reinterpret_cast<bf16_t*>(lds);
  epi_put<C>(stg, acc, wm, wn);
  __syncthreads();
  epi_store<C>(stg, dxs + (int64_t)ti.row0 * H + nt * C::BN, H, ti.rows, ncols);
}

template <class C>
__global__ __launch_bounds__(C::NT, C::MINB) void k_dx(const bf16_t* __restrict__ dg, const bf16_t* __restrict__ du,
                                              const bf16_t* __restrict__ wg, const bf16_t* __restrict__ wu,
                                              const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles,
                                              bf16_t* __restrict__ dxs, int H, int F, int gm) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  dx_tile<C>(lds, blockIdx.x, dg, du, wg, wu, tiles, num_tiles, dxs, H, F, gm);
}

// Weight gradients, one workgroup per BM x BN output tile of one expert:
//   problem 0: dW_gate[e] = xs_e^T . dG_e   [H, F]
//   problem 1: dW_up[e]   = xs_e^T . dU_e   [H, F]
//   problem 2: dW_down[e] = A_e^T  . dys_e  [F, H]
// The contraction runs over the expert's rows in ascending 64-row steps;
// experts without rows write exact zeros.
// b: this workgroup's block index within the dW part of the launch.
// GATHER: xs is the token matrix x and row i of the grouped order is read as
// x[sorted_flat[i] / K] (dW_gate and dW_up gather their rows on load).
template <class C, bool GATHER = false>
__device__ __forceinline__ void dw_tile(char* lds, int b, const bf16_t* __restrict__ xs,
                                        const bf16_t* __restrict__ act, const bf16_t* __restrict__ dys,
                                        const bf16_t* __restrict__ dg, const bf16_t* __restrict__ du,
                                        const int32_t* __restrict__ offsets, float* __restrict__ dwg,
                                        float* __restrict__ dwu, float* __restrict__ dwd, int H, int F, int E,
                                        const int32_t* __restrict__ sorted_flat = nullptr, int K = 1) {
  const int tf = (F + C::BN - 1) / C::BN, th2 = (H + C::BN - 1) / C::BN;
  const int tpe = ((H + C::BM - 1) / C::BM) * tf;    // output tiles of problems 0 and 1 per expert
  const int tpe2 = ((F + C::BM - 1) / C::BM) * th2;  // ... of problem 2
  const int per = 2 * tpe + tpe2;
  // experts largest first, each expert's tiles consecutive, dealt to the XCDs
  // in runs of dw_run (one patch when there are enough tiles)
  const int blk = xcd_window_block_rt(b, E * per, dw_run(int64_t(E) * per));
  if (blk < 0) return;
  const int e = expert_of_rank<C::NT>(offsets, E, blk / per, reinterpret_cast<int*>(lds));
  const int within = blk % per;
  const int prob = within < 2 * tpe ? within / tpe : 2;
  const int t = within - prob * tpe;
  const bf16_t *Lm, *Rm;
  float* out;
  int P, Q, mt, nt;
  if (prob < 2) {
    P = H; Q = F;
    Lm = xs; Rm = (prob == 0) ? dg : du;
    out = ((prob == 0) ? dwg : dwu) + (int64_t)e * H * F;
    patch_tile(t, tpe / tf, tf, mt, nt);
  } else {
    P = F; Q = H;
    Lm = act; Rm = dys;
    out = dwd + (int64_t)e * F * H;
    patch_tile(t, tpe2 / th2, th2, mt, nt);
  }
  const int prow = min(C::BM, P - mt * C::BM), qcol = min(C::BN, Q - nt * C::BN);
  const int w = threadIdx.x >> 6, wm = w / C::WN, wn = w % C::WN;
  const int r0 = offsets[e], cnt = offsets[e + 1] - r0;
  const bf16_t* l_base = Lm + (int64_t)r0 * P + mt * C::BM;
  const bf16_t* r_base = Rm + (int64_t)r0 * Q + nt * C::BN;
  Acc<C> acc;
  const int nk = (cnt + C::BK - 1) / C::BK;
  if constexpr (GATHER && C::REG && C::NW >= 8) {
    // dW_gate / dW_up: the k rows of xs gathered from x by DMA (their token numbers loaded a step ahead)
    if (prob < 2)
      k_loop_dma2<C, true, true>(lds, acc, nk,
                                 MnGatherDma<C::BM, C::BK, C::NW>(xs + mt * C::BM, sorted_flat + r0, K, P, prow, cnt),
                                 MnDma<C::BN, C::BK, C::NW>(r_base, Q, qcol, cnt), wm, wn, true,
                                 cnt - (nk - 1) * C::BK);
    else
      k_loop_dma2<C, true, true>(lds, acc, nk, MnDma<C::BM, C::BK, C::NW>(l_base, P, prow, cnt),
                                 MnDma<C::BN, C::BK, C::NW>(r_base, Q, qcol, cnt), wm, wn, true,
                                 cnt - (nk - 1) * C::BK);
  } else if constexpr (GATHER) {
    static_assert(C::REG, "the gathered rows use the register-staged loop");
    if (prob < 2)
      k_loop_reg<C, true, true>(lds, acc, nk,
                                MnGather<C::BM, C::BK, C::NT>(xs + mt * C::BM, sorted_flat + r0, K, P, prow, cnt),
                                MnBuf<C::BN, C::BK, C::NT>(r_base, Q, qcol, cnt), wm, wn, cnt - (nk - 1) * C::BK);
    else
      k_loop_reg<C, true, true>(lds, acc, nk, MnBuf<C::BM, C::BK, C::NT>(l_base, P, prow, cnt),
                                MnBuf<C::BN, C::BK, C::NT>(r_base, Q, qcol, cnt), wm, wn, cnt - (nk - 1) * C::BK);
  } else if constexpr (C::REG && C::NW >= 8) {
    k_loop_dma2<C, true, true>(lds, acc, nk, MnDma<C::BM, C::BK, C::NW>(l_base, P, prow, cnt),
                            MnDma<C::BN, C::BK, C::NW>(r_base, Q, qcol, cnt), wm, wn, true,
                            cnt - (nk - 1) * C::BK);
  } else if constexpr (C::REG) {
    k_loop_reg<C, true, true>(lds, acc, nk, MnBuf<C::BM, C::BK, C::NT>(l_base, P, prow, cnt),
                              MnBuf<C::BN, C::BK, C::NT>(r_base, Q, qcol, cnt), wm, wn, cnt - (nk - 1) * C::BK);
  } else {
  k_loop<C, true, true>(
      lds, acc, nk,
      [&](int kt, char* st, int j) {
        const bf16_t* b = l_base + (int64_t)kt * C::BK * P;
        dma_mn<C::BM, C::BK, C::NW>(st, b, b, C::BM, P, cnt - kt * C::BK, prow, j);
      },
      [&](int kt, char* st, int j) {
        const bf16_t* b = r_base + (int64_t)kt * C::BK * Q;
        dma_mn<C::BN, C::BK, C::NW>(st, b, b, C::BN, Q, cnt - kt * C::BK, qcol, j);
      },
      wm, wn, cnt - (nk - 1) * C::BK);
  }
  const int lr = lane_row<C>(wm), lc = lane_col<C>(wn);
  float* o = out + (int64_t)(mt * C::BM + lr) * Q + nt * C::BN + lc;
#pragma unroll
  for (int mi = 0; mi < C::FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < C::FN; ++ni) {
      if (lc + ni * 32 < qcol) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (lr + frag_row(mi, r) < prow) o[(int64_t)frag_row(mi, r) * Q + ni * 32] = acc.a[mi][ni][r];
      }
    }
}

template <class C, bool GATHER = false>
__global__ __launch_bounds__(C::NT, C::MINB) void k_dw(const bf16_t* __restrict__ xs, const bf16_t* __restrict__ act,
                                              const bf16_t* __restrict__ dys, const bf16_t* __restrict__ dg,
                                              const bf16_t* __restrict__ du, const int32_t* __restrict__ offsets,
                                              float* __restrict__ dwg, float* __restrict__ dwu,
                                              float* __restrict__ dwd, int H, int F, int E,
                                              const int32_t* __restrict__ sorted_flat, int K) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  dw_tile<C, GATHER>(lds, blockIdx.x, xs, act, dys, dg, du, offsets, dwg, dwu, dwd, H, F, E, sorted_flat, K);
}

// dX and dW in one launch.  Both read only dG and dU (plus xs, A, dys and the
// weights), so their tiles are independent: the first dw_grid workgroups take
// the weight-gradient tiles (longest contractions first), the rest the dX
// tiles, which fill the CUs the weight gradients leave idle and their tail.
// dw_grid is a multiple of 8 * dw_run, so both parts keep their XCD mapping.
// CW: the weight-gradient tiles' shape; CX: the dX tiles' shape (same block
// size; the launch gets the larger LDS of the two).
template <class CW, class CX, bool GATHER = false>
__global__ __launch_bounds__(CW::NT, CW::MINB) void k_dx_dw(
    const bf16_t* __restrict__ dg, const bf16_t* __restrict__ du, const bf16_t* __restrict__ wg,
    const bf16_t* __restrict__ wu, const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles,
    bf16_t* __restrict__ dxs, const bf16_t* __restrict__ xs, const bf16_t* __restrict__ act,
    const bf16_t* __restrict__ dys, const int32_t* __restrict__ offsets, float* __restrict__ dwg,
    float* __restrict__ dwu, float* __restrict__ dwd, int H, int F, int E, int dw_grid, int dx_grid,
    const int32_t* __restrict__ sorted_flat, int K, int gm) {
  static_assert(CW::NT == CX::NT, "one block size");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int b = blockIdx.x;
  // Longest contraction first: a dX tile runs 2F deep, a weight-gradient tile
  // as deep as its expert's rows (the largest expert's first, inside dw_tile).
  // Decided on the device from the counts, so no host sync: at N = 16384,
  // H = 4096, F = 14336, E = 8 (dX first) the launch went from 17.67-17.74 to
  // 17.51-17.52 ms (interleaved runs on one box); with skewed routing
  // (H = 2048, F = 1408, E = 64, largest expert 16 324 rows) dW first is 3 %
  // faster than dX first.  Both grids are whole XCD rounds, so either order
  // keeps the XCD mapping of each part.
  // (wave-uniform in a scalar register: as a vector value the branch below
  // would count as divergent and keep both tile paths live, spilling)
  const bool dx_first = __builtin_amdgcn_readfirstlane(2 * F >= max_expert_rows(offsets, E) ? 1 : 0) != 0;
  if (dx_first ? b < dx_grid : b >= dw_grid)
    dx_tile<CX>(lds, dx_first ? b : b - dw_grid, dg, du, wg, wu, tiles, num_tiles, dxs, H, F, gm);
  else
    dw_tile<CW, GATHER>(lds, dx_first ? b - dx_grid : b, xs, act, dys, dg, du, offsets, dwg, dwu, dwd, H, F, E,
                        sorted_flat, K);
}

}  // namespace

namespace moe_launch {

// Dynamic LDS of a launch: the 8-wave register-staged tiles may run the
// mixed-depth DMA loop, whose slots take 160 KiB (one workgroup per CU either
// way).
template <class C>
constexpr int lds_bytes_of() {
  return C::REG && C::NW >= 8 && C::BM == 256 ? Dma2Layout<C>::LDS : C::LDS;
}

// grid size rounded up to whole XCD rounds
static unsigned grid8(int64_t n) { return unsigned((n + kXcds - 1) / kXcds * kXcds); }

// Row tiles per patch of the row-tile GEMMs: kGroupM when the experts average
// more than one row tile of bm rows, so a patch's row tiles mostly belong to
// one expert and share its weight tiles; else 1, so a patch covers all n
// tiles of one row tile, which share its activation panel (row tiles of
// different experts share nothing).  At N = 8192, H = 7168, F = 2048,
// E = 256, K = 8 (256 rows per expert): gate/up 5.27-5.28 -> 5.13 ms and down
// 2.71-2.72 -> 2.66 ms against patches of 8 row tiles (2 and 4: no gain).
static int group_rows(const Dims& d, int bm) {
  return int64_t(d.N) * d.K > int64_t(d.E) * bm ? kGroupM : 1;
}

template <class C, bool GATHER = false>
static hipError_t gate_up_t(const Dims& d, const void* xs, const int32_t* sorted_flat, const void* wg, const void* wu,
                            const int32_t* tiles, const int32_t* num_tiles, void* g, void* u, void* a, hipStream_t s) {
  constexpr int lds_bytes = lds_bytes_of<C>();
  hipError_t st = allow_lds<k_gate_up<C, GATHER>>(lds_bytes);
  if (st != hipSuccess) return st;
  unsigned grid = grid8(max_tiles(d) * C::SUB * (d.F / (C::BN / 2)));
  hipLaunchKernelGGL((k_gate_up<C, GATHER>), dim3(grid), dim3(C::NT), lds_bytes, s,
                     static_cast<const bf16_t*>(xs), sorted_flat, int(d.K), static_cast<const bf16_t*>(wg),
                     static_cast<const bf16_t*>(wu), tiles, num_tiles, static_cast<bf16_t*>(g),
                     static_cast<bf16_t*>(u), static_cast<bf16_t*>(a), int(d.H), int(d.F), group_rows(d, C::BM));
  return hipGetLastError();
}

// sorted_flat non-null: xs is x and the rows are gathered on load
hipError_t ffn_gate_up_big(const Dims& d, const void* xs, const int32_t* sorted_flat, const void* wg, const void* wu,
                           const int32_t* tiles, const int32_t* num_tiles, void* g, void* u, void* a, hipStream_t s) {
  return sorted_flat ? gate_up_t<Big8, true>(d, xs, sorted_flat, wg, wu, tiles, num_tiles, g, u, a, s)
                     : gate_up_t<Big8>(d, xs, nullptr, wg, wu, tiles, num_tiles, g, u, a, s);
}

template <class C>
static hipError_t down_t(const Dims& d, const void* a, const void* wd, const int32_t* tiles, const int32_t* num_tiles,
                         void* ys, hipStream_t s) {
  constexpr int lds_bytes = lds_bytes_of<C>();
  hipError_t st = allow_lds<k_down<C>>(lds_bytes);
  if (st != hipSuccess) return st;
  unsigned grid = grid8(max_tiles(d) * C::SUB * ((d.H + C::BN - 1) / C::BN));
  hipLaunchKernelGGL(k_down<C>, dim3(grid), dim3(C::NT), lds_bytes, s, static_cast<const bf16_t*>(a),
                     static_cast<const bf16_t*>(wd), tiles, num_tiles, static_cast<bf16_t*>(ys), int(d.H), int(d.F),
                     group_rows(d, C::BM));
  return hipGetLastError();
}

hipError_t ffn_down_big(const Dims& d, const void* a, const void* wd, const int32_t* tiles, const int32_t* num_tiles,
                         void* ys, hipStream_t s) {
  return down_t<Big8>(d, a, wd, tiles, num_tiles, ys, s);
}

template <class C>
static hipError_t dact_t(const Dims& d, const void* dys, const void* wd, const void* g, const void* u,
                         const int32_t* tiles, const int32_t* num_tiles, void* dg, void* du, hipStream_t s) {
  hipError_t st = allow_lds<k_dact<C>>(lds_bytes_of<C>());
  if (st != hipSuccess) return st;
  unsigned grid = grid8(max_tiles(d) * C::SUB * ((d.F + C::BN - 1) / C::BN));
  hipLaunchKernelGGL(k_dact<C>, dim3(grid), dim3(C::NT), lds_bytes_of<C>(), s, static_cast<const bf16_t*>(dys),
                     static_cast<const bf16_t*>(wd), static_cast<const bf16_t*>(g), static_cast<const bf16_t*>(u),
                     tiles, num_tiles, static_cast<bf16_t*>(dg), static_cast<bf16_t*>(du), int(d.H), int(d.F),
                     group_rows(d, C::BM));
  return hipGetLastError();
}

hipError_t ffn_bwd_dact_big(const Dims& d, const void* dys, const void* wd, const void* g, const void* u,
                             const int32_t* tiles, const int32_t* num_tiles, void* dg, void* du, hipStream_t s) {
  return dact_t<Big8>(d, dys, wd, g, u, tiles, num_tiles, dg, du, s);
}

hipError_t ffn_bwd_dact_mid(const Dims& d, const void* dys, const void* wd, const void* g, const void* u,
                            const int32_t* tiles, const int32_t* num_tiles, void* dg, void* du, hipStream_t s) {
  return dact_t<Mid>(d, dys, wd, g, u, tiles, num_tiles, dg, du, s);
}

template <class C>
static hipError_t dx_t(const Dims& d, const void* dg, const void* du, const void* wg, const void* wu,
                       const int32_t* tiles, const int32_t* num_tiles, void* dxs, hipStream_t s) {
  hipError_t st = allow_lds<k_dx<C>>(lds_bytes_of<C>());
  if (st != hipSuccess) return st;
  unsigned grid = grid8(max_tiles(d) * C::SUB * ((d.H + C::BN - 1) / C::BN));
  hipLaunchKernelGGL(k_dx<C>, dim3(grid), dim3(C::NT), lds_bytes_of<C>(), s, static_cast<const bf16_t*>(dg),
                     static_cast<const bf16_t*>(du), static_cast<const bf16_t*>(wg), static_cast<const bf16_t*>(wu),
                     tiles, num_tiles, static_cast<bf16_t*>(dxs), int(d.H), int(d.F), group_rows(d, C::BM));
  return hipGetLastError();
}

hipError_t ffn_bwd_dx_big(const Dims& d, const void* dg, const void* du, const void* wg, const void* wu,
                           const int32_t* tiles, const int32_t* num_tiles, void* dxs, hipStream_t s) {
  return dx_t<Big8>(d, dg, du, wg, wu, tiles, num_tiles, dxs, s);
}

// workgroups of a weight-gradient launch: E experts x (two H x F problems +
// one F x H), rounded up to whole XCD windows
template <class C>
static unsigned dw_grid(const Dims& d) {
  const int64_t tpe = ((d.H + C::BM - 1) / C::BM) * ((d.F + C::BN - 1) / C::BN);
  const int64_t tpe2 = ((d.F + C::BM - 1) / C::BM) * ((d.H + C::BN - 1) / C::BN);
  const int64_t total = d.E * (2 * tpe + tpe2);
  const int64_t win = 8 * dw_run(total);
  return unsigned((total + win - 1) / win * win);
}

// sorted_flat non-null: xs is x and dW_gate / dW_up gather their rows
template <class C>
static hipError_t dw_t(const Dims& d, const void* xs, const int32_t* sorted_flat, const void* a, const void* dys,
                       const void* dg, const void* du, const int32_t* offsets, float* dwg, float* dwu, float* dwd,
                       hipStream_t s) {
  auto run = [&](auto gather) -> hipError_t {
    constexpr bool G = decltype(gather)::value;
    hipError_t st = allow_lds<k_dw<C, G>>(lds_bytes_of<C>());
    if (st != hipSuccess) return st;
    const unsigned grid = dw_grid<C>(d);
    hipLaunchKernelGGL((k_dw<C, G>), dim3(grid), dim3(C::NT), lds_bytes_of<C>(), s, static_cast<const bf16_t*>(xs),
                       static_cast<const bf16_t*>(a), static_cast<const bf16_t*>(dys),
                       static_cast<const bf16_t*>(dg), static_cast<const bf16_t*>(du), offsets, dwg, dwu, dwd,
                       int(d.H), int(d.F), int(d.E), sorted_flat, int(d.K));
    return hipGetLastError();
  };
  return sorted_flat ? run(std::true_type{}) : run(std::false_type{});
}

hipError_t ffn_bwd_dw_big(const Dims& d, const void* xs, const int32_t* sorted_flat, const void* a, const void* dys,
                          const void* dg, const void* du, const int32_t* offsets, float* dwg, float* dwu, float* dwd,
                          hipStream_t s) {
  return dw_t<Big8>(d, xs, sorted_flat, a, dys, dg, du, offsets, dwg, dwu, dwd, s);
}

hipError_t ffn_bwd_dx_dw_big(const Dims& d, const void* dg, const void* du, const void* wg, const void* wu,
                             const int32_t* tiles, const int32_t* num_tiles, void* dxs, const void* xs,
                             const int32_t* sorted_flat, const void* a, const void* dys, const int32_t* offsets,
                             float* dwg, float* dwu, float* dwd, hipStream_t s) {
  using CW = Big8;
  using CX = DxInMerged;
  constexpr int lds_bytes = lds_bytes_of<CW>() > lds_bytes_of<CX>() ? lds_bytes_of<CW>() : lds_bytes_of<CX>();
  auto run = [&](auto gather) -> hipError_t {
    constexpr bool G = decltype(gather)::value;
    hipError_t st = allow_lds<k_dx_dw<CW, CX, G>>(lds_bytes);
    if (st != hipSuccess) return st;
    const unsigned gw = dw_grid<CW>(d);
    const unsigned gx = grid8(max_tiles(d) * CX::SUB * ((d.H + CX::BN - 1) / CX::BN));
    hipLaunchKernelGGL((k_dx_dw<CW, CX, G>), dim3(gw + gx), dim3(CW::NT), lds_bytes, s,
                       static_cast<const bf16_t*>(dg), static_cast<const bf16_t*>(du), static_cast<const bf16_t*>(wg),
                       static_cast<const bf16_t*>(wu), tiles, num_tiles, static_cast<bf16_t*>(dxs),
                       static_cast<const bf16_t*>(xs), static_cast<const bf16_t*>(a), static_cast<const bf16_t*>(dys),
                       offsets, dwg, dwu, dwd, int(d.H), int(d.F), int(d.E), int(gw), int(gx), sorted_flat,
                       int(d.K), group_rows(d, CX::BM));
    return hipGetLastError();
  };
  return sorted_flat ? run(std::true_type{}) : run(std::false_type{});
}

// 128 x 256 register-staged tiles
hipError_t ffn_gate_up_midr(const Dims& d, const void* xs, const int32_t* sorted_flat, const void* wg,
                            const void* wu, const int32_t* tiles, const int32_t* num_tiles, void* g, void* u, void* a,
                            hipStream_t s) {
  return sorted_flat ? gate_up_t<MidR, true>(d, xs, sorted_flat, wg, wu, tiles, num_tiles, g, u, a, s)
                     : gate_up_t<MidR>(d, xs, nullptr, wg, wu, tiles, num_tiles, g, u, a, s);
}
hipError_t ffn_down_midr(const Dims& d, const void* a, const void* wd, const int32_t* tiles, const int32_t* num_tiles,
                         void* ys, hipStream_t s) {
  return down_t<MidR>(d, a, wd, tiles, num_tiles, ys, s);
}
hipError_t ffn_gate_up_smallr(const Dims& d, const void* xs, const int32_t* sorted_flat, const void* wg,
                              const void* wu, const int32_t* tiles, const int32_t* num_tiles, void* g, void* u,
                              void* a, hipStream_t s) {
  return sorted_flat ? gate_up_t<SmallR32, true>(d, xs, sorted_flat, wg, wu, tiles, num_tiles, g, u, a, s)
                     : gate_up_t<SmallR32>(d, xs, nullptr, wg, wu, tiles, num_tiles, g, u, a, s);
}
hipError_t ffn_down_smallr(const Dims& d, const void* a, const void* wd, const int32_t* tiles,
                           const int32_t* num_tiles, void* ys, hipStream_t s) {
  return down_t<SmallR64>(d, a, wd, tiles, num_tiles, ys, s);
}
hipError_t ffn_bwd_dact_midr(const Dims& d, const void* dys, const void* wd, const void* g, const void* u,
                             const int32_t* tiles, const int32_t* num_tiles, void* dg, void* du, hipStream_t s) {
  return dact_t<MidR>(d, dys, wd, g, u, tiles, num_tiles, dg, du, s);
}
hipError_t ffn_bwd_dx_midr(const Dims& d, const void* dg, const void* du, const void* wg, const void* wu,
                           const int32_t* tiles, const int32_t* num_tiles, void* dxs, hipStream_t s) {
  return dx_t<MidR>(d, dg, du, wg, wu, tiles, num_tiles, dxs, s);
}
hipError_t ffn_bwd_dw_midr(const Dims& d, const void* xs, const int32_t* sorted_flat, const void* a, const void* dys,
                           const void* dg, const void* du, const int32_t* offsets, float* dwg, float* dwu, float* dwd,
                           hipStream_t s) {
  return dw_t<MidR>(d, xs, sorted_flat, a, dys, dg, du, offsets, dwg, dwu, dwd, s);
}

}  // namespace moe_launch
