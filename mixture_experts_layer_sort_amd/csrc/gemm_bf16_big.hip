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
// Workgroup tile 256 x 256, K step 64, 8 waves in a 4 x 2 arrangement, 64 x
// 128 per wave.  A 256 x 256 x 64 step moves 64 KB from L2 for 8.4 MFLOP.
// Used for the long contractions; gemm_bf16_small.hip holds the 128 x 128
// shape for small problems.
// Operands go from global memory straight into LDS with the gfx950 LDS DMA
// (16 bytes per lane, no register staging) into two stages: while the block
// multiplies one K tile the DMA of the next one is in flight.  A K-contiguous
// operand (token rows; weight rows in the backward) lands as [rows][64 k] and
// is read with 16-byte fragment loads; an MN-contiguous operand (the weights
// in the forward, both operands of the weight gradients) lands as
// [64 k][columns] and is read with the transposing LDS load
// (ds_read_b64_tr_b16), so no operand is ever transposed in registers.  Both
// layouts XOR-swizzle 16-byte chunks by row so the fragment reads are free of
// bank conflicts.  Output tiles leave through LDS with 16-byte row stores.
//
// Tails: N (and, for the weight gradients, M) may end on a 128 boundary
// inside a tile; loads past the end read clamped in-bounds positions whose
// results are never stored, and the ragged contraction tail of the weight
// gradients is zeroed in LDS.
//
// Determinism: every output element has exactly one owning workgroup and its
// K loop runs in ascending order.
#include "common.h"

namespace {
using namespace moe;

template <int BM_, int BN_, int WM_, int WN_, int MINB_, int BK_, int S_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int MINB = MINB_;  // workgroups per CU the registers must allow
  static constexpr int BK = BK_;      // K depth of one pipeline stage (32 or 64)
  static constexpr int S = S_;        // pipeline stages in LDS
  static constexpr int NW = WM * WN, NT = 64 * NW;
  static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  static constexpr int FM = TM / 32, FN = TN / 32;  // 32 x 32 fragments per wave
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int DPT = STAGE / 1024 / NW;              // LDS DMA instructions per stage and wave
  static constexpr int OP_BYTES = S * STAGE;
  static constexpr int PITCH = BN + 8;                       // bf16 per staged output row
  static constexpr int EPI_BYTES = BM * PITCH * 2;
  static constexpr int DACT_BYTES = 2 * TM * PITCH * 2;      // G and U rows of one wave row
  static constexpr int LDS_A = OP_BYTES > EPI_BYTES ? OP_BYTES : EPI_BYTES;
  static constexpr int LDS = LDS_A > DACT_BYTES ? LDS_A : DACT_BYTES;
  static constexpr int SUB = MOE_TILE_M / BM;  // workgroup row tiles per list tile
  static_assert(STAGE % (1024 * NW) == 0, "every wave issues the same number of DMA instructions");
  static_assert(BK == 32 || BK == 64, "stage depth");
};
using Big = TileCfg<256, 256, 4, 2, 1, 64, 2>;  // 8 waves, 64 x 128 per wave
static_assert(MOE_TILE_M % Big::BM == 0, "list tiles split into row tiles");

#define LDS_AS __attribute__((address_space(3)))
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef short v8s_t __attribute__((ext_vector_type(8)));

// 16 bytes per lane from global memory straight into LDS: the wave's 64
// lanes fill lds_wave[0 .. 1024) in lane order (gfx950 LDS DMA).
__device__ __forceinline__ void dma16(const bf16_t* g, char* lds_wave) {
  __builtin_amdgcn_global_load_lds(g, (LDS_AS void*)lds_wave, 16, 0, 0);
}

// s_waitcnt with vmcnt(n) and the other counters free (gfx9 encoding:
// vmcnt[3:0] at bits 3:0 and vmcnt[5:4] at bits 15:14, expcnt bits 6:4,
// lgkmcnt bits 11:8).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---- K-contiguous tile: ROWS rows x BK k, 2*BK bytes per row.  16-byte chunk
// c of row r sits at physical chunk c ^ fk(r), so the MFMA fragment reads (16
// consecutive rows, one chunk, per 16-lane phase) hit 16 different 16-byte
// bank slots.
template <int BK>
__device__ __forceinline__ int fk(int row) {
  return BK == 64 ? ((row ^ (row >> 3)) & 7) : ((row >> 2) & 3);
}

// Issue the DMA of rows [0, ROWS) x k [0, BK) of a row-major matrix (k
// contiguous, leading dimension ld).  Rows at or past rows_valid read row
// rows_valid - 1 instead (their results are never stored).
template <int ROWS, int BK, int NW>
__device__ __forceinline__ void dma_kc(char* stage, const bf16_t* base, int64_t ld, int rows_valid) {
  constexpr int CPR = BK / 8, RPI = 1024 / (2 * BK);  // chunks per row, rows per wave instruction
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int i = w; i < ROWS / RPI; i += NW) {
    const int row = i * RPI + lane / CPR;
    const int c = (lane % CPR) ^ fk<BK>(row);
    const int rs = row < rows_valid ? row : rows_valid - 1;
    dma16(base + (int64_t)rs * ld + c * 8, stage + i * 1024);
  }
}

// MFMA operand fragment from a K-contiguous tile: lane l holds row
// rbase + l%32, k = kk*16 + 8*(l/32) .. +7.
template <int BK>
__device__ __forceinline__ bf16x8_t frag_kc(const char* stage, int rbase, int kk) {
  const int lane = lane_id();
  const int row = rbase + (lane & 31);
  const int c = kk * 2 + (lane >> 5);
  return *reinterpret_cast<const bf16x8_t*>(stage + row * (2 * BK) + ((c ^ fk<BK>(row)) << 4));
}

// ---- MN-contiguous tile: BK k-rows x COLS columns, COLS*2 bytes per row.
// 16-byte chunk c of row k sits at physical chunk c ^ fm(k), which makes the
// transposing fragment reads (4 rows x 64 bytes per 32 lanes) conflict-free.
__device__ __forceinline__ int fm(int k) { return 4 * (k & 3); }

// Issue the DMA of k [0, BK) x columns [0, COLS) of a row-major matrix
// (columns contiguous, leading dimension ld).  Columns [0, split) come from
// base0 and [split, COLS) from base1 (both indexed by the tile column).  k
// rows at or past k_valid and columns at or past cols_valid read clamped
// positions (the caller zeroes or discards them).
template <int COLS, int BK, int NW>
__device__ __forceinline__ void dma_mn(char* stage, const bf16_t* base0, const bf16_t* base1, int split, int64_t ld,
                                       int k_valid, int cols_valid) {
  constexpr int CPR = COLS / 8, RPI = 1024 / (COLS * 2);  // chunks per row, rows per wave instruction
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int i = w; i < BK / RPI; i += NW) {
    const int k = i * RPI + lane / CPR;
    const int c = (lane % CPR) ^ fm(k);
    const int ks = k < k_valid ? k : k_valid - 1;
    const int cs = c * 8 < cols_valid ? c : (cols_valid >> 3) - 1;
    const bf16_t* b = cs * 8 < split ? base0 : base1;
    dma16(b + (int64_t)ks * ld + cs * 8, stage + i * 1024);
  }
}

// MFMA operand fragment from an MN-contiguous tile with two transposing LDS
// reads (ds_read_b64_tr_b16): within each 16-lane group, input lane j points
// at 4 columns of row k0 + j/4 and output lane i receives the 4 k values of
// one column.  Lane l ends up with column nbase + l%32, k = kk*16 + 8*(l/32)
// .. +7, the same k order as frag_kc.
template <int COLS>
__device__ __forceinline__ bf16x8_t frag_mn(const char* stage, int nbase, int kk) {
  constexpr int ROWB = COLS * 2;
  const int lane = lane_id();
  const int g = lane >> 4, i = lane & 15;
  const int col = nbase + 16 * (g & 1) + 4 * (i & 3);
  const int k0 = kk * 16 + 8 * (g >> 1) + (i >> 2);
  const char* p0 = stage + k0 * ROWB + (((col >> 3) ^ fm(k0)) << 4) + (col & 7) * 2;
  const char* p1 = stage + (k0 + 4) * ROWB + (((col >> 3) ^ fm(k0 + 4)) << 4) + (col & 7) * 2;
  const v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s_t*)p0);
  const v4s_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s_t*)p1);
  const v8s_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

template <class C>
struct Acc {
  f32x16_t a[C::FM][C::FN];
};

template <class C>
__device__ __forceinline__ void zero_acc(Acc<C>& acc) {
#pragma unroll
  for (int mi = 0; mi < C::FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < C::FN; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.a[mi][ni][r] = 0.f;
}

// One stage (BK deep) of the wave tile: acc[mi][ni] += A . B^T, with each
// operand read as K-contiguous (ds_read_b128) or MN-contiguous (transposing
// reads) fragments.  The fragments of k step kk+1 are requested before the
// MFMAs of step kk are issued, so LDS latency overlaps the matrix cores.
template <class C, bool A_MN, bool B_MN>
__device__ __forceinline__ void load_frags(const char* sa, const char* sb, int kk, int wm, int wn,
                                           bf16x8_t (&a)[C::FM], bf16x8_t (&b)[C::FN]) {
#pragma unroll
  for (int mi = 0; mi < C::FM; ++mi)
    a[mi] = A_MN ? frag_mn<C::BM>(sa, wm * C::TM + mi * 32, kk) : frag_kc<C::BK>(sa, wm * C::TM + mi * 32, kk);
#pragma unroll
  for (int ni = 0; ni < C::FN; ++ni)
    b[ni] = B_MN ? frag_mn<C::BN>(sb, wn * C::TN + ni * 32, kk) : frag_kc<C::BK>(sb, wn * C::TN + ni * 32, kk);
}

template <class C, bool A_MN, bool B_MN>
__device__ __forceinline__ void mma_stage(const char* sa, const char* sb, Acc<C>& acc, int wm, int wn) {
  constexpr int KK = C::BK / 16;
  bf16x8_t a[2][C::FM], b[2][C::FN];
  load_frags<C, A_MN, B_MN>(sa, sb, 0, wm, wn, a[0], b[0]);
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const int cur = kk & 1;
    if (kk + 1 < KK) load_frags<C, A_MN, B_MN>(sa, sb, kk + 1, wm, wn, a[cur ^ 1], b[cur ^ 1]);
#pragma unroll
    for (int mi = 0; mi < C::FM; ++mi)
#pragma unroll
      for (int ni = 0; ni < C::FN; ++ni)
        acc.a[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][mi], b[cur][ni], acc.a[mi][ni], 0, 0, 0);
  }
}

// S-stage K loop.  ia(kt, stage) / ib(kt, stage) issue the LDS DMA of K tile
// kt.  Tiles 0 .. S-2 are issued up front; at step kt every wave waits until
// its own DMA of tile kt has landed (tiles kt+1 .. kt+S-2 stay in flight),
// the barrier makes tile kt visible to all waves and retires step kt-1's
// reads of the stage tile kt+S-1 now reuses, the DMA of tile kt+S-1 starts
// and the block multiplies tile kt.  When the last tile holds only k_last
// valid k rows (weight gradients), rows k_last.. of its A stage (an MN tile)
// are zeroed before it is used.
template <class C, bool A_MN, bool B_MN, class IA, class IB>
__device__ __forceinline__ void k_loop(char* lds, Acc<C>& acc, int nk, IA ia, IB ib, int wm, int wn,
                                       int k_last = C::BK) {
  zero_acc(acc);
  if (nk <= 0) return;
#pragma unroll
  for (int s = 0; s < C::S - 1; ++s)
    if (s < nk) {
      ia(s, lds + s * C::STAGE);
      ib(s, lds + s * C::STAGE + C::A_BYTES);
    }
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + C::S - 2 < nk)
      wait_vm<C::DPT * (C::S - 2)>();
    else
      wait_vm<0>();
    __syncthreads();
    const int nxt = kt + C::S - 1;
    if (nxt < nk) {
      char* st = lds + (nxt % C::S) * C::STAGE;
      ia(nxt, st);
      ib(nxt, st + C::A_BYTES);
    }
    char* cur = lds + (kt % C::S) * C::STAGE;
    if (A_MN && kt == nk - 1 && k_last < C::BK) {
      constexpr int ROWB = C::BM * 2;
      uint4* z = reinterpret_cast<uint4*>(cur + k_last * ROWB);
      for (int i = threadIdx.x; i < (C::BK - k_last) * ROWB / 16; i += C::NT) z[i] = make_uint4(0, 0, 0, 0);
      __syncthreads();
    }
    mma_stage<C, A_MN, B_MN>(cur, cur + C::A_BYTES, acc, wm, wn);
  }
  __syncthreads();
}

// Accumulator element r of fragment (mi, ni): MFMA 32x32 result layout
// (column = lane % 32, rows in groups of 4 interleaved across the two lane
// halves).  Offsets within the wave tile are compile-time constants added to
// one per-lane base.
__device__ __forceinline__ constexpr int frag_row(int mi, int r) { return mi * 32 + (r >> 2) * 8 + (r & 3); }
template <class C>
__device__ __forceinline__ int lane_row(int wm) { return wm * C::TM + (lane_id() >> 5) * 4; }
template <class C>
__device__ __forceinline__ int lane_col(int wn) { return wn * C::TN + (lane_id() & 31); }

// staged tile <- bf16(acc)
template <class C>
__device__ __forceinline__ void epi_put(bf16_t* stg, const Acc<C>& acc, int wm, int wn) {
  bf16_t* p = stg + lane_row<C>(wm) * C::PITCH + lane_col<C>(wn);
#pragma unroll
  for (int mi = 0; mi < C::FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < C::FN; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) p[frag_row(mi, r) * C::PITCH + ni * 32] = f32_to_bf16(acc.a[mi][ni][r]);
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
// a group the row tile varies fastest, so the ~32 workgroups an XCD runs at
// once cover a patch of kGroupM row tiles x 32/kGroupM n tiles and each
// weight tile and each activation tile is fetched from HBM once per patch.
constexpr int kGroupM = 8;
__device__ __forceinline__ void grouped(int L, int nrow, int ncol, int& row, int& col) {
  const int per_group = kGroupM * ncol;
  const int g = L / per_group, r = L % per_group;
  const int first = g * kGroupM;
  const int gm = min(kGroupM, nrow - first);
  row = first + r % gm;
  col = r / gm;
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
template <class C>
__global__ __launch_bounds__(C::NT, C::MINB) void k_gate_up(const bf16_t* __restrict__ xs, const bf16_t* __restrict__ wg,
                                                   const bf16_t* __restrict__ wu, const int32_t* __restrict__ tiles,
                                                   const int32_t* __restrict__ num_tiles, bf16_t* __restrict__ g_out,
                                                   bf16_t* __restrict__ u_out, bf16_t* __restrict__ a_out, int H,
                                                   int F) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr int HALF = C::BN / 2;
  const int ntn = F / HALF;
  const int nrow = *num_tiles * C::SUB;
  const int L = xcd_block(nrow * ntn);
  if (L < 0) return;
  int rt, nt;
  grouped(L, nrow, ntn, rt, nt);
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
  k_loop<C, false, true>(
      lds, acc, H / C::BK,
      [&](int kt, char* st) { dma_kc<C::BM, C::BK, C::NW>(st, a_base + kt * C::BK, H, ti.rows); },
      [&](int kt, char* st) {
        dma_mn<C::BN, C::BK, C::NW>(st, b_g + (int64_t)kt * C::BK * F, b_u + (int64_t)kt * C::BK * F, HALF, F, C::BK, C::BN);
      },
      wm, wn);

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
      aw[i] = uint32_t(f32_to_bf16(silu_f32(g0) * u0)) | (uint32_t(f32_to_bf16(silu_f32(g1) * u1)) << 16);
    }
    *reinterpret_cast<uint4*>(a_out + o) = make_uint4(aw[0], aw[1], aw[2], aw[3]);
  }
}

// ys = A.W_down[e]
template <class C>
__global__ __launch_bounds__(C::NT, C::MINB) void k_down(const bf16_t* __restrict__ act, const bf16_t* __restrict__ wd,
                                                const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles,
                                                bf16_t* __restrict__ ys, int H, int F) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int ntn = (H + C::BN - 1) / C::BN;
  const int nrow = *num_tiles * C::SUB;
  const int L = xcd_block(nrow * ntn);
  if (L < 0) return;
  int rt, nt;
  grouped(L, nrow, ntn, rt, nt);
  const TileInfo ti = row_tile<C>(tiles, rt);
  if (ti.rows <= 0) return;
  const int ncols = min(C::BN, H - nt * C::BN);
  const int w = threadIdx.x >> 6, wm = w / C::WN, wn = w % C::WN;
  const bf16_t* a_base = act + (int64_t)ti.row0 * F;
  const bf16_t* b_base = wd + (int64_t)ti.e * F * H + nt * C::BN;
  Acc<C> acc;
  k_loop<C, false, true>(
      lds, acc, F / C::BK, [&](int kt, char* st) { dma_kc<C::BM, C::BK, C::NW>(st, a_base + kt * C::BK, F, ti.rows); },
      [&](int kt, char* st) {
        const bf16_t* b = b_base + (int64_t)kt * C::BK * H;
        dma_mn<C::BN, C::BK, C::NW>(st, b, b, C::BN, H, C::BK, ncols);
      },
      wm, wn);
  bf16_t* stg = reinterpret_cast<bf16_t*>(lds);
  epi_put<C>(stg, acc, wm, wn);
  __syncthreads();
  epi_store<C>(stg, ys + (int64_t)ti.row0 * H + nt * C::BN, H, ti.rows, ncols);
}

// --------------------------------------------------------------- backward

// dA = dys.W_down[e]^T; dG = dA*U*s*(1+G*(1-s)), dU = dA*G*s with s = sigmoid(G).
template <class C>
__global__ __launch_bounds__(C::NT, C::MINB) void k_dact(const bf16_t* __restrict__ dys, const bf16_t* __restrict__ wd,
                                                const bf16_t* __restrict__ g_in, const bf16_t* __restrict__ u_in,
                                                const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles,
                                                bf16_t* __restrict__ dg, bf16_t* __restrict__ du, int H, int F) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int ntn = (F + C::BN - 1) / C::BN;
  const int nrow = *num_tiles * C::SUB;
  const int L = xcd_block(nrow * ntn);
  if (L < 0) return;
  int rt, nt;
  grouped(L, nrow, ntn, rt, nt);
  const TileInfo ti = row_tile<C>(tiles, rt);
  if (ti.rows <= 0) return;
  const int ncols = min(C::BN, F - nt * C::BN);
  const int w = threadIdx.x >> 6, wm = w / C::WN, wn = w % C::WN;
  const bf16_t* a_base = dys + (int64_t)ti.row0 * H;
  // B[k = h][n = f] = W_down[e][f][h]: rows f of W_down[e] are k-contiguous
  const bf16_t* b_base = wd + (int64_t)ti.e * F * H + (int64_t)nt * C::BN * H;
  Acc<C> acc;
  k_loop<C, false, false>(
      lds, acc, H / C::BK, [&](int kt, char* st) { dma_kc<C::BM, C::BK, C::NW>(st, a_base + kt * C::BK, H, ti.rows); },
      [&](int kt, char* st) { dma_kc<C::BN, C::BK, C::NW>(st, b_base + kt * C::BK, H, ncols); }, wm, wn);

  // Epilogue one wave row (TM rows) at a time: the G and U rows are staged
  // side by side, the waves owning those rows turn them into dG and dU in
  // place (each lane owns its positions), and both are stored.
  bf16_t* stg_g = reinterpret_cast<bf16_t*>(lds);
  bf16_t* stg_u = stg_g + C::TM * C::PITCH;
  const int64_t obase = (int64_t)ti.row0 * F + nt * C::BN;
  const int lane_off = ((lane_id() >> 5) * 4) * C::PITCH + lane_col<C>(wn);
#pragma unroll
  for (int part = 0; part < C::WM; ++part) {
    const int rb = part * C::TM;
    const int nr = min(C::TM, ti.rows - rb);
    if (nr <= 0) break;
    epi_load<C>(stg_g, g_in + obase + (int64_t)rb * F, F, nr, ncols);
    epi_load<C>(stg_u, u_in + obase + (int64_t)rb * F, F, nr, ncols);
    __syncthreads();
    if (wm == part) {
      bf16_t* pg = stg_g + lane_off;
      bf16_t* pu = stg_u + lane_off;
#pragma unroll
      for (int mi = 0; mi < C::FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::FN; ++ni)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int o = frag_row(mi, r) * C::PITCH + ni * 32;
            const float gv = bf16_to_f32(pg[o]), uv = bf16_to_f32(pu[o]);
            const float sg = sigmoid_f32(gv);
            const float da = acc.a[mi][ni][r];
            pg[o] = f32_to_bf16(da * uv * sg * (1.f + gv * (1.f - sg)));
            pu[o] = f32_to_bf16(da * gv * sg);
          }
    }
    __syncthreads();
    epi_store<C>(stg_g, dg + obase + (int64_t)rb * F, F, nr, ncols);
    epi_store<C>(stg_u, du + obase + (int64_t)rb * F, F, nr, ncols);
    __syncthreads();
  }
}

// dxs = dG.W_gate[e]^T + dU.W_up[e]^T  (one K loop over 2F)
template <class C>
__global__ __launch_bounds__(C::NT, C::MINB) void k_dx(const bf16_t* __restrict__ dg, const bf16_t* __restrict__ du,
                                              const bf16_t* __restrict__ wg, const bf16_t* __restrict__ wu,
                                              const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles,
                                              bf16_t* __restrict__ dxs, int H, int F) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int ntn = (H + C::BN - 1) / C::BN;
  const int nrow = *num_tiles * C::SUB;
  const int L = xcd_block(nrow * ntn);
  if (L < 0) return;
  int rt, nt;
  grouped(L, nrow, ntn, rt, nt);
  const TileInfo ti = row_tile<C>(tiles, rt);
  if (ti.rows <= 0) return;
  const int ncols = min(C::BN, H - nt * C::BN);
  const int w = threadIdx.x >> 6, wm = w / C::WN, wn = w % C::WN;
  // B[k = f][n = h] = W[e][h][f]: rows h of W[e] are k-contiguous
  const int64_t woff = (int64_t)ti.e * H * F + (int64_t)nt * C::BN * F;
  const int nkf = F / C::BK;
  Acc<C> acc;
  k_loop<C, false, false>(
      lds, acc, 2 * nkf,
      [&](int kt, char* st) {
        const bool second = kt >= nkf;
        dma_kc<C::BM, C::BK, C::NW>(st, (second ? du : dg) + (int64_t)ti.row0 * F + (second ? kt - nkf : kt) * C::BK, F,
                             ti.rows);
      },
      [&](int kt, char* st) {
        const bool second = kt >= nkf;
        dma_kc<C::BN, C::BK, C::NW>(st, (second ? wu : wg) + woff + (second ? kt - nkf : kt) * C::BK, F, ncols);
      },
      wm, wn);
  bf16_t* stg = reinterpret_cast<bf16_t*>(lds);
  epi_put<C>(stg, acc, wm, wn);
  __syncthreads();
  epi_store<C>(stg, dxs + (int64_t)ti.row0 * H + nt * C::BN, H, ti.rows, ncols);
}

// Weight gradients, one workgroup per BM x BN output tile of one expert:
//   problem 0: dW_gate[e] = xs_e^T . dG_e   [H, F]
//   problem 1: dW_up[e]   = xs_e^T . dU_e   [H, F]
//   problem 2: dW_down[e] = A_e^T  . dys_e  [F, H]
// The contraction runs over the expert's rows in ascending 64-row steps;
// experts without rows write exact zeros.
template <class C>
__global__ __launch_bounds__(C::NT, C::MINB) void k_dw(const bf16_t* __restrict__ xs, const bf16_t* __restrict__ act,
                                              const bf16_t* __restrict__ dys, const bf16_t* __restrict__ dg,
                                              const bf16_t* __restrict__ du, const int32_t* __restrict__ offsets,
                                              float* __restrict__ dwg, float* __restrict__ dwu,
                                              float* __restrict__ dwd, int H, int F, int E) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int th = (H + C::BM - 1) / C::BM, tf = (F + C::BN - 1) / C::BN;
  const int th2 = (H + C::BN - 1) / C::BN, tf2 = (F + C::BM - 1) / C::BM;
  const int tpe = th * tf;  // output tiles per expert, problems 0 and 1 (== tf2 * th2 for square tiles)
  const int blk = xcd_block(3 * E * tpe);
  if (blk < 0) return;
  const int prob = blk / (E * tpe);
  const int rem = blk % (E * tpe);
  const int e = rem / tpe, t = rem % tpe;
  const bf16_t *Lm, *Rm;
  float* out;
  int P, Q, mt, nt;
  if (prob < 2) {
    P = H; Q = F;
    Lm = xs; Rm = (prob == 0) ? dg : du;
    out = ((prob == 0) ? dwg : dwu) + (int64_t)e * H * F;
    mt = t / tf; nt = t % tf;
  } else {
    P = F; Q = H;
    Lm = act; Rm = dys;
    out = dwd + (int64_t)e * F * H;
    mt = t / th2; nt = t % th2;
    (void)tf2;
  }
  const int prow = min(C::BM, P - mt * C::BM), qcol = min(C::BN, Q - nt * C::BN);
  const int w = threadIdx.x >> 6, wm = w / C::WN, wn = w % C::WN;
  const int r0 = offsets[e], cnt = offsets[e + 1] - r0;
  const bf16_t* l_base = Lm + (int64_t)r0 * P + mt * C::BM;
  const bf16_t* r_base = Rm + (int64_t)r0 * Q + nt * C::BN;
  Acc<C> acc;
  const int nk = (cnt + C::BK - 1) / C::BK;
  k_loop<C, true, true>(
      lds, acc, nk,
      [&](int kt, char* st) {
        const bf16_t* b = l_base + (int64_t)kt * C::BK * P;
        dma_mn<C::BM, C::BK, C::NW>(st, b, b, C::BM, P, cnt - kt * C::BK, prow);
      },
      [&](int kt, char* st) {
        const bf16_t* b = r_base + (int64_t)kt * C::BK * Q;
        dma_mn<C::BN, C::BK, C::NW>(st, b, b, C::BN, Q, cnt - kt * C::BK, qcol);
      },
      wm, wn, cnt - (nk - 1) * C::BK);
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

// Dynamic LDS above 64 KiB has to be enabled per kernel once.
template <typename Kern>
hipError_t allow_lds(Kern kernel, int bytes) {
  static hipError_t st =
      hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  return st;
}

}  // namespace

namespace moe_launch {

// grid size rounded up to whole XCD rounds
static unsigned grid8(int64_t n) { return unsigned((n + kXcds - 1) / kXcds * kXcds); }

template <class C>
static hipError_t gate_up_t(const Dims& d, const void* xs, const void* wg, const void* wu, const int32_t* tiles,
                            const int32_t* num_tiles, void* g, void* u, void* a, hipStream_t s) {
  hipError_t st = allow_lds(k_gate_up<C>, C::LDS);
  if (st != hipSuccess) return st;
  unsigned grid = grid8(max_tiles(d) * C::SUB * (d.F / (C::BN / 2)));
  hipLaunchKernelGGL(k_gate_up<C>, dim3(grid), dim3(C::NT), C::LDS, s, static_cast<const bf16_t*>(xs),
                     static_cast<const bf16_t*>(wg), static_cast<const bf16_t*>(wu), tiles, num_tiles,
                     static_cast<bf16_t*>(g), static_cast<bf16_t*>(u), static_cast<bf16_t*>(a), int(d.H), int(d.F));
  return hipGetLastError();
}

hipError_t ffn_gate_up_big(const Dims& d, const void* xs, const void* wg, const void* wu, const int32_t* tiles,
                            const int32_t* num_tiles, void* g, void* u, void* a, hipStream_t s) {
  return gate_up_t<Big>(d, xs, wg, wu, tiles, num_tiles, g, u, a, s);
}

template <class C>
static hipError_t down_t(const Dims& d, const void* a, const void* wd, const int32_t* tiles, const int32_t* num_tiles,
                         void* ys, hipStream_t s) {
  hipError_t st = allow_lds(k_down<C>, C::LDS);
  if (st != hipSuccess) return st;
  unsigned grid = grid8(max_tiles(d) * C::SUB * ((d.H + C::BN - 1) / C::BN));
  hipLaunchKernelGGL(k_down<C>, dim3(grid), dim3(C::NT), C::LDS, s, static_cast<const bf16_t*>(a),
                     static_cast<const bf16_t*>(wd), tiles, num_tiles, static_cast<bf16_t*>(ys), int(d.H), int(d.F));
  return hipGetLastError();
}

hipError_t ffn_down_big(const Dims& d, const void* a, const void* wd, const int32_t* tiles, const int32_t* num_tiles,
                         void* ys, hipStream_t s) {
  return down_t<Big>(d, a, wd, tiles, num_tiles, ys, s);
}

template <class C>
static hipError_t dact_t(const Dims& d, const void* dys, const void* wd, const void* g, const void* u,
                         const int32_t* tiles, const int32_t* num_tiles, void* dg, void* du, hipStream_t s) {
  hipError_t st = allow_lds(k_dact<C>, C::LDS);
  if (st != hipSuccess) return st;
  unsigned grid = grid8(max_tiles(d) * C::SUB * ((d.F + C::BN - 1) / C::BN));
  hipLaunchKernelGGL(k_dact<C>, dim3(grid), dim3(C::NT), C::LDS, s, static_cast<const bf16_t*>(dys),
                     static_cast<const bf16_t*>(wd), static_cast<const bf16_t*>(g), static_cast<const bf16_t*>(u),
                     tiles, num_tiles, static_cast<bf16_t*>(dg), static_cast<bf16_t*>(du), int(d.H), int(d.F));
  return hipGetLastError();
}

hipError_t ffn_bwd_dact_big(const Dims& d, const void* dys, const void* wd, const void* g, const void* u,
                             const int32_t* tiles, const int32_t* num_tiles, void* dg, void* du, hipStream_t s) {
  return dact_t<Big>(d, dys, wd, g, u, tiles, num_tiles, dg, du, s);
}

template <class C>
static hipError_t dx_t(const Dims& d, const void* dg, const void* du, const void* wg, const void* wu,
                       const int32_t* tiles, const int32_t* num_tiles, void* dxs, hipStream_t s) {
  hipError_t st = allow_lds(k_dx<C>, C::LDS);
  if (st != hipSuccess) return st;
  unsigned grid = grid8(max_tiles(d) * C::SUB * ((d.H + C::BN - 1) / C::BN));
  hipLaunchKernelGGL(k_dx<C>, dim3(grid), dim3(C::NT), C::LDS, s, static_cast<const bf16_t*>(dg),
                     static_cast<const bf16_t*>(du), static_cast<const bf16_t*>(wg), static_cast<const bf16_t*>(wu),
                     tiles, num_tiles, static_cast<bf16_t*>(dxs), int(d.H), int(d.F));
  return hipGetLastError();
}

hipError_t ffn_bwd_dx_big(const Dims& d, const void* dg, const void* du, const void* wg, const void* wu,
                           const int32_t* tiles, const int32_t* num_tiles, void* dxs, hipStream_t s) {
  return dx_t<Big>(d, dg, du, wg, wu, tiles, num_tiles, dxs, s);
}

template <class C>
static hipError_t dw_t(const Dims& d, const void* xs, const void* a, const void* dys, const void* dg, const void* du,
                       const int32_t* offsets, float* dwg, float* dwu, float* dwd, hipStream_t s) {
  hipError_t st = allow_lds(k_dw<C>, C::LDS);
  if (st != hipSuccess) return st;
  const int64_t tpe = ((d.H + C::BM - 1) / C::BM) * ((d.F + C::BN - 1) / C::BN);
  unsigned grid = grid8(3 * d.E * tpe);
  hipLaunchKernelGGL(k_dw<C>, dim3(grid), dim3(C::NT), C::LDS, s, static_cast<const bf16_t*>(xs),
                     static_cast<const bf16_t*>(a), static_cast<const bf16_t*>(dys), static_cast<const bf16_t*>(dg),
                     static_cast<const bf16_t*>(du), offsets, dwg, dwu, dwd, int(d.H), int(d.F), int(d.E));
  return hipGetLastError();
}

hipError_t ffn_bwd_dw_big(const Dims& d, const void* xs, const void* a, const void* dys, const void* dg,
                           const void* du, const int32_t* offsets, float* dwg, float* dwu, float* dwd, hipStream_t s) {
  return dw_t<Big>(d, xs, a, dys, dg, du, offsets, dwg, dwu, dwd, s);
}

}  // namespace moe_launch
