// MFMA tile machinery for gfx950 shared by the grouped GEMMs and the router:
// a workgroup tile configuration, operand tiles moved from global memory
// straight into LDS with the LDS DMA (global_load_lds, 16 bytes per lane),
// conflict-free XOR-swizzled LDS layouts for K-contiguous and MN-contiguous
// operands, MFMA fragment reads (16-byte loads, or the transposing
// ds_read_b64_tr_b16 for MN-contiguous operands), the S-stage K loop on
// v_mfma_f32_32x32x16_bf16 with float32 accumulation, and the accumulator
// layout of the 32 x 32 result fragments.
#pragma once
#include "common.h"

namespace moe_mma {
using namespace moe;

template <int BM_, int BN_, int WM_, int WN_, int MINB_, int BK_, int S_, bool REG_ = false>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr bool REG = REG_;   // register-staged K loop (k_loop_reg) instead of the LDS DMA (k_loop)
  static constexpr int MINB = MINB_;  // workgroups per CU the registers must allow
  static constexpr int BK = BK_;      // K depth of one pipeline stage (32 or 64)
  static constexpr int S = S_;        // pipeline stages in LDS
  static constexpr int NW = WM * WN, NT = 64 * NW;
  static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  static constexpr int FM = TM / 32, FN = TN / 32;  // 32 x 32 fragments per wave
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int DPT = STAGE / 1024 / NW;              // LDS DMA instructions per stage and wave
  static constexpr int JA = A_BYTES / 1024 / NW, JB = B_BYTES / 1024 / NW;  // ... of which A, B
  static constexpr int OP_BYTES = S * STAGE;
  static constexpr int PITCH = BN + 8;                       // bf16 per staged output row
  static constexpr int EPI_BYTES = BM * PITCH * 2;
  static constexpr int DACT_BYTES = TM * (BN + 4) * 4;       // float32 dA of one wave row
  static constexpr int LDS_A = OP_BYTES > EPI_BYTES ? OP_BYTES : EPI_BYTES;
  static constexpr int LDS = LDS_A > DACT_BYTES ? LDS_A : DACT_BYTES;
  static constexpr int SUB = MOE_TILE_M / BM;  // workgroup row tiles per list tile
  static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0,
                "every wave issues the same number of DMA instructions per operand");
  static_assert(BK == 32 || BK == 64, "stage depth");
};

#define LDS_AS __attribute__((address_space(3)))
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
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

// The wave's j-th LDS DMA instruction (instruction i = w + j * NW of the
// ROWS * 2 * BK / 1024 that move the tile) of rows [0, ROWS) x k [0, BK) of a
// row-major matrix (k contiguous, leading dimension ld).  Rows at or past
// rows_valid read row rows_valid - 1 instead (their results are never
// stored).
template <int ROWS, int BK, int NW>
__device__ __forceinline__ void dma_kc(char* stage, const bf16_t* base, int64_t ld, int rows_valid, int j) {
  constexpr int CPR = BK / 8, RPI = 1024 / (2 * BK);  // chunks per row, rows per wave instruction
  static_assert((ROWS / RPI) % NW == 0, "instructions split evenly over the waves");
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = w + j * NW;
  const int row = i * RPI + lane / CPR;
  const int c = (lane % CPR) ^ fk<BK>(row);
  const int rs = row < rows_valid ? row : rows_valid - 1;
  dma16(base + (int64_t)rs * ld + c * 8, stage + i * 1024);
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

// The wave's j-th LDS DMA instruction (instruction i = w + j * NW of the
// BK * COLS * 2 / 1024 that move the tile) of k [0, BK) x columns [0, COLS)
// of a row-major matrix (columns contiguous, leading dimension ld).  Columns
// [0, split) come from base0 and [split, COLS) from base1 (both indexed by
// the tile column).  k rows at or past k_valid and columns at or past
// cols_valid read clamped positions (the caller zeroes or discards them).
template <int COLS, int BK, int NW>
__device__ __forceinline__ void dma_mn(char* stage, const bf16_t* base0, const bf16_t* base1, int split, int64_t ld,
                                       int k_valid, int cols_valid, int j) {
  constexpr int CPR = COLS / 8, RPI = 1024 / (COLS * 2);  // chunks per row, rows per wave instruction
  static_assert((BK / RPI) % NW == 0, "instructions split evenly over the waves");
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = w + j * NW;
  const int k = i * RPI + lane / CPR;
  const int c = (lane % CPR) ^ fm(k);
  const int ks = k < k_valid ? k : k_valid - 1;
  const int cs = c * 8 < cols_valid ? c : (cols_valid >> 3) - 1;
  const bf16_t* b = cs * 8 < split ? base0 : base1;
  dma16(b + (int64_t)ks * ld + cs * 8, stage + i * 1024);
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

// Workgroup barrier without the memory fence of __syncthreads: with LDS DMA
// in flight that fence waits for all of it (vmcnt 0), which drains the later
// stages of the pipeline at every step.  The caller has waited for the DMA
// it needs; the LDS accesses before it complete first (lgkmcnt 0), and the
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt free
  asm volatile("s_barrier" ::: "memory");
}

// One step of the S-stage loop: the DMA of K tile nxt into stage wst (if
// issue) and the MFMAs over stage rst.  The stages are distinct (restrict),
// which lets the compiler keep its waits for LDS DMA per stage instead of
// waiting for every DMA in flight before the first fragment read.
template <class C, bool A_MN, bool B_MN, class IA, class IB>
__device__ __forceinline__ void dma_mma_step(char* __restrict__ wst, const char* __restrict__ rst, int nxt, bool issue,
                                             IA& ia, IB& ib, Acc<C>& acc, int wm, int wn) {
  if (issue) {
#pragma unroll
    for (int j = 0; j < C::JA; ++j) ia(nxt, wst, j);
#pragma unroll
    for (int j = 0; j < C::JB; ++j) ib(nxt, wst + C::A_BYTES, j);
  }
  mma_stage<C, A_MN, B_MN>(rst, rst + C::A_BYTES, acc, wm, wn);
}

// S-stage K loop.  ia(kt, stage, j) / ib(kt, stage, j) issue the wave's
// j-th LDS DMA instruction of K tile kt (j < C::JA resp. C::JB).  Tiles
// 0 .. S-2 are issued up front; at step kt every wave waits until its own DMA
// of tile kt has landed (tiles kt+1 .. kt+S-2 stay in flight), the barrier
// makes tile kt visible to all waves and retires step kt-1's reads of the
// stage tile kt+S-1 now reuses, the DMA of tile kt+S-1 starts and the block
// multiplies tile kt.  When the last tile holds
// only k_last valid k rows (weight gradients), rows k_last.. of its A stage
// (an MN tile) are zeroed before it is used.
template <class C, bool A_MN, bool B_MN, class IA, class IB>
__device__ __forceinline__ void k_loop(char* lds, Acc<C>& acc, int nk, IA ia, IB ib, int wm, int wn,
                                       int k_last = C::BK) {
  zero_acc(acc);
  if (nk <= 0) return;
#pragma unroll
  for (int s = 0; s < C::S - 1; ++s)
    if (s < nk) {
      char* st = lds + s * C::STAGE;
#pragma unroll
      for (int j = 0; j < C::JA; ++j) ia(s, st, j);
#pragma unroll
      for (int j = 0; j < C::JB; ++j) ib(s, st + C::A_BYTES, j);
    }
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + C::S - 2 < nk)
      wait_vm<C::DPT * (C::S - 2)>();
    else
      wait_vm<0>();
    lds_barrier();
    const int nxt = kt + C::S - 1;
    char* cur = lds + (kt % C::S) * C::STAGE;
    if (!(A_MN && kt == nk - 1 && k_last < C::BK)) {
      dma_mma_step<C, A_MN, B_MN>(lds + (nxt % C::S) * C::STAGE, cur, nxt, nxt < nk, ia, ib, acc, wm, wn);
      continue;
    }
    // last tile with k_last valid k rows (weight gradients; no DMA left to issue)
    {
      constexpr int ROWB = C::BM * 2;
      uint4* z = reinterpret_cast<uint4*>(cur + k_last * ROWB);
      for (int i = threadIdx.x; i < (C::BK - k_last) * ROWB / 16; i += C::NT) z[i] = make_uint4(0, 0, 0, 0);
      __syncthreads();
    }
    mma_stage<C, A_MN, B_MN>(cur, cur + C::A_BYTES, acc, wm, wn);
  }
  __syncthreads();
}

// ---- register-staged operand tiles (same LDS layouts as the DMA tiles)
//
// Thread t of the workgroup moves the 16-byte chunks q = t + i * NT of a
// tile: global memory -> registers (issued early, spread between MFMAs) ->
// LDS (after the MFMAs that read the other stage).

// K-contiguous operand: ROWS rows x BK k of a row-major matrix (leading
// dimension ld).  K tile kt starts at k = kt * BK of base0, or, from tile
// nk0 on, at k = (kt - nk0) * BK of base1 (two stacked contractions).  Rows
// at or past rows_valid read row rows_valid - 1 (results never stored).
template <int ROWS, int BK, int NT>
struct KcOp {
  static constexpr int CPR = BK / 8, RP = NT / CPR, N = ROWS / RP;
  static_assert(NT % CPR == 0 && ROWS % RP == 0, "chunks split evenly over the threads");
  const bf16_t *base0, *base1;  // the same address in every lane
  int nk0;
  int off[N];  // byte offset of chunk i within a K tile (ROWS * ld * 2 < 2^31)
  __device__ __forceinline__ KcOp(const bf16_t* b0, const bf16_t* b1, int nk0_, int64_t ld, int rows_valid)
      : base0(b0), base1(b1), nk0(nk0_) {
    const int r0 = threadIdx.x / CPR, c = threadIdx.x % CPR;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int r = r0 + i * RP;
      off[i] = int(((r < rows_valid ? r : rows_valid - 1) * ld + c * 8) * 2);
    }
  }
  // Through a buffer resource at the K tile's base: each chunk's address is
  // its 32-bit lane offset, with no per-row 64-bit add.  Every offset is in
  // bounds (rows clamped above), so the range check never applies.
  __device__ __forceinline__ void load(u32x4_t (&v)[N], int kt) const {
    const bf16_t* p = kt < nk0 ? base0 + kt * BK : base1 + (kt - nk0) * BK;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(p), (short)0, 0x7fffffff, 0x00020000);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, off[i], 0, 0);
  }
  __device__ __forceinline__ void store(const u32x4_t (&v)[N], char* st, int) const {
    const int r0 = threadIdx.x / CPR, c = threadIdx.x % CPR;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int r = r0 + i * RP;
      *reinterpret_cast<u32x4_t*>(st + r * (2 * BK) + ((c ^ fk<BK>(r)) << 4)) = v[i];
    }
  }
};

// K-contiguous operand whose rows are gathered: tile row r is row
// rows_src[r] / K of x (leading dimension ld), so the expert-grouped rows
// are read straight from the token rows (rows_src = the sorted flat indices
// of the tile's first row on).  Rows at or past rows_valid read the last
// valid row.  Element offsets are 32-bit (callers keep N * ld < 2^31).
template <int ROWS, int BK, int NT>
struct KcGather {
  static constexpr int CPR = BK / 8, RP = NT / CPR, N = ROWS / RP;
  static_assert(NT % CPR == 0 && ROWS % RP == 0, "chunks split evenly over the threads");
  const bf16_t* base;
  int off[N];
  __device__ __forceinline__ KcGather(const bf16_t* x, const int32_t* rows_src, int K, int64_t ld, int rows_valid)
      : base(x) {
    const int r0 = threadIdx.x / CPR, c = threadIdx.x % CPR;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int r = r0 + i * RP;
      const int tok = rows_src[r < rows_valid ? r : rows_valid - 1] / K;
      off[i] = int(tok * ld) + c * 8;
    }
  }
  // Through a buffer resource at the K tile's base: each chunk's address is
  // its 32-bit lane offset in bytes (N * ld * 2 < 2^32), with no 64-bit add
  // per chunk.  The resource spans 4 GiB and every offset is in bounds (rows
  // clamped above), so the range check never applies.  gate/up against plain
  // 64-bit loads: 7.31-7.33 -> 7.13-7.17 ms at H = 4096, F = 14336, 5.45 ->
  // 5.35 ms at H = 7168, E = 256, 1.28-1.30 -> 1.27 ms at H = 2048, E = 64.
  __device__ __forceinline__ void load(u32x4_t (&v)[N], int kt) const {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(base + kt * BK), (short)0,
                                                                       -1, 0x00020000);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, int(unsigned(off[i]) * 2u), 0, 0);
  }
  __device__ __forceinline__ void store(const u32x4_t (&v)[N], char* st, int) const {
    const int r0 = threadIdx.x / CPR, c = threadIdx.x % CPR;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int r = r0 + i * RP;
      *reinterpret_cast<u32x4_t*>(st + r * (2 * BK) + ((c ^ fk<BK>(r)) << 4)) = v[i];
    }
  }
};

// MN-contiguous operand: BK k rows x COLS columns of a row-major matrix
// (leading dimension ld); K tile kt covers k rows [kt * BK, kt * BK + BK),
// all of them valid (the contraction length is a multiple of BK).  Columns
// [0, split) come from base0 and [split, COLS) from base1 (both indexed by
// the tile column); columns at or past cols_valid read a clamped column
// (results discarded).  Each row's address is this thread's pointer plus a
// multiple of the (uniform) row stride.
template <int COLS, int BK, int NT>
struct MnOp {
  static constexpr int CPR = COLS / 8, KP = NT / CPR, N = BK / KP;
  static_assert(NT % CPR == 0 && BK % KP == 0, "chunks split evenly over the threads");
  const bf16_t* base;  // this thread's column, k row 0
  int64_t ld;
  __device__ __forceinline__ MnOp(const bf16_t* b0, const bf16_t* b1, int split, int64_t ld_, int cols_valid)
      : ld(ld_) {
    const int c = threadIdx.x % CPR;
    const int cs = c * 8 < cols_valid ? c : (cols_valid >> 3) - 1;
    base = (cs * 8 < split ? b0 : b1) + (int64_t)(threadIdx.x / CPR) * ld_ + cs * 8;
  }
  __device__ __forceinline__ void load(u32x4_t (&v)[N], int kt) const {
    const bf16_t* p = base + (int64_t)kt * BK * ld;
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = *reinterpret_cast<const u32x4_t*>(p + (int64_t)(i * KP) * ld);
  }
  __device__ __forceinline__ void store(const u32x4_t (&v)[N], char* st, int) const {
    const int k0 = threadIdx.x / CPR, c = threadIdx.x % CPR;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int k = k0 + i * KP;
      *reinterpret_cast<u32x4_t*>(st + k * (COLS * 2) + ((c ^ fm(k)) << 4)) = v[i];
    }
  }
};

// MN-contiguous operand of one source read through a buffer resource: BK k
// rows x COLS columns of a row-major slab (leading dimension ld) whose row 0,
// column 0 is `tile` (the same address in every lane).  The resource of K
// tile kt ends after its last valid k row, so rows past k_total read zeros
// from the hardware's range check and each row's address is one 32-bit add
// (no clamp, no 64-bit multiply per row).  Columns at or past cols_valid read
// a clamped column (results discarded).  Needs BK * ld * 2 < 2^31.
template <int COLS, int BK, int NT>
struct MnBuf {
  static constexpr int CPR = COLS / 8, KP = NT / CPR, N = BK / KP;
  static_assert(NT % CPR == 0 && BK % KP == 0, "chunks split evenly over the threads");
  const char* tile;
  int64_t ld;
  int k_total;
  int voff;      // this thread's byte offset in a K tile: first k row, column chunk
  int row_step;  // bytes between the k rows of one thread (KP rows)
  __device__ __forceinline__ MnBuf(const bf16_t* tile_, int64_t ld_, int cols_valid, int k_total_)
      : tile(reinterpret_cast<const char*>(tile_)), ld(ld_), k_total(k_total_) {
    const int c = threadIdx.x % CPR;
    const int cs = c * 8 < cols_valid ? c : (cols_valid >> 3) - 1;
    voff = int((threadIdx.x / CPR) * ld_ * 2) + cs * 16;
    row_step = int(KP * ld_ * 2);
  }
  __device__ __forceinline__ void load(u32x4_t (&v)[N], int kt) const {
    const int kv = k_total - kt * BK;  // valid k rows of the tile (at least one)
    const int rows = kv < BK ? kv : BK;
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(tile + (int64_t)kt * BK * ld * 2), (short)0, int(rows * ld * 2), 0x00020000);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, voff + i * row_step, 0, 0);
  }
  __device__ __forceinline__ void store(const u32x4_t (&v)[N], char* st, int) const {
    const int k0 = threadIdx.x / CPR, c = threadIdx.x % CPR;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int k = k0 + i * KP;
      *reinterpret_cast<u32x4_t*>(st + k * (COLS * 2) + ((c ^ fm(k)) << 4)) = v[i];
    }
  }
};

// MN-contiguous operand whose k rows are gathered: k row r of the
// contraction (r from 0 over the expert's rows) is token row rows_src[r] / K
// of x (leading dimension ld), so the weight gradients read x instead of the
// grouped copy of its rows.  Columns as in MnOp; k rows at or past k_total
// read the last valid row (k_loop_reg zeroes them in the A operand).
template <int COLS, int BK, int NT>
struct MnGather {
  static constexpr int CPR = COLS / 8, KP = NT / CPR, N = BK / KP;
  static_assert(NT % CPR == 0 && BK % KP == 0, "chunks split evenly over the threads");
  const bf16_t* base;  // x + this thread's column
  const int32_t* rows_src;
  int K;
  int64_t ld;
  int k_total;
  __device__ __forceinline__ MnGather(const bf16_t* x_cols, const int32_t* rows_src_, int K_, int64_t ld_,
                                      int cols_valid, int k_total_)
      : rows_src(rows_src_), K(K_), ld(ld_), k_total(k_total_) {
    const int c = threadIdx.x % CPR;
    const int cs = c * 8 < cols_valid ? c : (cols_valid >> 3) - 1;
    base = x_cols + cs * 8;
  }
  __device__ __forceinline__ void load(u32x4_t (&v)[N], int kt) const {
    const int k0 = threadIdx.x / CPR;
    const int kv = k_total - kt * BK;  // valid k rows of the tile
    int src[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int k = k0 + i * KP < kv ? k0 + i * KP : kv - 1;
      src[i] = rows_src[kt * BK + k] / K;
    }
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = *reinterpret_cast<const u32x4_t*>(base + (int64_t)src[i] * ld);
  }
  __device__ __forceinline__ void store(const u32x4_t (&v)[N], char* st, int) const {
    const int k0 = threadIdx.x / CPR, c = threadIdx.x % CPR;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int k = k0 + i * KP;
      *reinterpret_cast<u32x4_t*>(st + k * (COLS * 2) + ((c ^ fm(k)) << 4)) = v[i];
    }
  }
};

// Instruction order of one step of k_loop_reg (sched_group_barrier masks:
// 0x008 MFMA, 0x020 VMEM read, 0x100 LDS read, 0x200 LDS write).  The
// step's KK * MK MFMAs are the slots; after slot j come its share of
//   - the next k step's fragment reads (FR per k step, k steps 0..KK-2),
//   - the next K tile's global loads (GL, over the first LK k steps),
//   - the LDS stores of those loads (GL, over the last k step),
// each spread evenly over the slots it covers.  The first k step's fragment
// reads open the step.
template <int KK, int MK, int FR, int GL, int LK, int J = 0>
__device__ __forceinline__ void reg_step_schedule() {
  static_assert(LK >= 1 && LK <= KK, "loads spread over 1..KK k steps");
  if constexpr (J == 0) __builtin_amdgcn_sched_group_barrier(0x100, FR, 0);
  if constexpr (J < KK * MK) {
    constexpr int kk = J / MK, i = J % MK;
    constexpr int r = kk + 1 < KK ? (i + 1) * FR / MK - i * FR / MK : 0;
    constexpr int g = kk < LK ? (J + 1) * GL / (LK * MK) - J * GL / (LK * MK) : 0;
    constexpr int w = kk == KK - 1 ? (i + 1) * GL / MK - i * GL / MK : 0;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
    if constexpr (g > 0) __builtin_amdgcn_sched_group_barrier(0x020, g, 0);
    if constexpr (w > 0) __builtin_amdgcn_sched_group_barrier(0x200, w, 0);
    reg_step_schedule<KK, MK, FR, GL, LK, J + 1>();
  }
}

// Steps of the register-staged K loop (below).  MMA = false: a wave whose
// tile rows all lie past the tile's valid rows only moves its share of the
// operand chunks (its MFMAs and fragment reads would only make rows that are
// never stored); the barriers are the same, so the workgroup stays in step.
template <class C, bool A_MN, bool B_MN, bool MMA, class OA, class OB>
__device__ __forceinline__ void k_steps_reg(char* lds, Acc<C>& acc, int nk, const OA& oa, const OB& ob,
                                            u32x4_t (&va)[OA::N], u32x4_t (&vb)[OB::N], int wm, int wn,
                                            int k_last) {
  constexpr int KK = C::BK / 16;
  constexpr int FR = C::FM * (A_MN ? 2 : 1) + C::FN * (B_MN ? 2 : 1);  // LDS reads per k step
  constexpr int MK = C::FM * C::FN;                                    // MFMAs per k step
  constexpr int GL = OA::N + OB::N;                                    // chunks per thread and tile
  // k steps the next tile's loads are spread over: all in the first one with
  // two waves per SIMD (the other wave covers the burst; more time for the
  // loads to land: at H = 4096, F = 14336 merged dX/dW 17.64 -> 17.33 ms, dA
  // 4.70 -> 4.56, down 3.64 -> 3.57), the first half with one wave per SIMD
  // (gate/up 7.27 -> 7.42 ms when all in the first)
  constexpr int LOAD_STEPS = C::NW >= 8 ? 1 : (KK / 2 > 0 ? KK / 2 : 1);
  for (int kt = 0; kt < nk; ++kt) {
    char* cur = lds + (kt & 1) * C::STAGE;
    char* nxt = lds + ((kt + 1) & 1) * C::STAGE;
    const int kn = kt + 1 < nk ? kt + 1 : kt;
    if (A_MN && kt == nk - 1 && k_last < C::BK) {
      constexpr int ROWB = C::BM * 2;
      u32x4_t* z = reinterpret_cast<u32x4_t*>(cur + k_last * ROWB);
      for (int i = threadIdx.x; i < (C::BK - k_last) * ROWB / 16; i += C::NT) z[i] = u32x4_t{0u, 0u, 0u, 0u};
      __syncthreads();
    }
    if constexpr (MMA) {
      bf16x8_t fa[2][C::FM], fb[2][C::FN];
      load_frags<C, A_MN, B_MN>(cur, cur + C::A_BYTES, 0, wm, wn, fa[0], fb[0]);
      oa.load(va, kn);
      ob.load(vb, kn);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int cb = kk & 1;
        if (kk + 1 < KK) load_frags<C, A_MN, B_MN>(cur, cur + C::A_BYTES, kk + 1, wm, wn, fa[cb ^ 1], fb[cb ^ 1]);
#pragma unroll
        for (int mi = 0; mi < C::FM; ++mi)
#pragma unroll
          for (int ni = 0; ni < C::FN; ++ni)
            acc.a[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cb][mi], fb[cb][ni], acc.a[mi][ni], 0, 0, 0);
      }
      oa.store(va, nxt, kn);
      ob.store(vb, nxt + C::A_BYTES, kn);
      reg_step_schedule<KK, MK, FR, GL, LOAD_STEPS>();
    } else {
      oa.load(va, kn);
      ob.load(vb, kn);
      oa.store(va, nxt, kn);
      ob.store(vb, nxt + C::A_BYTES, kn);
    }
    __syncthreads();
  }
}

// Register-staged K loop over two LDS stages (KK = BK / 16 MFMA k steps per
// stage).  Each step: the k-step-0 fragments of the current stage are read,
// the next K tile's chunks are requested into registers, spread between the
// MFMAs of the first k step (8 waves) or the first half of the step (4), each later k step's fragments are
// read while the previous k step multiplies, the chunks go to the other
// stage between the last k step's MFMAs, and one barrier ends the step.  The
// last step reloads its own tile (in bounds, never read).  Spreading the
// requests keeps the wave's in-order issue from stalling its MFMAs behind a
// burst of loads.  When the last tile holds only k_last valid k rows (weight
// gradients), rows k_last.. of its A stage (an MN tile) are zeroed before it
// is used.  mma = false (wave-uniform): the wave's rows are all past the
// tile's valid rows, so it moves operand chunks only and its accumulators
// stay zero; with two waves per SIMD that halves the matrix-core work of a
// SIMD on a tile of at most half its rows (skewed routing, H = 2048,
// F = 1408, E = 64, where 36 of 64 experts have fewer than 128 rows: merged
// dX/dW 3.376-3.414 -> 3.345-3.356 ms; no change where few tiles are ragged).
template <class C, bool A_MN, bool B_MN, class OA, class OB>
__device__ __forceinline__ void k_loop_reg(char* lds, Acc<C>& acc, int nk, const OA& oa, const OB& ob, int wm,
                                           int wn, int k_last = C::BK, bool mma = true) {
  constexpr int KK = C::BK / 16;
  static_assert(C::S == 2 && KK >= 2 && KK % 2 == 0, "two stages, an even number of k steps per stage");
  zero_acc(acc);
  if (nk <= 0) return;
  u32x4_t va[OA::N], vb[OB::N];
  oa.load(va, 0);
  ob.load(vb, 0);
  oa.store(va, lds, 0);
  ob.store(vb, lds + C::A_BYTES, 0);
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(mma ? 1 : 0))
    k_steps_reg<C, A_MN, B_MN, true>(lds, acc, nk, oa, ob, va, vb, wm, wn, k_last);
  else
    k_steps_reg<C, A_MN, B_MN, false>(lds, acc, nk, oa, ob, va, vb, wm, wn, k_last);
}

// ---- LDS DMA through buffer resources, and the mixed-depth DMA K loop
//
// The 8-wave 256 x 256 tiles (gate/up, down, dA, dX and the weight gradients) move
// both operands by LDS DMA instead of through registers: operand A one K
// tile ahead into two LDS slots, operand B two K tiles ahead into three, so
// 96 KB per CU are in flight without a register holding any of it (the
// register-staged loop holds one 64 KB K tile, and a second register set
// does not fit beside 128 accumulators per lane).  Each request is a buffer
// load with a 32-bit lane offset fixed for the whole loop (the resource base
// moves per K tile): one instruction and an M0 write, against ten address
// instructions per request of the global-address LDS DMA.  Against the
// register-staged loop at N = 16384, H = 4096, F = 14336, E = 8: down 3.58 ->
// 3.46 ms, dA 3.99 -> 3.79 ms, merged dX / weight gradients 17.05 -> 16.27 ms
// (one box, interleaved runs).  gate/up runs it too, on 8 waves with B as two
// 128-column sub-tiles (one per weight tensor); with 4 waves (one per SIMD)
// the loop was slower than the register-staged one (7.04 -> 7.13 ms).
// LDS: A slots at [0, 2 * A_BYTES), B slots at [2 * A_BYTES, + 3 * B_BYTES).

// 16 bytes per lane from a buffer resource into LDS: the wave's lanes fill
// lds_wave[0 .. 1024) in lane order.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, int off, char* lds_wave) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS_AS void*)lds_wave, 16, off, 0, 0, 0);
}

// K-contiguous operand by DMA: ROWS rows x BK k of a row-major matrix
// (leading dimension ld) starting at base; K tile kt starts at k = kt * BK.
// Rows at or past rows_valid read row rows_valid - 1 (never stored).  Same
// LDS layout as dma_kc.  Byte offsets within a K tile must fit 31 bits.
template <int ROWS, int BK, int NW>
struct KcDma {
  static constexpr int CPR = BK / 8, RPI = 1024 / (2 * BK), J = ROWS / RPI / NW;
  static_assert((ROWS / RPI) % NW == 0, "instructions split evenly over the waves");
  const bf16_t *base0, *base1;  // K tiles from nk0 on come from base1 (two stacked contractions)
  int nk0;
  int off[J];
  __device__ __forceinline__ KcDma(const bf16_t* b0, const bf16_t* b1, int nk0_, int64_t ld, int rows_valid)
      : base0(b0), base1(b1), nk0(nk0_) {
    const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int row = (w + j * NW) * RPI + lane / CPR;
      const int c = (lane % CPR) ^ fk<BK>(row);
      const int rs = row < rows_valid ? row : rows_valid - 1;
      off[j] = int((rs * ld + c * 8) * 2);
    }
  }
  __device__ __forceinline__ KcDma(const bf16_t* b, int64_t ld, int rows_valid) : KcDma(b, b, 1 << 30, ld, rows_valid) {}
  __device__ __forceinline__ void issue(int kt, char* slot) const {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bf16_t* p = kt < nk0 ? base0 + kt * BK : base1 + (kt - nk0) * BK;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(p), (short)0, 0x7fffffff, 0x00020000);
#pragma unroll
    for (int j = 0; j < J; ++j) dma16_buf(r, off[j], slot + (w + j * NW) * 1024);
  }
};

// K-contiguous operand by DMA with gathered rows: tile row r is row
// rows_src[r] / K of x (leading dimension ld), as KcGather.  Byte offsets are
// 32-bit unsigned (callers keep x under 4 GiB).
template <int ROWS, int BK, int NW>
struct KcGatherDma {
  static constexpr int CPR = BK / 8, RPI = 1024 / (2 * BK), J = ROWS / RPI / NW;
  static_assert((ROWS / RPI) % NW == 0, "instructions split evenly over the waves");
  const bf16_t* base;
  unsigned off[J];
  __device__ __forceinline__ KcGatherDma(const bf16_t* x, const int32_t* rows_src, int K, int64_t ld, int rows_valid)
      : base(x) {
    const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int row = (w + j * NW) * RPI + lane / CPR;
      const int c = (lane % CPR) ^ fk<BK>(row);
      const int tok = rows_src[row < rows_valid ? row : rows_valid - 1] / K;
      off[j] = unsigned(tok * ld + c * 8) * 2u;
    }
  }
  __device__ __forceinline__ void issue(int kt, char* slot) const {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(base + kt * BK), (short)0, -1, 0x00020000);
#pragma unroll
    for (int j = 0; j < J; ++j) dma16_buf(r, int(off[j]), slot + (w + j * NW) * 1024);
  }
};

// MN-contiguous operand by DMA: BK k rows x COLS columns of a row-major slab
// (leading dimension ld) whose row 0, column 0 is tile; K tile kt covers k
// rows [kt * BK, kt * BK + BK) of which those below k_total are valid: the
// resource of a tile ends after its last valid row, so rows past it read
// zeros (k_loop_dma2 also zeroes them in LDS).  Columns at or past
// cols_valid read a clamped column (results discarded).  Same LDS layout as
// dma_mn.  Needs BK * ld * 2 < 2^31.
template <int COLS, int BK, int NW>
struct MnDma {
  static constexpr int CPR = COLS / 8, RPI = 1024 / (COLS * 2), J = BK / RPI / NW;
  static_assert((BK / RPI) % NW == 0, "instructions split evenly over the waves");
  const char* tile;
  int64_t ld;
  int k_total;
  int off[J];
  __device__ __forceinline__ MnDma(const bf16_t* tile_, int64_t ld_, int cols_valid, int k_total_ = 1 << 30)
      : tile(reinterpret_cast<const char*>(tile_)), ld(ld_), k_total(k_total_) {
    const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int k = (w + j * NW) * RPI + lane / CPR;
      const int c = (lane % CPR) ^ fm(k);
      const int cs = c * 8 < cols_valid ? c : (cols_valid >> 3) - 1;
      off[j] = int(k * ld_ * 2) + cs * 16;
    }
  }
  __device__ __forceinline__ void issue(int kt, char* slot) const {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kv = k_total - kt * BK;
    const int rows = kv < BK ? kv : BK;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(tile + (int64_t)kt * BK * ld * 2), (short)0, int(rows * ld * 2), 0x00020000);
#pragma unroll
    for (int j = 0; j < J; ++j) dma16_buf(r, off[j], slot + (w + j * NW) * 1024);
  }
};

// Two MN-contiguous sources side by side (the W_gate and W_up halves of a
// gate/up tile): B as two sub-tiles of COLS / 2 columns, [half][BK k][COLS /
// 2], each moved by its own MnDma, so every DMA instruction reads one tensor.
// A wave whose tile columns lie in one half reads that sub-tile as an MN tile
// of COLS / 2 columns (k_loop_dma2 with B_HALVES).
template <int COLS, int BK, int NW>
struct MnDma2 {
  using Half = MnDma<COLS / 2, BK, NW>;
  static constexpr int J = 2 * Half::J;
  static constexpr int HALF_BYTES = BK * COLS;  // bytes of one sub-tile
  Half g, u;
  __device__ __forceinline__ MnDma2(const bf16_t* t0, const bf16_t* t1, int64_t ld)
      : g(t0, ld, COLS / 2), u(t1, ld, COLS / 2) {}
  __device__ __forceinline__ void issue(int kt, char* slot) const {
    g.issue(kt, slot);
    u.issue(kt, slot + HALF_BYTES);
  }
};

// MN-contiguous operand by DMA whose k rows are gathered: k row r of the
// contraction (r from 0 over the expert's rows) is token row rows_src[r] / K
// of x (leading dimension ld), as MnGather; x_cols points at the tile's first
// column.  The token numbers of K tile kt + 1 are loaded while tile kt is
// requested (one index load per request, landing a step before they are
// needed).  k rows at or past k_total read the last valid row (k_loop_dma2
// zeroes them).  Byte offsets are 32-bit unsigned (callers keep x under 4 GiB).
template <int COLS, int BK, int NW>
struct MnGatherDma {
  static constexpr int CPR = COLS / 8, RPI = 1024 / (COLS * 2), J = BK / RPI / NW;
  static_assert((BK / RPI) % NW == 0, "instructions split evenly over the waves");
  static_assert(RPI == 2 && NW % 2 == 0, "a lane's k row has the same k & 3 in every request");
  const bf16_t* base;
  const int32_t* rows_src;
  int K, k_total;
  int64_t ld;
  unsigned coff;   // this lane's column chunk, in bytes
  int src[J];      // token rows of the next tile to request (loaded one step ahead)
  int ks[J];       // this lane's k row within a tile, per request
  __device__ __forceinline__ MnGatherDma(const bf16_t* x_cols, const int32_t* rows_src_, int K_, int64_t ld_,
                                         int cols_valid, int k_total_)
      : base(x_cols), rows_src(rows_src_), K(K_), k_total(k_total_), ld(ld_) {
    const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int j = 0; j < J; ++j) ks[j] = (w + j * NW) * RPI + lane / CPR;
    // the chunk's XOR swizzle depends on the k row only through k & 3, the same for every request of a lane
    const int c = (lane % CPR) ^ fm(ks[0]);
    const int cs = c * 8 < cols_valid ? c : (cols_valid >> 3) - 1;
    coff = unsigned(cs) * 16u;
    load_rows(0);
  }
  __device__ __forceinline__ void load_rows(int kt) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int r = kt * BK + ks[j];
      src[j] = rows_src[r < k_total ? r : k_total - 1];
    }
  }
  // requests tile kt (whose rows were loaded by the previous call or the
  // constructor), then loads the rows of tile kt + 1
  __device__ __forceinline__ void issue(int kt, char* slot) {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(base), (short)0, -1, 0x00020000);
#pragma unroll
    for (int j = 0; j < J; ++j)
      dma16_buf(r, int(unsigned((src[j] / K) * ld) * 2u + coff), slot + (w + j * NW) * 1024);
    load_rows(kt + 1);
  }
};

// Keeps every memory request before it ahead of every one after it (other
// instructions may still move across): the end-of-step wait of k_loop_dma2
// counts on operand A's requests being older than B's (vmcnt retires loads
// in issue order).
__device__ __forceinline__ void dma_order_fence() {
  __builtin_amdgcn_sched_barrier(0x0001 | 0x0002 | 0x0004 | 0x0008 | 0x0080 | 0x0100 | 0x0200 | 0x0400);
}

template <class C>
struct Dma2Layout {
  static constexpr int A0 = 0, B0 = 2 * C::A_BYTES;
  static constexpr int BYTES = 2 * C::A_BYTES + 3 * C::B_BYTES;
  static constexpr int LDS = BYTES > C::LDS_A ? BYTES : C::LDS_A;
};

// Instruction order of one step of k_loop_dma2 (masks as in
// reg_step_schedule): the first k step's fragment reads open the step; after
// each MFMA slot come its share of the next k step's fragment reads and of
// the step's VL DMA requests (spread over the first LK k steps).
// EARLY: all VL requests open the step, before the first fragment reads (the
// forward GEMMs: at N = 16384, H = 4096, F = 14336, E = 8 gate/up 6.92-6.93
// -> 6.80-6.86 ms and down 3.51-3.55 -> 3.41-3.42 ms; dA and the merged dX /
// weight-gradient launch were 1-2 % slower that way, so they keep the
// requests spread over the first k step).
template <int KK, int MK, int FR, int VL, int LK, bool EARLY = false, int J = 0>
__device__ __forceinline__ void dma2_schedule() {
  if constexpr (EARLY && J == 0 && VL > 0) {
    __builtin_amdgcn_sched_group_barrier(0x020, VL, 0);
    dma2_schedule<KK, MK, FR, 0, LK>();
    return;
  }
  if constexpr (J == 0) __builtin_amdgcn_sched_group_barrier(0x100, FR, 0);
  if constexpr (J < KK * MK) {
    constexpr int kk = J / MK, i = J % MK;
    constexpr int r = kk + 1 < KK ? (i + 1) * FR / MK - i * FR / MK : 0;
    constexpr int g = kk < LK ? (J + 1) * VL / (LK * MK) - J * VL / (LK * MK) : 0;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
    if constexpr (g > 0) __builtin_amdgcn_sched_group_barrier(0x020, g, 0);
    dma2_schedule<KK, MK, FR, VL, LK, false, J + 1>();
  }
}

// One step: the DMA of A tile ka into slot wa and of B tile kb into slot wb
// (A first: the end-of-step wait for it then leaves the B request in
// flight), then the MFMAs over slots ra / rb.  The four regions are distinct
// (restrict), so the compiler does not wait for the DMA before the fragment
// reads.
template <class C, bool A_MN, bool B_MN, bool MMA, bool B_HALVES, bool EARLY, class DA, class DB>
__device__ __forceinline__ void dma2_step(const char* __restrict__ ra, const char* __restrict__ rb,
                                          char* __restrict__ wa, char* __restrict__ wb, int ka, int kb,
                                          DA& da, DB& db, Acc<C>& acc, int wm, int wn) {
  if constexpr (!MMA) {
    da.issue(ka, wa);
    dma_order_fence();
    db.issue(kb, wb);
  } else {
    constexpr int KK = C::BK / 16;
    constexpr int FR = C::FM * (A_MN ? 2 : 1) + C::FN * (B_MN ? 2 : 1);
    constexpr int MK = C::FM * C::FN;
    constexpr int LOAD_STEPS = C::NW >= 8 ? 1 : (KK / 2 > 0 ? KK / 2 : 1);
    static_assert(!B_HALVES || (B_MN && C::WN == 2 && C::TN * 2 == C::BN), "one B half per wave column");
    // the wave's B columns: its own half (B_HALVES, a TN-column MN tile) or the whole B tile
    constexpr int BC = B_HALVES ? C::TN : C::BN;
    const char* sb = B_HALVES ? rb + wn * (C::BK * C::TN * 2) : rb;
    const int nb = B_HALVES ? 0 : wn * C::TN;
    bf16x8_t fa[2][C::FM], fb[2][C::FN];
#pragma unroll
    for (int mi = 0; mi < C::FM; ++mi)
      fa[0][mi] = A_MN ? frag_mn<C::BM>(ra, wm * C::TM + mi * 32, 0) : frag_kc<C::BK>(ra, wm * C::TM + mi * 32, 0);
#pragma unroll
    for (int ni = 0; ni < C::FN; ++ni)
      fb[0][ni] = B_MN ? frag_mn<BC>(sb, nb + ni * 32, 0) : frag_kc<C::BK>(sb, nb + ni * 32, 0);
    da.issue(ka, wa);
    dma_order_fence();
    db.issue(kb, wb);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int cb = kk & 1;
      if (kk + 1 < KK) {
#pragma unroll
        for (int mi = 0; mi < C::FM; ++mi)
          fa[cb ^ 1][mi] = A_MN ? frag_mn<C::BM>(ra, wm * C::TM + mi * 32, kk + 1)
                                : frag_kc<C::BK>(ra, wm * C::TM + mi * 32, kk + 1);
#pragma unroll
        for (int ni = 0; ni < C::FN; ++ni)
          fb[cb ^ 1][ni] = B_MN ? frag_mn<BC>(sb, nb + ni * 32, kk + 1) : frag_kc<C::BK>(sb, nb + ni * 32, kk + 1);
      }
#pragma unroll
      for (int mi = 0; mi < C::FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::FN; ++ni)
          acc.a[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cb][mi], fb[cb][ni], acc.a[mi][ni], 0, 0, 0);
    }
    dma2_schedule<KK, MK, FR, DA::J + DB::J, LOAD_STEPS, EARLY>();
    // every MFMA of the step is issued before the end-of-step wait and
    // barrier (otherwise the scheduler sinks the last k step's MFMAs past
    // them and a wave waits at the barrier with its matrix work undone)
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <class C, bool A_MN, bool B_MN, bool MMA, bool B_HALVES, bool EARLY, class DA, class DB>
__device__ __forceinline__ void k_steps_dma2(char* lds, Acc<C>& acc, int nk, DA& da, DB& db, int wm,
                                             int wn, int k_last) {
  using L = Dma2Layout<C>;
  int rs = 0;  // B slot of tile kt
  for (int kt = 0; kt < nk; ++kt) {
    const int ka = kt + 1 < nk ? kt + 1 : kt;
    const int kb = kt + 2 < nk ? kt + 2 : nk - 1;
    const int ws = rs == 0 ? 2 : rs - 1;  // (kt + 2) % 3
    char* ra = lds + L::A0 + (kt & 1) * C::A_BYTES;
    char* rb = lds + L::B0 + rs * C::B_BYTES;
    if (A_MN && kt == nk - 1 && k_last < C::BK) {
      // ragged contraction tail (both operands MN: k rows are LDS rows)
      static_assert(!A_MN || B_MN, "ragged tails with MN operands only");
      u32x4_t* za = reinterpret_cast<u32x4_t*>(ra + k_last * C::BM * 2);
      u32x4_t* zb = reinterpret_cast<u32x4_t*>(rb + k_last * C::BN * 2);
      for (int i = threadIdx.x; i < (C::BK - k_last) * C::BM * 2 / 16; i += C::NT) za[i] = u32x4_t{0u, 0u, 0u, 0u};
      for (int i = threadIdx.x; i < (C::BK - k_last) * C::BN * 2 / 16; i += C::NT) zb[i] = u32x4_t{0u, 0u, 0u, 0u};
      __syncthreads();
    }
    dma2_step<C, A_MN, B_MN, MMA, B_HALVES, EARLY>(ra, rb, lds + L::A0 + ((kt + 1) & 1) * C::A_BYTES,
                                     lds + L::B0 + ws * C::B_BYTES, ka, kb, da, db, acc, wm, wn);
    wait_vm<C::JB>();
    lds_barrier();
    rs = rs == 2 ? 0 : rs + 1;
  }
}

// Mixed-depth DMA K loop (see above).  Every step issues both requests (the
// last steps re-fetch the last tiles into slots nobody reads), so each wait
// is the same on every path: at the end of step kt only B tile kt + 2 may
// still be in flight.  mma = false (wave-uniform): the wave's rows are all
// past the tile's valid rows; it issues its requests and waits, no MFMAs.
// Each operand is K-contiguous (KcDma) or MN-contiguous (MnDma); with both
// MN-contiguous (the weight gradients) the last K tile may hold only k_last
// valid k rows.  B_HALVES: B is two MN sub-tiles (MnDma2), one per wave column.
// EARLY: each step's requests are issued before its first fragment reads.
template <class C, bool A_MN, bool B_MN, class DA, class DB, bool B_HALVES = false, bool EARLY = false>
__device__ __forceinline__ void k_loop_dma2(char* lds, Acc<C>& acc, int nk, DA da, DB db, int wm,
                                            int wn, bool mma = true, int k_last = C::BK) {
  using L = Dma2Layout<C>;
  static_assert(DA::J == C::JA && DB::J == C::JB, "one request per wave instruction");
  zero_acc(acc);
  if (nk <= 0) return;
  da.issue(0, lds + L::A0);
  db.issue(0, lds + L::B0);
  db.issue(nk > 1 ? 1 : 0, lds + L::B0 + C::B_BYTES);
  wait_vm<C::JB>();
  lds_barrier();
  if (__builtin_amdgcn_readfirstlane(mma ? 1 : 0))
    k_steps_dma2<C, A_MN, B_MN, true, B_HALVES, EARLY>(lds, acc, nk, da, db, wm, wn, k_last);
  else
    k_steps_dma2<C, A_MN, B_MN, false, B_HALVES, EARLY>(lds, acc, nk, da, db, wm, wn, k_last);
  // the last steps' requests land in slots nobody reads, but before the
  // caller reuses the LDS
  wait_vm<0>();
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

// Dynamic LDS above 64 KiB is enabled once per kernel (one static per
// kernel, keyed by the kernel itself).
template <auto Kern>
hipError_t allow_lds(int bytes) {
  static const hipError_t st =
      hipFuncSetAttribute(reinterpret_cast<const void*>(Kern), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  return st;
}

}  // namespace moe_mma
