/*
 * moe.h - C ABI of the MI355X (gfx950) dropless top-k Mixture-of-Experts
 * SwiGLU FFN layer, forward and backward, on one GPU.
 *
 * The layer (for a token x_n, a row of x [N, H]):
 *     l_n   = x_n . W_r (+ b)                       router logits, W_r [H, E]
 *     e_n,k = the K experts of largest logit, ordered (logit desc, id asc)
 *     g_n,k = softmax over the K selected logits     renormalised gates
 *     y_n   = sum_k g_n,k * FFN_{e_n,k}(x_n)
 *     FFN_e(v) = (silu(v . W_gate[e]) * (v . W_up[e])) . W_down[e]
 * Sources: "MoE computation principle and execution process: from Router
 * scoring to expert parallelism and load balancing" (icman.com.cn) sections
 * 2.1-2.3; "MoE technical analysis: from theory to practice"
 * (intelliparadigm.com) sections 2.1 and 2.3; dropless routing metadata and
 * the gather / grouped GEMM / weighted scatter structure from "MegaBlocks -
 * architecture and principles" (ai-reference-codex) sections 2.1 and 2.3.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor argument is a caller-owned DEVICE pointer to a contiguous
 *    row-major buffer with the shape stated below, aligned to 16 bytes.
 *    The library never allocates, frees or keeps device memory between
 *    calls; scratch memory comes only through (ws, ws_bytes), sized by
 *    moe_workspace_bytes().
 *  - "act" tensors (x, xs, G, U, A, ys, y, dy, dys, dG, dU, dxs, dx) and the
 *    weights (W_r, W_gate, W_up, W_down) have the element type dims->dtype:
 *    MOE_BF16 (bfloat16 storage, float32 accumulation, round-to-nearest-even
 *    on every store) or MOE_F32.  gates, dgates, dlogits, the logit bias and
 *    every weight gradient (dW_r, dW_gate, dW_up, dW_down) are float32.
 *  - Index tensors are int32.
 *  - All work is enqueued on `stream`; no call synchronises the stream or
 *    copies device memory to the host (num_tiles stays on the device).
 *  - Results are bitwise reproducible run to run: no floating-point atomics,
 *    every reduction has a fixed order and every output element has one
 *    owner.
 *  - Return value: MOE_OK, or a negative moe_status.  Arguments are checked
 *    on the host before anything is enqueued; on error nothing is enqueued.
 *    MOE_EHIP reports a launch error from the HIP runtime.  Faults inside a
 *    kernel surface at the caller's next synchronisation.
 *  - N == 0 is valid: the call returns MOE_OK and enqueues nothing (weight
 *    gradient outputs are then left untouched).
 *  - Limits: 1 <= E <= 256, 1 <= K <= min(E, 8), H and F multiples of 128,
 *    N*K < 2^31, N*E < 2^31.
 */
#ifndef MOE_MI355X_MOE_H_
#define MOE_MI355X_MOE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 9
/* Rows per tile of the grouped-GEMM tile list built by moe_permute_meta. */
#define MOE_TILE_M 256
#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOPK 8

typedef enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = -1,       /* bad shape, null or misaligned pointer */
  MOE_EUNSUPPORTED = -2, /* outside the limits above, or unknown dtype */
  MOE_EWORKSPACE = -3,   /* workspace missing or smaller than required */
  MOE_EHIP = -4,         /* the HIP runtime reported a launch error */
  MOE_ESCRATCH = -5      /* needs more than MOE_NOALLOC_SCRATCH_BYTES (no-allocation entry point) */
} moe_status;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Entry points that take a workspace (argument of moe_workspace_bytes). */
typedef enum moe_entry {
  MOE_ENTRY_PERMUTE_META = 1,
  MOE_ENTRY_ROUTE_BWD = 2,
  MOE_ENTRY_PERMUTE_BWD = 3, /* also moe_permute_bwd_dense */
  MOE_ENTRY_AUX_LOSS = 4,
  MOE_ENTRY_ROUTE_BWD_AUX = 5,
  MOE_ENTRY_SHARED_FFN = 6,    /* shared-expert dims only (E = K = 1) */
  MOE_ENTRY_SHARED_FFN_BWD = 7, /* shared-expert dims only (E = K = 1) */
  MOE_ENTRY_ROUTE_META = 8
} moe_entry;

/* bf16 grouped-GEMM tile family (moe_dims.gemm_tiles).  AUTO lets the
 * library choose per stage from the problem size (what the layer runs); the
 * others force one family on every GEMM stage of the call, so that tests can
 * reach each kernel family at small sizes.  Every family computes the same
 * values up to float32 summation order.  Ignored for MOE_F32. */
typedef enum moe_gemm_tiles {
  MOE_TILES_AUTO = 0,
  MOE_TILES_256 = 1,     /* 256 x 256 tiles */
  MOE_TILES_128X256 = 2, /* 128 x 256 register-staged tiles */
  MOE_TILES_128 = 3      /* 128 x 128 tiles (dA: 128 x 256 through the LDS DMA) */
} moe_gemm_tiles;

/* Problem sizes: N tokens, hidden size H, expert FFN size F, E experts,
 * K experts per token, dtype a moe_dtype.  NK = N*K routed rows.
 * gemm_tiles is a moe_gemm_tiles value (0 = AUTO); with a forced family the
 * merged dX/dW call makes two launches of that family. */
typedef struct moe_dims {
  int64_t N, H, F, E, K;
  int32_t dtype;
  int32_t gemm_tiles;
} moe_dims;

/* ABI version of the loaded library (MOE_ABI_VERSION it was built with). */
int moe_abi_version(void);

/* Static English text of a status code (never NULL). */
const char* moe_status_str(int status);

/* Capacity, in tiles, of the tile list: floor((NK + E*(MOE_TILE_M-1)) /
 * MOE_TILE_M), an upper bound of sum_e ceil(count_e / MOE_TILE_M) for any
 * routing.  The tiles buffer holds 3 int32 per tile.  Returns -1 on invalid
 * dims. */
int64_t moe_max_tiles(const moe_dims* d);

/* Workspace bytes needed by `entry` (a moe_entry) for these dims; 0 if the
 * entry needs none; (size_t)-1 on invalid dims or entry. */
size_t moe_workspace_bytes(const moe_dims* d, int32_t entry);

/* ---------------------------------------------------------------- forward */

/* Router: logits l = x.W_r (+ logit_bias), top-K by (logit desc, expert id
 * asc), gates = softmax over the K selected logits (icman sections 2.1 and
 * 2.2; intelliparadigm section 2.3).  Logits are accumulated in float32 and
 * not stored.
 *   x [N,H] act; w_r [H,E] act; logit_bias [E] f32 or NULL (a constant that
 *   changes selection and gate values);
 *   topk_idx [N,K] int32 out (slot k = rank k); gates [N,K] f32 out. */
int moe_route(const moe_dims* d, const void* x, const void* w_r, const float* logit_bias, int32_t* topk_idx,
              float* gates, hipStream_t stream);

/* moe_route followed by moe_permute_meta_capacity (capacity INT32_MAX: the
 * dropless metadata), with the same outputs, fused into two launches: the
 * router also leaves each 32-token block's histogram of the chosen experts
 * in the workspace, and one metadata kernel turns those histograms into the
 * bins, the stable ranks and the tile list without a separate histogram or
 * scan launch (MegaBlocks sections 2.1 and 2.3: histogram, cumsum into bins,
 * sort; routing and sort fused as in "MoK: high-performance Megakernel for
 * deterministic training of large MoE models" (jsqmd.com), section 1.3).
 * Every workgroup of that kernel re-reads all block histograms, so the
 * fusion is used while ceil(N/32)*E <= 32768; above that the call runs the
 * unfused kernels.  capacity < 0: MOE_EINVAL.  ws: MOE_ENTRY_ROUTE_META. */
int moe_route_meta(const moe_dims* d, const void* x, const void* w_r, const float* logit_bias, int32_t capacity,
                   int32_t* topk_idx, float* gates, int32_t* sorted_flat, int32_t* inv, int32_t* counts,
                   int32_t* offsets, int32_t* tiles, int32_t* num_tiles, void* ws, size_t ws_bytes,
                   hipStream_t stream);

/* Dropless routing metadata from the flat assignment f = n*K + k (MegaBlocks
 * sections 2.1, 2.3 and 4: sort by expert id, histogram, cumsum into bins):
 *   counts [E]      rows per expert (histogram);
 *   offsets [E+1]   exclusive cumsum of counts, offsets[E] = NK;
 *   sorted_flat [NK] flat indices grouped by expert, ascending f within an
 *                   expert (a stable sort on the expert id);
 *   inv [NK]        inv[f] = row of f in the grouped order;
 *   tiles [3*moe_max_tiles] (expert, first row, rows) per MOE_TILE_M-row tile,
 *                   experts ascending; only the first *num_tiles are written;
 *   num_tiles [1]   number of tiles, on the device.
 * topk_idx [N,K] int32 in, every value in [0,E).  ws: MOE_ENTRY_PERMUTE_META. */
int moe_permute_meta(const moe_dims* d, const int32_t* topk_idx, int32_t* sorted_flat, int32_t* inv, int32_t* counts,
                     int32_t* offsets, int32_t* tiles, int32_t* num_tiles, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* Token-dropping variant of moe_permute_meta with an expert capacity C >= 0
 * ("MoE computation principle and execution process" section 3.4: each
 * expert takes at most C rows, the overflow is dropped).  Expert e keeps the
 * first min(counts[e], C) of its rows in the stable grouped order (lowest
 * flat index first); every other row is dropped.
 *   counts [E]      full histogram of the assignment (before dropping);
 *   offsets [E+1]   exclusive cumsum of the kept counts, offsets[E] = kept
 *                   rows in total;
 *   sorted_flat [NK] the kept rows grouped by expert, then -1 for each
 *                   dropped row;
 *   inv [NK]        row of f, or -1 when f is dropped;
 *   tiles, num_tiles over the kept rows.
 * Downstream, moe_permute skips -1 rows, moe_combine / moe_combine_bwd /
 * moe_permute_bwd(_dense) treat inv < 0 as a slot that adds nothing (zero
 * gate gradient, no dxs row); the GEMMs see only the kept rows through the
 * tile list and offsets.  C >= max(counts) reproduces moe_permute_meta.
 * capacity < 0 -> MOE_EINVAL.  ws: MOE_ENTRY_PERMUTE_META. */
int moe_permute_meta_capacity(const moe_dims* d, const int32_t* topk_idx, int32_t capacity, int32_t* sorted_flat,
                              int32_t* inv, int32_t* counts, int32_t* offsets, int32_t* tiles, int32_t* num_tiles,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/* Permuting gather: xs[i] = x[sorted_flat[i] / K]  (MegaBlocks section 2.1).
 *   x [N,H] act in; sorted_flat [NK] in; xs [NK,H] act out. */
int moe_permute(const moe_dims* d, const void* x, const int32_t* sorted_flat, void* xs, hipStream_t stream);

/* Grouped SwiGLU experts over the tile list (icman section 2.3;
 * intelliparadigm section 2.1), for every row i of expert e:
 *   G[i] = xs[i].W_gate[e], U[i] = xs[i].W_up[e]    (stored rounded),
 *   A[i] = silu(G[i]) * U[i]                         (from the rounded G, U),
 *   ys[i] = A[i].W_down[e].
 *   xs [NK,H]; w_gate, w_up [E,H,F]; w_down [E,F,H]; tiles/num_tiles from
 *   moe_permute_meta; g_save, u_save [NK,F] out or both NULL (forward only);
 *   act [NK,F] out (A, needed by the backward); ys [NK,H] out.
 * Calls moe_ffn_gate_up then moe_ffn_down. */
int moe_expert_ffn(const moe_dims* d, const void* xs, const void* w_gate, const void* w_up, const void* w_down,
                   const int32_t* tiles, const int32_t* num_tiles, void* g_save, void* u_save, void* act, void* ys,
                   hipStream_t stream);

/* First grouped GEMM of moe_expert_ffn: the gate and up projections of the
 * SwiGLU expert and its activation (icman section 2.3: silu on the gate
 * branch times the linear up branch; intelliparadigm section 2.1: the
 * expert FeedForward without biases), over the variable-size expert groups
 * of the tile list (MegaBlocks section 2.3, grouped GEMM), row i of expert e:
 *   G[i] = xs[i].W_gate[e], U[i] = xs[i].W_up[e]  (float32 sums, stored
 *   rounded); A[i] = silu(G[i]) * U[i] from the rounded G, U.
 *   xs [NK,H] act; w_gate, w_up [E,H,F]; tiles, num_tiles from
 *   moe_permute_meta; g_save, u_save [NK,F] out or both NULL (no backward);
 *   act [NK,F] out.  Rows past offsets[E] are not written.
 * Errors: MOE_EINVAL for a bad shape or a null/misaligned xs, weight, tile
 * or act pointer (or exactly one of g_save, u_save NULL). */
int moe_ffn_gate_up(const moe_dims* d, const void* xs, const void* w_gate, const void* w_up, const int32_t* tiles,
                    const int32_t* num_tiles, void* g_save, void* u_save, void* act, hipStream_t stream);

/* moe_ffn_gate_up with the permuting gather fused into its row loads
 * (MegaBlocks section 2.1 gather, folded into the grouped GEMM as the
 * "MoE computation principle..." page's section 3.4 merges tokens per expert):
 * row i of the grouped order is read as x[sorted_flat[i] / K], so no xs
 * buffer is written or read.  Results are bit-identical to moe_permute
 * followed by moe_ffn_gate_up.  For callers that need no backward (the
 * weight gradients read xs).
 *   x [N,H] act in; sorted_flat [NK] from moe_permute_meta; the rest as
 *   moe_ffn_gate_up.  Requires N*H < 2^31 (MOE_EUNSUPPORTED otherwise). */
int moe_ffn_gate_up_gather(const moe_dims* d, const void* x, const int32_t* sorted_flat, const void* w_gate,
                           const void* w_up, const int32_t* tiles, const int32_t* num_tiles, void* g_save,
                           void* u_save, void* act, hipStream_t stream);

/* Second grouped GEMM of moe_expert_ffn: the SwiGLU expert's down
 * projection (icman section 2.3; MegaBlocks section 2.3, grouped GEMM over
 * the variable-size groups), row i of expert e:
 *   ys[i] = A[i].W_down[e]  (float32 sums, stored rounded).
 *   act [NK,F] from moe_ffn_gate_up; w_down [E,F,H]; tiles, num_tiles from
 *   moe_permute_meta; ys [NK,H] out.  Errors: MOE_EINVAL for a bad shape or a
 *   null/misaligned pointer. */
int moe_ffn_down(const moe_dims* d, const void* act, const void* w_down, const int32_t* tiles,
                 const int32_t* num_tiles, void* ys, hipStream_t stream);

/* Gate-weighted combine back to token order (MegaBlocks section 2.1:
 * weighted scatter with a sum over the top-k; icman section 2.3):
 *   y[n] = sum_{k=0..K-1} gates[n,k] * ys[inv[n*K+k]], k ascending, float32
 *   accumulation, one rounding.
 *   ys [NK,H]; gates [N,K]; inv [NK]; y [N,H] out. */
int moe_combine(const moe_dims* d, const void* ys, const float* gates, const int32_t* inv, void* y,
                hipStream_t stream);

/* --------------------------------------------------------------- backward */

/* Backward of the combine (the backward of a weighted scatter is a weighted
 * gather, MegaBlocks section 4):
 *   dys[inv[n*K+k]] = gates[n,k] * dy[n];
 *   dgates[n,k] = <dy[n], ys[inv[n*K+k]]> (float32, fixed reduction order).
 *   dy [N,H]; ys [NK,H]; gates [N,K]; inv [NK]; dys [NK,H] out;
 *   dgates [N,K] out. */
int moe_combine_bwd(const moe_dims* d, const void* dy, const void* ys, const float* gates, const int32_t* inv,
                    void* dys, float* dgates, hipStream_t stream);

/* Router backward through the softmax over the selected logits only (icman
 * section 2.2: the gradient flows through the continuous gate weights):
 *   s_n = sum_k gates[n,k]*dgates[n,k];
 *   dlogits[n,e_k] = gates[n,k]*(dgates[n,k] - s_n), 0 for unselected e;
 *   dw_r = x^T . dlogits (fixed partition of the tokens, fixed-order sum).
 *   x [N,H]; topk_idx, gates, dgates [N,K]; dlogits [N,E] f32 out;
 *   dw_r [H,E] f32 out.  ws: MOE_ENTRY_ROUTE_BWD. */
int moe_route_bwd(const moe_dims* d, const void* x, const int32_t* topk_idx, const float* gates,
                  const float* dgates, float* dlogits, float* dw_r, void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward of the grouped SwiGLU experts (the expert of icman section 2.3,
 * differentiated; the activation is recomputed from the stored G and U as
 * MegaBlocks section 4 recomputes it in the backward), for every row i of
 * expert e:
 *   dA = dys[i].W_down[e]^T; s = sigmoid(G[i]);
 *   dG[i] = dA*U[i]*s*(1 + G[i]*(1-s)), dU[i] = dA*G[i]*s   (stored rounded);
 *   dxs[i] = dG[i].W_gate[e]^T + dU[i].W_up[e]^T;
 *   dW_gate[e] = xs_e^T.dG_e, dW_up[e] = xs_e^T.dU_e, dW_down[e] = A_e^T.dys_e
 *   (float32, rows summed in ascending order inside each tile; experts with
 *   no rows get exact zeros).
 *   dys, xs [NK,H]; w_gate, w_up [E,H,F]; w_down [E,F,H]; g_save, u_save,
 *   act [NK,F] from moe_expert_ffn; offsets, tiles, num_tiles from
 *   moe_permute_meta; dg, du [NK,F] out; dxs [NK,H] out; dw_gate, dw_up
 *   [E,H,F] f32 out; dw_down [E,F,H] f32 out.
 * Calls moe_ffn_bwd_dact, then moe_ffn_bwd_dx_dw. */
int moe_expert_ffn_bwd(const moe_dims* d, const void* dys, const void* xs, const void* w_gate, const void* w_up,
                       const void* w_down, const void* g_save, const void* u_save, const void* act,
                       const int32_t* offsets, const int32_t* tiles, const int32_t* num_tiles, void* dg, void* du,
                       void* dxs, float* dw_gate, float* dw_up, float* dw_down, hipStream_t stream);

/* First step of moe_expert_ffn_bwd: the down projection's input gradient
 * and the SwiGLU derivative (icman section 2.3, differentiated), row i of
 * expert e:
 *   dA = dys[i].W_down[e]^T (float32, not stored); s = sigmoid(G[i]);
 *   dG[i] = dA*U[i]*s*(1 + G[i]*(1-s)), dU[i] = dA*G[i]*s (stored rounded).
 *   dys [NK,H] act from moe_combine_bwd; w_down [E,F,H]; g_save, u_save
 *   [NK,F] from moe_ffn_gate_up; tiles, num_tiles from moe_permute_meta;
 *   dg, du [NK,F] out.  Errors: MOE_EINVAL for a bad shape or a
 *   null/misaligned pointer. */
int moe_ffn_bwd_dact(const moe_dims* d, const void* dys, const void* w_down, const void* g_save, const void* u_save,
                     const int32_t* tiles, const int32_t* num_tiles, void* dg, void* du, hipStream_t stream);

/* Input gradient of the expert rows (icman section 2.3, differentiated),
 * row i of expert e:
 *   dxs[i] = dG[i].W_gate[e]^T + dU[i].W_up[e]^T (one float32 sum over both
 *   contractions, stored rounded).
 *   dg, du [NK,F] from moe_ffn_bwd_dact; w_gate, w_up [E,H,F]; tiles,
 *   num_tiles from moe_permute_meta; dxs [NK,H] out.  Errors: MOE_EINVAL for
 *   a bad shape or a null/misaligned pointer. */
int moe_ffn_bwd_dx(const moe_dims* d, const void* dg, const void* du, const void* w_gate, const void* w_up,
                   const int32_t* tiles, const int32_t* num_tiles, void* dxs, hipStream_t stream);

/* Weight gradients of the experts (icman section 2.3, differentiated; fp32
 * gradient buffers as the MoonEP page's section 04 keeps them):
 *   dW_gate[e] = xs_e^T.dG_e, dW_up[e] = xs_e^T.dU_e, dW_down[e] = A_e^T.dys_e
 * with xs_e, A_e, ... the rows offsets[e] .. offsets[e+1]-1.  One workgroup
 * owns each output tile and sums the expert's rows in ascending order, so
 * results are bitwise reproducible; experts with no rows get exact zeros.
 *   xs [NK,H]; act [NK,F]; dys [NK,H]; dg, du [NK,F]; offsets [E+1];
 *   dw_gate, dw_up [E,H,F] f32 out; dw_down [E,F,H] f32 out.  Errors:
 *   MOE_EINVAL for a bad shape or a null/misaligned pointer. */
int moe_ffn_bwd_dw(const moe_dims* d, const void* xs, const void* act, const void* dys, const void* dg,
                   const void* du, const int32_t* offsets, float* dw_gate, float* dw_up, float* dw_down,
                   hipStream_t stream);

/* moe_ffn_bwd_dx and moe_ffn_bwd_dw in one call.  For bf16 it is one launch
 * of 256 x 256 tiles: the weight-gradient tiles are dispatched first and the
 * dX tiles fill the CUs they leave idle (the weight gradients alone have
 * 3*E*ceil(H/256)*ceil(F/256) tiles, 192 at H = 512, F = 1024, E = 8).  Every
 * output element has one owner and the same ascending contraction order as
 * in the separate calls.  With a forced tile family (moe_dims.gemm_tiles),
 * and for float32, it makes the two separate launches.  Arguments as in
 * those two calls. */
int moe_ffn_bwd_dx_dw(const moe_dims* d, const void* dg, const void* du, const void* w_gate, const void* w_up,
                      const int32_t* tiles, const int32_t* num_tiles, void* dxs, const void* xs, const void* act,
                      const void* dys, const int32_t* offsets, float* dw_gate, float* dw_up, float* dw_down,
                      hipStream_t stream);

/* moe_ffn_bwd_dx_dw with the grouped rows read from the token rows: x [N,H]
 * replaces xs and row i of the grouped order is x[sorted_flat[i] / K] in
 * dW_gate = xs_e^T.dG_e and dW_up = xs_e^T.dU_e (the gather of moe_permute
 * done inside the weight-gradient loads, MegaBlocks section 2.1, so a
 * training step needs no xs).  Same bytes as moe_permute + moe_ffn_bwd_dx_dw.
 * It saves the NK x H xs buffer and the permute, but the launch itself is
 * slower than the xs form (scattered row loads), so it is meant for callers
 * short of memory.
 *   sorted_flat [NK] from moe_permute_meta (or moe_route_meta), read only in
 *   the expert ranges offsets[e] .. offsets[e+1], which hold no dropped row;
 *   other arguments as moe_ffn_bwd_dx_dw.  Errors: as moe_ffn_bwd_dx_dw, plus
 *   MOE_EINVAL for a null or misaligned x or sorted_flat. */
int moe_ffn_bwd_dx_dw_gather(const moe_dims* d, const void* dg, const void* du, const void* w_gate,
                             const void* w_up, const int32_t* tiles, const int32_t* num_tiles, void* dxs,
                             const void* x, const int32_t* sorted_flat, const void* act, const void* dys,
                             const int32_t* offsets, float* dw_gate, float* dw_up, float* dw_down,
                             hipStream_t stream);

/* Backward of the gather plus the router's input gradient (MegaBlocks
 * section 4: the backward of a gather is a scatter, here a gather-sum over
 * each token's K rows so that no atomics are needed; the router term is the
 * logits' input gradient, icman section 2.2):
 *   dx[n] = sum_k dxs[inv[n*K+k]] + sum_k dlogits[n,e_k] * W_r[:,e_k],
 *   k ascending, float32 accumulation, one rounding.
 *   dxs [NK,H]; inv [NK]; topk_idx [N,K]; dlogits [N,E] f32; w_r [H,E];
 *   dx [N,H] out.  ws: MOE_ENTRY_PERMUTE_BWD (holds W_r transposed). */
int moe_permute_bwd(const moe_dims* d, const void* dxs, const int32_t* inv, const int32_t* topk_idx,
                    const float* dlogits, const void* w_r, void* dx, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------ load-balancing loss */
/* Switch load-balancing loss ("MoE computation principle and execution
 * process", icman.com.cn, section 4.2):
 *     L_aux = alpha * E * sum_e f_e * P_e
 * with f_e = counts[e] / (N*K), the share of the N*K routed assignments that
 * went to expert e (the token share for K = 1), and P_e the softmax over all
 * E router logits (the same logits, bias included, that select the experts)
 * averaged over the N tokens.  f is a count and carries no gradient.  */

/* Forward: recomputes the logits x.W_r (+ logit_bias) as moe_route does and
 * writes probs [N,E] f32 (the full softmax of every token; the backward needs
 * it) and loss [1] f32 (device memory; never read back by the library).
 * P_e is summed over token blocks in a fixed order, so the loss is
 * bitwise reproducible.  counts [E] int32 from moe_permute_meta; alpha finite
 * (else MOE_EINVAL).  ws: MOE_ENTRY_AUX_LOSS.  N == 0 enqueues nothing and
 * leaves loss untouched. */
int moe_aux_loss(const moe_dims* d, const void* x, const void* w_r, const float* logit_bias, const int32_t* counts,
                 float alpha, float* probs, float* loss, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_route_bwd with the gradient of aux_scale * L_aux / alpha added to every
 * router logit before dW_r is formed (aux_scale = alpha times the upstream
 * gradient of L_aux, usually alpha):
 *     dlogits[n,e] += aux_scale * E / N * probs[n,e] * (f_e - sum_i f_i probs[n,i]).
 * dlogits is then dense: use moe_permute_bwd_dense for dx.  probs from
 * moe_aux_loss; counts [E].  ws: MOE_ENTRY_ROUTE_BWD_AUX. */
int moe_route_bwd_aux(const moe_dims* d, const void* x, const int32_t* topk_idx, const float* gates,
                      const float* dgates, const float* probs, const int32_t* counts, float aux_scale,
                      float* dlogits, float* dw_r, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_permute_bwd with the router term over all E experts:
 *     dx[n] = sum_k dxs[inv[n*K+k]] + sum_e dlogits[n,e] * W_r[:,e],
 *   k and e ascending, float32 accumulation, one rounding.  Same arguments and
 *   workspace (MOE_ENTRY_PERMUTE_BWD) as moe_permute_bwd. */
int moe_permute_bwd_dense(const moe_dims* d, const void* dxs, const int32_t* inv, const int32_t* topk_idx,
                          const float* dlogits, const void* w_r, void* dx, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* ------------------------------------------------------- shared expert */
/* A shared expert ("MegaBlocks - architecture and principles",
 * ai-reference-codex, section 2.1: the layer's output plus an optional
 * shared-expert MLP that every token passes through): one dense SwiGLU
 * expert of intermediate size Fs over all N tokens, weight 1,
 *     y[n] = sum_k g_n,k FFN_{e_n,k}(x_n) + FFN_s(x_n).
 * Its calls take the shared expert's own dims ds = {N, H, Fs, E = 1, K = 1,
 * dtype} (any other E or K: MOE_EINVAL; moe_workspace_bytes returns
 * (size_t)-1).  Its weights: w_gate, w_up [H,Fs]; w_down [Fs,H]; its rows
 * are x itself, in token order. */

/* Forward of the shared expert:
 *   G = x.W_gate_s, U = x.W_up_s, A = silu(G)*U, ys_shared = A.W_down_s
 *   (each stored rounded, float32 accumulation).
 *   x [N,H]; g_save, u_save [N,Fs] out or both NULL (forward only);
 *   act [N,Fs] out; ys_shared [N,H] out.  ws: MOE_ENTRY_SHARED_FFN (its tile
 *   list, rebuilt on every call). */
int moe_shared_ffn(const moe_dims* ds, const void* x, const void* w_gate, const void* w_up, const void* w_down,
                   void* g_save, void* u_save, void* act, void* ys_shared, void* ws, size_t ws_bytes,
                   hipStream_t stream);

/* moe_combine with the shared expert's output added after the K routed
 * terms: y[n] = sum_k gates[n,k]*ys[inv[n*K+k]] + ys_shared[n], float32,
 * one rounding.  d: the layer's dims; ys_shared [N,H] act. */
int moe_combine_shared(const moe_dims* d, const void* ys, const float* gates, const int32_t* inv,
                       const void* ys_shared, void* y, hipStream_t stream);

/* Backward of the shared expert (its upstream gradient is dy itself):
 *   dA = dy.W_down_s^T; s = sigmoid(G);
 *   dG = dA*U*s*(1 + G*(1-s)), dU = dA*G*s (stored rounded);
 *   dx_shared = dG.W_gate_s^T + dU.W_up_s^T (stored rounded);
 *   dW_gate_s = x^T.dG, dW_up_s = x^T.dU, dW_down_s = A^T.dy (float32).
 * The weight gradients contract over all N tokens: the tokens are cut into
 * fixed row chunks whose float32 partial products are summed in chunk
 * order, so results are bitwise reproducible for a given N, H, Fs.
 *   dy [N,H]; g_save, u_save, act [N,Fs] from moe_shared_ffn; dg, du [N,Fs]
 *   out; dx_shared [N,H] out (add it with moe_permute_bwd_add);
 *   dw_gate, dw_up [H,Fs] f32 out; dw_down [Fs,H] f32 out.
 *   ws: MOE_ENTRY_SHARED_FFN_BWD (tile list, chunk bounds and, when the
 *   contraction is split, 3*S*H*Fs float32 partials). */
int moe_shared_ffn_bwd(const moe_dims* ds, const void* x, const void* dy, const void* w_gate, const void* w_up,
                       const void* w_down, const void* g_save, const void* u_save, const void* act, void* dg, void* du,
                       void* dx_shared, float* dw_gate, float* dw_up, float* dw_down, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* moe_permute_bwd (dense = 0) or moe_permute_bwd_dense (dense = 1; other
 * values MOE_EINVAL) with one more row added last:
 *   dx[n] = sum_k dxs[inv[n*K+k]] + (router term) + dx_add[n],
 *   float32, one rounding.  dx_add [N,H] act (the shared expert's
 *   dx_shared).  d: the layer's dims.  ws: MOE_ENTRY_PERMUTE_BWD. */
int moe_permute_bwd_add(const moe_dims* d, const void* dxs, const int32_t* inv, const int32_t* topk_idx,
                        const float* dlogits, const void* w_r, int32_t dense, const void* dx_add, void* dx, void* ws,
                        size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------- no-allocation entry point */

/* Scratch held by the library for moe_route_meta_noalloc, per GPU, for the
 * life of the process. */
#define MOE_NOALLOC_SCRATCH_BYTES (4u << 20)

/* moe_route_meta for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments and results as moe_route_meta minus
 * (ws, ws_bytes): the scratch it needs lives in a file-scope device array of
 * MOE_NOALLOC_SCRATCH_BYTES per GPU, whose address is looked up on the first
 * call on each device (the current device; the stream must belong to it).
 * No call allocates or frees memory.
 * Limit: moe_workspace_bytes(d, MOE_ENTRY_ROUTE_META) <= 4 MiB, i.e.
 * ceil(N/32)*E*4 bytes while the fused path runs (ceil(N/32)*E <= 32768,
 * always within the limit) and (ceil(N*K/1024)*E + 2*E)*4 bytes otherwise
 * (about N*K*E <= 2^30); beyond it the call returns MOE_ESCRATCH and
 * enqueues nothing.  Every GPU's array is shared by all calls on that GPU
 * and keeps the last call's contents: each call writes every scratch byte it
 * reads before reading it, so nothing needs clearing, but calls that overlap
 * on one GPU (two streams, or two threads) race and must be serialised by
 * the caller.  Other errors: as moe_route_meta; MOE_EHIP if the device or
 * the array's address cannot be queried. */
int moe_route_meta_noalloc(const moe_dims* d, const void* x, const void* w_r, const float* logit_bias,
                           int32_t capacity, int32_t* topk_idx, float* gates, int32_t* sorted_flat, int32_t* inv,
                           int32_t* counts, int32_t* offsets, int32_t* tiles, int32_t* num_tiles, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_MOE_H_ */
