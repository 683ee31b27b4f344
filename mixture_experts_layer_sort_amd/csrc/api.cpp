// C ABI of the MoE layer library: argument validation on the host (nothing is
// enqueued when a check fails), then the kernel launches on the caller's
// stream.  No entry point allocates memory, synchronises or reads device
// memory back to the host.
#include <hip/hip_runtime_api.h>

#include <cstdint>

#include <cmath>

#include "common.h"
#include "moe.h"

namespace {

using moe_launch::Dims;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape and limit checks shared by every entry point.
int check_dims(const moe_dims* d, Dims* out) {
  if (d == nullptr) return MOE_EINVAL;
  if (d->gemm_tiles < MOE_TILES_AUTO || d->gemm_tiles > MOE_TILES_128) return MOE_EINVAL;
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if (d->N < 0 || d->H <= 0 || d->F <= 0 || d->E <= 0 || d->K <= 0) return MOE_EINVAL;
  if (d->H % 128 != 0 || d->F % 128 != 0) return MOE_EINVAL;
  if (d->E > MOE_MAX_EXPERTS || d->K > MOE_MAX_TOPK || d->K > d->E) return MOE_EUNSUPPORTED;
  if (d->H > (int64_t(1) << 20) || d->F > (int64_t(1) << 20)) return MOE_EUNSUPPORTED;
  const int64_t lim = int64_t(1) << 31;
  if (d->N >= lim || d->N * d->K >= lim || d->N * d->E >= lim) return MOE_EUNSUPPORTED;
  out->N = d->N;
  out->H = d->H;
  out->F = d->F;
  out->E = d->E;
  out->K = d->K;
  out->dtype = d->dtype;
  out->tiles = d->gemm_tiles;
  return MOE_OK;
}

// Every listed pointer must be non-null and 16-byte aligned.
template <typename... P>
bool ptrs_ok(P... p) {
  const void* arr[] = {static_cast<const void*>(p)...};
  for (const void* q : arr)
    if (q == nullptr || !aligned16(q)) return false;
  return true;
}

int from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// The shared expert's dims: one expert, every token routed to it once.
bool is_shared(const Dims& D) { return D.E == 1 && D.K == 1; }

#define MOE_CHECK_DIMS(d, D)            \
  Dims D;                               \
  {                                     \
    int st_ = check_dims((d), &D);      \
    if (st_ != MOE_OK) return st_;      \
  }

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (shape, null or misaligned pointer)";
    case MOE_EUNSUPPORTED: return "unsupported configuration (limits or dtype)";
    case MOE_EWORKSPACE: return "workspace missing or too small";
    case MOE_EHIP: return "HIP runtime reported a launch error";
    case MOE_ESCRATCH: return "problem needs more scratch than the no-allocation entry point holds (4 MiB)";
    default: return "unknown status";
  }
}

int64_t moe_max_tiles(const moe_dims* d) {
  Dims D;
  if (check_dims(d, &D) != MOE_OK) return -1;
  return moe_launch::max_tiles(D);
}

size_t moe_workspace_bytes(const moe_dims* d, int32_t entry) {
  Dims D;
  if (check_dims(d, &D) != MOE_OK) return size_t(-1);
  switch (entry) {
    case MOE_ENTRY_PERMUTE_META: return moe_launch::permute_meta_ws(D);
    case MOE_ENTRY_ROUTE_BWD: return moe_launch::route_bwd_ws(D);
    case MOE_ENTRY_PERMUTE_BWD: return moe_launch::permute_bwd_ws(D);
    case MOE_ENTRY_AUX_LOSS: return moe_launch::aux_loss_ws(D);
    case MOE_ENTRY_ROUTE_BWD_AUX: return moe_launch::route_bwd_aux_ws(D);
    case MOE_ENTRY_SHARED_FFN: return is_shared(D) ? moe_launch::shared_ffn_ws(D) : size_t(-1);
    case MOE_ENTRY_SHARED_FFN_BWD: return is_shared(D) ? moe_launch::shared_ffn_bwd_ws(D) : size_t(-1);
    case MOE_ENTRY_ROUTE_META: return moe_launch::route_meta_ws(D);
    default: return size_t(-1);
  }
}

int moe_route(const moe_dims* d, const void* x, const void* w_r, const float* logit_bias, int32_t* topk_idx,
              float* gates, hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(x, w_r, topk_idx, gates)) return MOE_EINVAL;
  if (logit_bias != nullptr && !aligned16(logit_bias)) return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  return from_hip(moe_launch::route(D, x, w_r, logit_bias, topk_idx, gates, stream));
}

int moe_route_meta(const moe_dims* d, const void* x, const void* w_r, const float* logit_bias, int32_t capacity,
                   int32_t* topk_idx, float* gates, int32_t* sorted_flat, int32_t* inv, int32_t* counts,
                   int32_t* offsets, int32_t* tiles, int32_t* num_tiles, void* ws, size_t ws_bytes,
                   hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(x, w_r, topk_idx, gates, sorted_flat, inv, counts, offsets, tiles, num_tiles)) return MOE_EINVAL;
  if (logit_bias != nullptr && !aligned16(logit_bias)) return MOE_EINVAL;
  if (capacity < 0) return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  const size_t need = moe_launch::route_meta_ws(D);
  if (ws == nullptr || ws_bytes < need || !aligned16(ws)) return MOE_EWORKSPACE;
  return from_hip(moe_launch::route_meta(D, x, w_r, logit_bias, capacity, topk_idx, gates, sorted_flat, inv, counts,
                                         offsets, tiles, num_tiles, ws, stream));
}

int moe_permute_meta_capacity(const moe_dims* d, const int32_t* topk_idx, int32_t capacity, int32_t* sorted_flat,
                              int32_t* inv, int32_t* counts, int32_t* offsets, int32_t* tiles, int32_t* num_tiles,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(topk_idx, sorted_flat, inv, counts, offsets, tiles, num_tiles)) return MOE_EINVAL;
  if (capacity < 0) return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  const size_t need = moe_launch::permute_meta_ws(D);
  if (need > 0 && (ws == nullptr || ws_bytes < need || !aligned16(ws))) return MOE_EWORKSPACE;
  return from_hip(moe_launch::permute_meta(D, topk_idx, capacity, sorted_flat, inv, counts, offsets, tiles, num_tiles,
                                           ws, stream));
}

int moe_permute_meta(const moe_dims* d, const int32_t* topk_idx, int32_t* sorted_flat, int32_t* inv, int32_t* counts,
                     int32_t* offsets, int32_t* tiles, int32_t* num_tiles, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  return moe_permute_meta_capacity(d, topk_idx, INT32_MAX, sorted_flat, inv, counts, offsets, tiles, num_tiles, ws,
                                   ws_bytes, stream);
}

int moe_permute(const moe_dims* d, const void* x, const int32_t* sorted_flat, void* xs, hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(x, sorted_flat, xs)) return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  return from_hip(moe_launch::permute(D, x, sorted_flat, xs, stream));
}

int moe_ffn_gate_up(const moe_dims* d, const void* xs, const void* w_gate, const void* w_up, const int32_t* tiles,
                    const int32_t* num_tiles, void* g_save, void* u_save, void* act, hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(xs, w_gate, w_up, tiles, num_tiles, act)) return MOE_EINVAL;
  if ((g_save == nullptr) != (u_save == nullptr)) return MOE_EINVAL;
  if (g_save != nullptr && !ptrs_ok(g_save, u_save)) return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  return from_hip(moe_launch::ffn_gate_up(D, xs, nullptr, w_gate, w_up, tiles, num_tiles, g_save, u_save, act, stream));
}

int moe_ffn_gate_up_gather(const moe_dims* d, const void* x, const int32_t* sorted_flat, const void* w_gate,
                           const void* w_up, const int32_t* tiles, const int32_t* num_tiles, void* g_save,
                           void* u_save, void* act, hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(x, sorted_flat, w_gate, w_up, tiles, num_tiles, act)) return MOE_EINVAL;
  if ((g_save == nullptr) != (u_save == nullptr)) return MOE_EINVAL;
  if (g_save != nullptr && !ptrs_ok(g_save, u_save)) return MOE_EINVAL;
  if (D.N * D.H >= (int64_t(1) << 31)) return MOE_EUNSUPPORTED;  // 32-bit row offsets into x
  if (D.N == 0) return MOE_OK;
  return from_hip(
      moe_launch::ffn_gate_up(D, x, sorted_flat, w_gate, w_up, tiles, num_tiles, g_save, u_save, act, stream));
}

int moe_ffn_down(const moe_dims* d, const void* act, const void* w_down, const int32_t* tiles,
                 const int32_t* num_tiles, void* ys, hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(act, w_down, tiles, num_tiles, ys)) return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  return from_hip(moe_launch::ffn_down(D, act, w_down, tiles, num_tiles, ys, stream));
}

int moe_expert_ffn(const moe_dims* d, const void* xs, const void* w_gate, const void* w_up, const void* w_down,
                   const int32_t* tiles, const int32_t* num_tiles, void* g_save, void* u_save, void* act, void* ys,
                   hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(xs, w_gate, w_up, w_down, tiles, num_tiles, act, ys)) return MOE_EINVAL;
  if ((g_save == nullptr) != (u_save == nullptr)) return MOE_EINVAL;
  if (g_save != nullptr && !ptrs_ok(g_save, u_save)) return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  int st = from_hip(moe_launch::ffn_gate_up(D, xs, nullptr, w_gate, w_up, tiles, num_tiles, g_save, u_save, act, stream));
  if (st != MOE_OK) return st;
  return from_hip(moe_launch::ffn_down(D, act, w_down, tiles, num_tiles, ys, stream));
}

int moe_combine(const moe_dims* d, const void* ys, const float* gates, const int32_t* inv, void* y,
                hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(ys, gates, inv, y)) return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  return from_hip(moe_launch::combine(D, ys, gates, inv, nullptr, y, stream));
}

int moe_combine_bwd(const moe_dims* d, const void* dy, const void* ys, const float* gates, const int32_t* inv,
                    void* dys, float* dgates, hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(dy, ys, gates, inv, dys, dgates)) return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  return from_hip(moe_launch::combine_bwd(D, dy, ys, gates, inv, dys, dgates, stream));
}

int moe_route_bwd(const moe_dims* d, const void* x, const int32_t* topk_idx, const float* gates,
                  const float* dgates, float* dlogits, float* dw_r, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(x, topk_idx, gates, dgates, dlogits, dw_r)) return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  const size_t need = moe_launch::route_bwd_ws(D);
  if (ws == nullptr || ws_bytes < need || !aligned16(ws)) return MOE_EWORKSPACE;
  return from_hip(moe_launch::route_bwd(D, x, topk_idx, gates, dgates, dlogits, dw_r, ws, stream));
}

int moe_ffn_bwd_dact(const moe_dims* d, const void* dys, const void* w_down, const void* g_save, const void* u_save,
                     const int32_t* tiles, const int32_t* num_tiles, void* dg, void* du, hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(dys, w_down, g_save, u_save, tiles, num_tiles, dg, du)) return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  return from_hip(moe_launch::ffn_bwd_dact(D, dys, w_down, g_save, u_save, tiles, num_tiles, dg, du, stream));
}

int moe_ffn_bwd_dx(const moe_dims* d, const void* dg, const void* du, const void* w_gate, const void* w_up,
                   const int32_t* tiles, const int32_t* num_tiles, void* dxs, hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(dg, du, w_gate, w_up, tiles, num_tiles, dxs)) return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  return from_hip(moe_launch::ffn_bwd_dx(D, dg, du, w_gate, w_up, tiles, num_tiles, dxs, stream));
}

int moe_ffn_bwd_dw(const moe_dims* d, const void* xs, const void* act, const void* dys, const void* dg,
                   const void* du, const int32_t* offsets, float* dw_gate, float* dw_up, float* dw_down,
                   hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(xs, act, dys, dg, du, offsets, dw_gate, dw_up, dw_down)) return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  return from_hip(
      moe_launch::ffn_bwd_dw(D, xs, nullptr, act, dys, dg, du, offsets, dw_gate, dw_up, dw_down, stream));
}

int moe_ffn_bwd_dx_dw(const moe_dims* d, const void* dg, const void* du, const void* w_gate, const void* w_up,
                      const int32_t* tiles, const int32_t* num_tiles, void* dxs, const void* xs, const void* act,
                      const void* dys, const int32_t* offsets, float* dw_gate, float* dw_up, float* dw_down,
                      hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(dg, du, w_gate, w_up, tiles, num_tiles, dxs, xs, act, dys, offsets, dw_gate, dw_up, dw_down))
    return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  return from_hip(moe_launch::ffn_bwd_dx_dw(D, dg, du, w_gate, w_up, tiles, num_tiles, dxs, xs, nullptr, act, dys, offsets,
                                            dw_gate, dw_up, dw_down, stream));
}

int moe_ffn_bwd_dx_dw_gather(const moe_dims* d, const void* dg, const void* du, const void* w_gate,
                             const void* w_up, const int32_t* tiles, const int32_t* num_tiles, void* dxs,
                             const void* x, const int32_t* sorted_flat, const void* act, const void* dys,
                             const int32_t* offsets, float* dw_gate, float* dw_up, float* dw_down,
                             hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(dg, du, w_gate, w_up, tiles, num_tiles, dxs, x, sorted_flat, act, dys, offsets, dw_gate, dw_up,
               dw_down))
    return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  return from_hip(moe_launch::ffn_bwd_dx_dw(D, dg, du, w_gate, w_up, tiles, num_tiles, dxs, x, sorted_flat, act, dys,
                                            offsets, dw_gate, dw_up, dw_down, stream));
}

int moe_expert_ffn_bwd(const moe_dims* d, const void* dys, const void* xs, const void* w_gate, const void* w_up,
                       const void* w_down, const void* g_save, const void* u_save, const void* act,
                       const int32_t* offsets, const int32_t* tiles, const int32_t* num_tiles, void* dg, void* du,
                       void* dxs, float* dw_gate, float* dw_up, float* dw_down, hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(dys, xs, w_gate, w_up, w_down, g_save, u_save, act, offsets, tiles, num_tiles, dg, du, dxs, dw_gate,
               dw_up, dw_down))
    return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  int st = from_hip(moe_launch::ffn_bwd_dact(D, dys, w_down, g_save, u_save, tiles, num_tiles, dg, du, stream));
  if (st != MOE_OK) return st;
  return from_hip(moe_launch::ffn_bwd_dx_dw(D, dg, du, w_gate, w_up, tiles, num_tiles, dxs, xs, nullptr, act, dys, offsets,
                                            dw_gate, dw_up, dw_down, stream));
}

int moe_permute_bwd(const moe_dims* d, const void* dxs, const int32_t* inv, const int32_t* topk_idx,
                    const float* dlogits, const void* w_r, void* dx, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(dxs, inv, topk_idx, dlogits, w_r, dx)) return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  const size_t need = moe_launch::permute_bwd_ws(D);
  if (ws == nullptr || ws_bytes < need || !aligned16(ws)) return MOE_EWORKSPACE;
  return from_hip(moe_launch::permute_bwd(D, dxs, inv, topk_idx, dlogits, w_r, nullptr, dx, ws, stream, false));
}

int moe_permute_bwd_dense(const moe_dims* d, const void* dxs, const int32_t* inv, const int32_t* topk_idx,
                          const float* dlogits, const void* w_r, void* dx, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(dxs, inv, topk_idx, dlogits, w_r, dx)) return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  const size_t need = moe_launch::permute_bwd_ws(D);
  if (ws == nullptr || ws_bytes < need || !aligned16(ws)) return MOE_EWORKSPACE;
  return from_hip(moe_launch::permute_bwd(D, dxs, inv, topk_idx, dlogits, w_r, nullptr, dx, ws, stream, true));
}

int moe_combine_shared(const moe_dims* d, const void* ys, const float* gates, const int32_t* inv,
                       const void* ys_shared, void* y, hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(ys, gates, inv, ys_shared, y)) return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  return from_hip(moe_launch::combine(D, ys, gates, inv, ys_shared, y, stream));
}

int moe_permute_bwd_add(const moe_dims* d, const void* dxs, const int32_t* inv, const int32_t* topk_idx,
                        const float* dlogits, const void* w_r, int32_t dense, const void* dx_add, void* dx, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(dxs, inv, topk_idx, dlogits, w_r, dx_add, dx)) return MOE_EINVAL;
  if (dense != 0 && dense != 1) return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  const size_t need = moe_launch::permute_bwd_ws(D);
  if (ws == nullptr || ws_bytes < need || !aligned16(ws)) return MOE_EWORKSPACE;
  return from_hip(moe_launch::permute_bwd(D, dxs, inv, topk_idx, dlogits, w_r, dx_add, dx, ws, stream, dense == 1));
}

int moe_shared_ffn(const moe_dims* ds, const void* x, const void* w_gate, const void* w_up, const void* w_down,
                   void* g_save, void* u_save, void* act, void* ys, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_CHECK_DIMS(ds, D);
  if (!is_shared(D)) return MOE_EINVAL;
  if (!ptrs_ok(x, w_gate, w_up, w_down, act, ys)) return MOE_EINVAL;
  if ((g_save == nullptr) != (u_save == nullptr)) return MOE_EINVAL;
  if (g_save != nullptr && !ptrs_ok(g_save, u_save)) return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  const size_t need = moe_launch::shared_ffn_ws(D);
  if (ws == nullptr || ws_bytes < need || !aligned16(ws)) return MOE_EWORKSPACE;
  return from_hip(moe_launch::shared_ffn(D, x, w_gate, w_up, w_down, g_save, u_save, act, ys, ws, stream));
}

int moe_shared_ffn_bwd(const moe_dims* ds, const void* x, const void* dy, const void* w_gate, const void* w_up,
                       const void* w_down, const void* g_save, const void* u_save, const void* act, void* dg, void* du,
                       void* dx_shared, float* dw_gate, float* dw_up, float* dw_down, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  MOE_CHECK_DIMS(ds, D);
  if (!is_shared(D)) return MOE_EINVAL;
  if (!ptrs_ok(x, dy, w_gate, w_up, w_down, g_save, u_save, act, dg, du, dx_shared, dw_gate, dw_up, dw_down))
    return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  const size_t need = moe_launch::shared_ffn_bwd_ws(D);
  if (ws == nullptr || ws_bytes < need || !aligned16(ws)) return MOE_EWORKSPACE;
  return from_hip(moe_launch::shared_ffn_bwd(D, x, dy, w_gate, w_up, w_down, g_save, u_save, act, dg, du, dx_shared,
                                             dw_gate, dw_up, dw_down, ws, stream));
}

int moe_aux_loss(const moe_dims* d, const void* x, const void* w_r, const float* logit_bias, const int32_t* counts,
                 float alpha, float* probs, float* loss, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(x, w_r, counts, probs, loss)) return MOE_EINVAL;
  if (logit_bias != nullptr && !aligned16(logit_bias)) return MOE_EINVAL;
  if (!std::isfinite(alpha)) return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  const size_t need = moe_launch::aux_loss_ws(D);
  if (ws == nullptr || ws_bytes < need || !aligned16(ws)) return MOE_EWORKSPACE;
  return from_hip(moe_launch::aux_loss(D, x, w_r, logit_bias, counts, alpha, probs, loss, ws, stream));
}

int moe_route_bwd_aux(const moe_dims* d, const void* x, const int32_t* topk_idx, const float* gates,
                      const float* dgates, const float* probs, const int32_t* counts, float aux_scale,
                      float* dlogits, float* dw_r, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_CHECK_DIMS(d, D);
  if (!ptrs_ok(x, topk_idx, gates, dgates, probs, counts, dlogits, dw_r)) return MOE_EINVAL;
  if (!std::isfinite(aux_scale)) return MOE_EINVAL;
  if (D.N == 0) return MOE_OK;
  const size_t need = moe_launch::route_bwd_aux_ws(D);
  if (ws == nullptr || ws_bytes < need || !aligned16(ws)) return MOE_EWORKSPACE;
  return from_hip(moe_launch::route_bwd_aux(D, x, topk_idx, gates, dgates, probs, counts, aux_scale, dlogits, dw_r,
                                            ws, stream));
}

}  // extern "C"
