// moe_route_meta for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc): the
// router's block histograms (or the unfused metadata's chunk histograms) live
// in a file-scope device array instead of a caller workspace.
//
// Every GPU the library runs on holds its own copy of `scratch` until the
// process ends.  Its device address is looked up once per device, with that
// device current, on the first call on that device; host code uses that
// address only (the array's name in host code is a host-side stand-in).
// Every byte of scratch a call reads is written earlier by the same call, so
// nothing needs clearing between calls; calls that overlap on one GPU share
// the array and race.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "common.h"
#include "moe.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_init;

// Device address of this device's scratch (the current device), or nullptr
// when the lookup fails.
void* device_scratch(int dev) {
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_init);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) return nullptr;
    p = addr;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" int moe_route_meta_noalloc(const moe_dims* d, const void* x, const void* w_r, const float* logit_bias,
                                      int32_t capacity, int32_t* topk_idx, float* gates, int32_t* sorted_flat,
                                      int32_t* inv, int32_t* counts, int32_t* offsets, int32_t* tiles,
                                      int32_t* num_tiles, hipStream_t stream) {
  const size_t need = moe_workspace_bytes(d, MOE_ENTRY_ROUTE_META);
  if (need == size_t(-1) || d->N == 0)  // invalid dims, or nothing to do: moe_route_meta's own answer
    return moe_route_meta(d, x, w_r, logit_bias, capacity, topk_idx, gates, sorted_flat, inv, counts, offsets,
                          tiles, num_tiles, nullptr, 0, stream);
  if (need > size_t(MOE_NOALLOC_SCRATCH_BYTES)) return MOE_ESCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EHIP;
  void* ws = device_scratch(dev);
  if (ws == nullptr) return MOE_EHIP;
  return moe_route_meta(d, x, w_r, logit_bias, capacity, topk_idx, gates, sorted_flat, inv, counts, offsets, tiles,
                        num_tiles, ws, size_t(MOE_NOALLOC_SCRATCH_BYTES), stream);
}
