// kvc_decode_step_noalloc: the decode step (append + attention, one launch)
// for callers that cannot allocate device memory, such as code under HIP
// graph capture or serving loops that forbid hipMalloc. The split exchange
// (ready flags and partial results) that kvc_decode_step keeps in the
// caller's workspace lives here in a device array of this file instead.
//
// The array is one copy per GPU, allocated when the library is loaded there
// and held until the process ends. Ready flags come first, one row of
// KVC_MAX_SPLITS words per (sequence, KV head, head block), so that every
// row's epoch word (its last) stays in place whatever the geometry of the
// calls: flags only ever hold epoch values and an epoch only grows, so a
// flag left by an earlier call, of any geometry, never equals what a later
// call waits for. The wide-group kernel's merge words come next, one row of
// 64 per (sequence, KV head) at a fixed stride, which holds its own epoch
// beside the claim words compared with it, so that stale claims are told
// apart the same way whatever the geometry; its arrival count is back at
// zero after every call. The partial outputs and (reference, sum) pairs
// follow, rewritten by every call before they are read. The array is zero at load,
// the state the epoch protocol starts from. Calls that overlap on one GPU
// (two streams at once) share the array and race.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "kvc.h"
#include "kvc_internal.h"

// The array's size in MiB and the (sequence, KV head, head block) rows its
// flag region holds.
#define KVC_NOALLOC_SCRATCH_MIB 16
#define KVC_NOALLOC_MAX_ROWS 2048

namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(KVC_NOALLOC_SCRATCH_MIB) << 20;
constexpr size_t kScratchFlagBytes = static_cast<size_t>(KVC_NOALLOC_MAX_ROWS) * KVC_MAX_SPLITS * 4;
constexpr size_t kScratchSyncBytes = static_cast<size_t>(KVC_NOALLOC_MAX_ROWS) * kvc::kWideSyncBytes;
constexpr size_t kScratchHeadBytes = kScratchFlagBytes + kScratchSyncBytes;
static_assert(kScratchFlagBytes % 256 == 0 && kScratchSyncBytes % 256 == 0 && kScratchHeadBytes < kScratchBytes,
              "scratch layout");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch[kMaxDevices] = {};    // the array's device address on each GPU

// The current device's copy of the array. Its address comes from
// hipGetSymbolAddress, once per device with that device current; in host
// code `scratch` only names the array, and kernels are given this address.
kvc_status_t scratch_on_current_device(uint8_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVC_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return KVC_ERR_HIP;
    g_scratch[dev] = static_cast<uint8_t*>(ptr);
  }
  *out = g_scratch[dev];
  return KVC_OK;
}

// The array laid out for one call; KVC_ERR_WORKSPACE when the call needs more
// flag rows or more partial bytes than it holds.
kvc_status_t noalloc_regions(const kvc_cache_t* c, int32_t n_q_heads, int32_t splits, kvc::WsRegions* r) {
  const int64_t rows = static_cast<int64_t>(c->batch) * c->n_kv_heads * kvc::head_blocks(n_q_heads / c->n_kv_heads);
  const int64_t prows = static_cast<int64_t>(c->batch) * n_q_heads * splits;
  const int64_t o_bytes = (prows * c->head_dim * 4 + 255) & ~int64_t{255};
  const int64_t ml_bytes = (prows * 8 + 255) & ~int64_t{255};
  if (rows > KVC_NOALLOC_MAX_ROWS ||
      static_cast<int64_t>(kScratchHeadBytes) + o_bytes + ml_bytes > static_cast<int64_t>(kScratchBytes))
    return KVC_ERR_WORKSPACE;
  uint8_t* base = nullptr;
  const kvc_status_t st = scratch_on_current_device(&base);
  if (st != KVC_OK) return st;
  r->flags = reinterpret_cast<uint32_t*>(base);
  r->flag_stride = KVC_MAX_SPLITS;
  r->sync = reinterpret_cast<uint32_t*>(base + kScratchFlagBytes);   // (sequence, KV head) rows <= rows
  r->o = reinterpret_cast<float*>(base + kScratchHeadBytes);
  r->ml = reinterpret_cast<float*>(base + kScratchHeadBytes + o_bytes);
  return KVC_OK;
}

}  // namespace

extern "C" kvc_status_t kvc_decode_step_noalloc(const kvc_cache_t* cache, const int32_t* seq_lens,
                                                const void* k_new, const void* v_new, int64_t new_stride_b,
                                                int64_t new_stride_h, const void* q, int32_t n_q_heads, float scale,
                                                void* out, int32_t out_dtype, int32_t n_splits,
                                                uint32_t* dev_status, hipStream_t stream) {
  if (cache != nullptr && cache->batch > 0 && (k_new == nullptr || v_new == nullptr)) return KVC_ERR_NULL;
  return kvc::decode_step_in_regions(cache, seq_lens, k_new, v_new, new_stride_b, new_stride_h, q, n_q_heads, scale,
                                     out, out_dtype, n_splits, dev_status, stream, noalloc_regions);
}
