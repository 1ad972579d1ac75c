// Streaming-read calibration kernel for gfx950: the rate at which the chip
// streams a large buffer from HBM with the same 16-byte non-temporal buffer
// loads the decode kernel issues. A decode launch cannot stream its K/V faster than
// this, so it is the achievable ceiling beside the published 8 TB/s (the
// textbook "11.7 KV Cache" §4.4 and the course notes §1.5 put decode on the
// bandwidth roof).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;   // 16-byte loads in flight per thread and iteration
constexpr int kStream = 2;   // non-temporal loads, as the decode kernel's K/V stream

// Thread i reads the 16-byte words i, i + stride, i + 2*stride, ... of its
// 1 GiB window (a buffer resource addresses 32-bit offsets), XOR-folds them
// and stores the fold, so no load can be dropped.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const char* buf, uint64_t words, uint32_t* sink) {
  const uint64_t tid = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kThreads;
  u32x4 acc = u32x4{0u, 0u, 0u, 0u};
  constexpr uint64_t kWindowWords = (1ull << 30) / 16;
  for (uint64_t w0 = 0; w0 < words; w0 += kWindowWords) {
    const uint64_t n = words - w0 < kWindowWords ? words - w0 : kWindowWords;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(buf + w0 * 16), 0, static_cast<int>(n * 16), 0x00020000);
    uint64_t i = tid;
    for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             r, static_cast<int>((i + u * stride) * 16), 0, kStream));
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    for (; i < n; i += stride)
      acc ^= __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(i * 16), 0, kStream));
  }
  sink[tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

extern "C" size_t kvc_stream_read_sink_bytes(int32_t n_workgroups) {
  if (n_workgroups <= 0) return 0;
  return static_cast<size_t>(n_workgroups) * kThreads * sizeof(uint32_t);
}

extern "C" kvc_status_t kvc_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t n_workgroups,
                                        hipStream_t stream) {
  if (buf == nullptr || sink == nullptr) return KVC_ERR_NULL;
  if (n_workgroups <= 0 || bytes % 16 != 0) return KVC_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(buf) % 16) return KVC_ERR_ALIGN;
  if (bytes == 0) return KVC_OK;
  hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<unsigned>(n_workgroups)), dim3(kThreads), 0, stream,
                     static_cast<const char*>(buf), static_cast<uint64_t>(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}
