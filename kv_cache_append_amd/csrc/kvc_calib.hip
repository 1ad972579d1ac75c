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

// The decode launch's data movement without its arithmetic: the workgroups
// and splits of a decode call on this cache (a (sequence, KV head) unit's
// splits on one XCD), the same 16-byte non-temporal K/V loads of 16-row tiles
// one tile ahead, the waves' merge through LDS, and the split exchange (the
// other splits publish a 2 KB partial and raise an epoch flag, the last split
// waits for the flags, folds the partials and writes 2 KB per unit). Every
// loaded word is XOR-folded into the result, so no load can be dropped, and
// the XOR of a unit's output words is the XOR of every 16-byte word of its
// rows (each read once).
struct SplitReadParams {
  const char* k;
  const char* v;
  int64_t sb, sh, st;            // cache strides in bytes
  const int32_t* seq_lens;
  uint32_t* flags;               // [units][S]: word S - 1 is the unit's epoch
  u32x4* partial;                // [units][S][128]
  u32x4* out;                    // [units][128]
  int32_t batch, n_kv, max_len, n_splits, row_bytes;
  int32_t spins;                 // bound on the wait for flags (polls)
};

constexpr int kSrTile = 64;      // rows per workgroup tile: 4 waves x 16
constexpr int kSrWords = 128;    // 16-byte words of a partial and of a unit's output

// NPL: 16-byte slices per lane per row (a row of 4 NPL slices).
template <int NPL>
__global__ __launch_bounds__(kThreads, 2) void split_read_kernel(const SplitReadParams p) {
  const int xcd = blockIdx.x & 7;
  const int r8 = blockIdx.x >> 3;
  const int split = r8 % p.n_splits;
  const int unit = (r8 / p.n_splits) * 8 + xcd;
  if (unit >= p.batch * p.n_kv) return;                 // grid padding
  const int b = unit / p.n_kv;
  const int g = unit - b * p.n_kv;
  const int c0 = p.seq_lens[b];
  const int n = c0 < 0 ? 0 : min(c0 + 1, p.max_len);  // the rows a decode step attends
  uint32_t* const flags = p.flags + static_cast<int64_t>(unit) * p.n_splits;
  uint32_t epoch = 0u;
  if (p.n_splits > 1) epoch = __hip_atomic_load(flags + p.n_splits - 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int chunk = max(16, ((n + p.n_splits - 1) / p.n_splits + 15) & ~15);
  const int ns = n > 0 ? min(p.n_splits, (n + chunk - 1) / chunk) : 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // (uniform: buffer bases stay scalar)
  __shared__ u32x4 sm[4][64];
  __shared__ uint32_t s_ok;
  if (split >= ns) return;                              // inactive split
  const int t0 = split * chunk;
  const int t1 = split == ns - 1 ? n : t0 + chunk;
  // Wave w takes rows 16 w .. 16 w + 15 of each tile. K in the decode
  // kernel's score layout (lane l: 16-byte slices (l / 16) + 4 m of row
  // l % 16), V in its row layout (lane l: slice l % LPR of row
  // 4 m + l / LPR, LPR = 4 NPL lanes per row: whole rows per load).
  const char* const ku = p.k + b * p.sb + g * p.sh;
  const char* const vu = p.v + b * p.sb + g * p.sh;
  const int n_tiles = t1 > t0 ? (t1 - t0 + kSrTile - 1) / kSrTile : 0;
  u32x4 acc = u32x4{0u, 0u, 0u, 0u};
  auto load = [&](int t, u32x4* kk, u32x4* vv) {
    const int base = t0 + t * kSrTile + wave * 16;
    const int rows = t < n_tiles ? t1 - base : 0;
    const uint32_t range = rows > 0 ? static_cast<uint32_t>(rows) * static_cast<uint32_t>(p.st) : 0u;
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(ku + static_cast<int64_t>(base) * p.st), 0, static_cast<int>(range), 0x00020000);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(vu + static_cast<int64_t>(base) * p.st), 0, static_cast<int>(range), 0x00020000);
    constexpr int LPR = 4 * NPL, RPP = 64 / LPR;
#pragma unroll
    for (int m = 0; m < NPL; ++m) {
      const uint32_t koff = static_cast<uint32_t>((lane & 15) * p.st + ((lane >> 4) + 4 * m) * 16);
      kk[m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, static_cast<int>(koff), 0, kStream));
    }
#pragma unroll
    for (int m = 0; m < NPL; ++m) {
      const uint32_t voff = static_cast<uint32_t>((m * RPP + lane / LPR) * p.st + (lane % LPR) * 16);
      vv[m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vr, static_cast<int>(voff), 0, kStream));
    }
  };
  // a ring of two tile buffers, as the decode kernel keeps: tile t + 1's
  // loads leave before the wait for tile t (tiles past the last read zeros)
  u32x4 kbuf[2][NPL], vbuf[2][NPL];
  load(0, kbuf[0], vbuf[0]);
  for (int it = 0; it < n_tiles; it += 2) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      load(it + r + 1, kbuf[r ^ 1], vbuf[r ^ 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < NPL; ++m) acc ^= kbuf[r][m] ^ vbuf[r][m];
    }
  }
  // the waves' merge through LDS; the first 64 words of the partial hold it
  sm[wave][lane] = acc;
  __syncthreads();
  u32x4 word = u32x4{0u, 0u, 0u, 0u};
  if (tid < 64) word = sm[0][tid] ^ sm[1][tid] ^ sm[2][tid] ^ sm[3][tid];
  u32x4* const orow = p.out + static_cast<int64_t>(unit) * kSrWords;
  if (ns == 1) {
    if (tid < kSrWords) orow[tid] = word;
    return;
  }
  u32x4* const prow = p.partial + static_cast<int64_t>(unit) * p.n_splits * kSrWords;
  if (split < ns - 1) {                                 // publish, then raise the flag to epoch + 1
    if (tid < kSrWords) __builtin_nontemporal_store(word, prow + split * kSrWords + tid);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) __hip_atomic_store(flags + split, epoch + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  // the last split: wait for every other split's flag (bounded), fold the
  // partials, write the unit's words and advance the epoch
  if (tid == 0) s_ok = 1u;
  __syncthreads();
  if (tid < ns - 1) {
    uint32_t f = 0u;
    for (int i = 0; i < p.spins; ++i) {
      f = __hip_atomic_load(flags + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (f == epoch + 1u) break;
      __builtin_amdgcn_s_sleep(1);
    }
    if (f != epoch + 1u) atomicAnd(&s_ok, 0u);        // (never expected: the unit's words are then zero)
  }
  __syncthreads();
  if (tid < kSrWords) {
    for (int k = 0; k < ns - 1; ++k) word ^= __builtin_nontemporal_load(prow + k * kSrWords + tid);
    orow[tid] = s_ok ? word : u32x4{0u, 0u, 0u, 0u};
  }
  if (tid == 0) __hip_atomic_store(flags + p.n_splits - 1, epoch + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

extern "C" size_t kvc_split_read_workspace_bytes(const kvc_cache_t* cache, int32_t n_splits) {
  if (cache == nullptr || cache->batch <= 0 || cache->n_kv_heads <= 0 || n_splits <= 0 || n_splits > KVC_MAX_SPLITS)
    return 0;
  const size_t units = static_cast<size_t>(cache->batch) * cache->n_kv_heads;
  const size_t flag_bytes = (units * n_splits * 4 + 255) & ~static_cast<size_t>(255);
  return flag_bytes + units * n_splits * kSrWords * 16;
}

extern "C" kvc_status_t kvc_split_read(const kvc_cache_t* cache, const int32_t* seq_lens, int32_t n_splits,
                                       void* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (cache == nullptr || seq_lens == nullptr || out == nullptr || workspace == nullptr) return KVC_ERR_NULL;
  const int s = cache->dtype == KVC_F32 ? 4 : (cache->dtype == KVC_F16 || cache->dtype == KVC_BF16) ? 2 : 0;
  if (s == 0) return KVC_ERR_DTYPE;
  if (cache->batch <= 0 || cache->n_kv_heads <= 0 || cache->max_len <= 0 || n_splits <= 0 ||
      n_splits > KVC_MAX_SPLITS || cache->stride_t < cache->head_dim)
    return KVC_ERR_SHAPE;
  const int row_bytes = cache->head_dim * s;
  // rows of 4, 8, 16 or 32 16-byte slices (each lane reads 1, 2, 4 or 8 of them per row)
  if (row_bytes != 64 && row_bytes != 128 && row_bytes != 256 && row_bytes != 512) return KVC_ERR_UNSUPPORTED;
  if ((static_cast<int64_t>(cache->max_len) + kSrTile) * cache->stride_t * s > 0x7fffffffll) return KVC_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(cache->k) % 16 || reinterpret_cast<uintptr_t>(cache->v) % 16 ||
      reinterpret_cast<uintptr_t>(out) % 16 || reinterpret_cast<uintptr_t>(workspace) % 256 ||
      (cache->stride_t * s) % 16 || (cache->stride_h * s) % 16 || (cache->stride_b * s) % 16)
    return KVC_ERR_ALIGN;
  if (workspace_bytes < kvc_split_read_workspace_bytes(cache, n_splits)) return KVC_ERR_WORKSPACE;
  const int64_t units = static_cast<int64_t>(cache->batch) * cache->n_kv_heads;
  SplitReadParams p;
  p.k = static_cast<const char*>(cache->k);
  p.v = static_cast<const char*>(cache->v);
  p.sb = cache->stride_b * s;
  p.sh = cache->stride_h * s;
  p.st = cache->stride_t * s;
  p.seq_lens = seq_lens;
  p.flags = static_cast<uint32_t*>(workspace);
  p.partial = reinterpret_cast<u32x4*>(static_cast<char*>(workspace) +
                                       ((units * n_splits * 4 + 255) & ~static_cast<int64_t>(255)));
  p.out = static_cast<u32x4*>(out);
  p.batch = cache->batch;
  p.n_kv = cache->n_kv_heads;
  p.max_len = cache->max_len;
  p.n_splits = n_splits;
  p.row_bytes = row_bytes;
  p.spins = 1 << 20;
  const int64_t wgs = (units + 7) / 8 * 8 * n_splits;
  if (wgs > 0x7fffffffll) return KVC_ERR_SHAPE;
  const dim3 grid(static_cast<unsigned>(wgs)), block(kThreads);
  switch (row_bytes / 64) {
    case 1: hipLaunchKernelGGL(split_read_kernel<1>, grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL(split_read_kernel<2>, grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL(split_read_kernel<4>, grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL(split_read_kernel<8>, grid, block, 0, stream, p); break;
  }
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

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
