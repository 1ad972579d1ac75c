// HIP kernels for gfx950 (CDNA4) and the C-ABI entry points that launch them.
//
// Append / prefill fill: a bit-exact copy of new K/V rows into their slots of
// the preallocated cache (course notes "第 1 周 · Day 4" §3.1, the update of
// the preallocated KVCache; glossary "KV 缓存", path B).
//
// Decode attention: one query per head attends every cached token (textbook
// "11.7 KV Cache" §2.2 single-step decode). It is HBM-bound by construction
// (textbook §1.1 and course notes §1.5: about one FLOP per byte), so the
// kernel is organised around streaming K/V once:
//   * the T axis of every (sequence, KV head) is cut into n_splits chunks,
//     one 256-thread workgroup per chunk (and per block of <= 8 query heads);
//   * within a wave, each cache row of D elements is read by LPR = D*s/16
//     lanes with one 16-byte load each, so one wave-wide load covers 64/LPR
//     whole rows of contiguous memory (fully coalesced);
//   * every lane keeps the q slices of all query heads of its GQA group in
//     registers, so each K/V row is fetched once and used by all of them
//     (course notes §3.4: query head j reads KV head floor(j/(h/G)); no copy);
//   * dot products are reduced across the LPR lanes of a row with DPP row
//     operations; the softmax is online (running max and sum per head, in the
//     log2 domain), rescaled once per tile of rows;
//   * each workgroup writes an fp32 partial (max, sum, unnormalised output);
//     a second kernel merges the partials of every (sequence, query head).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc.h"
#include "kvc_internal.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- copies --

template <int VB> struct VecOf;
template <> struct VecOf<16> { typedef u32x4 type; };
template <> struct VecOf<8> { typedef u32x2 type; };
template <> struct VecOf<4> { typedef uint32_t type; };
template <> struct VecOf<2> { typedef uint16_t type; };

struct CopyParams {
  char* kc;
  char* vc;
  int64_t cb, ch, ct;        // cache strides in bytes
  const char* ks;
  const char* vs;
  int64_t sb, sh, st;        // source strides in bytes
  const int32_t* seq_lens;
  uint32_t* status;
  int32_t batch, n_kv, max_len, t_new;
  int32_t vecs_per_row;      // row bytes / VB
  int64_t total;             // batch * n_kv * t_new * vecs_per_row
};

// Thread i copies one VB-byte vector of K and the same vector of V.
template <int VB>
__global__ __launch_bounds__(256) void copy_rows_kernel(const CopyParams p) {
  typedef typename VecOf<VB>::type V;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < p.total; i += stride) {
    int64_t j = i;
    const int vv = static_cast<int>(j % p.vecs_per_row);
    j /= p.vecs_per_row;
    const int t = static_cast<int>(j % p.t_new);
    j /= p.t_new;
    const int h = static_cast<int>(j % p.n_kv);
    const int b = static_cast<int>(j / p.n_kv);
    const int32_t pos = p.seq_lens[b];
    if (pos < 0 || pos > p.max_len - p.t_new) {
      if (h == 0 && t == 0 && vv == 0 && p.status != nullptr)
        atomicOr(p.status, pos < 0 ? (KVC_DEVERR_BADLEN | KVC_DEVERR_CAPACITY) : KVC_DEVERR_CAPACITY);
      continue;
    }
    const int64_t src = b * p.sb + h * p.sh + t * p.st + static_cast<int64_t>(vv) * VB;
    const int64_t dst = b * p.cb + h * p.ch + static_cast<int64_t>(pos + t) * p.ct + static_cast<int64_t>(vv) * VB;
    const V kx = *reinterpret_cast<const V*>(p.ks + src);
    const V vx = *reinterpret_cast<const V*>(p.vs + src);
    *reinterpret_cast<V*>(p.kc + dst) = kx;
    *reinterpret_cast<V*>(p.vc + dst) = vx;
  }
}

__global__ void advance_kernel(int32_t* seq_lens, int32_t batch, int32_t n) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch) seq_lens[b] += n;
}

// ------------------------------------------------------- element formats --

struct F32T {
  static constexpr int kBytes = 4;
  static constexpr int kPerVec = 4;
  __device__ static inline void unpack(const u32x4 r, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(r[i]);
  }
  __device__ static inline void store(void* base, int64_t i, float x) { static_cast<float*>(base)[i] = x; }
};

struct F16T {
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;
  __device__ static inline void unpack(const u32x4 r, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const _Float16 lo = __builtin_bit_cast(_Float16, static_cast<uint16_t>(r[i] & 0xffffu));
      const _Float16 hi = __builtin_bit_cast(_Float16, static_cast<uint16_t>(r[i] >> 16));
      f[2 * i] = static_cast<float>(lo);
      f[2 * i + 1] = static_cast<float>(hi);
    }
  }
  __device__ static inline void store(void* base, int64_t i, float x) {
    // Pin x as an fp32 register value first: without this the compiler may
    // fuse the producing multiply and the conversion into one mixed-precision
    // op with a single rounding, and the fp16 output would no longer be the
    // fp32 output rounded to nearest even.
    asm volatile("" : "+v"(x));
    static_cast<_Float16*>(base)[i] = static_cast<_Float16>(x);  // round to nearest even
  }
};

struct BF16T {
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;
  __device__ static inline void unpack(const u32x4 r, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(r[i] << 16);
      f[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
  }
  __device__ static inline void store(void* base, int64_t i, float x) {
    // fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
    const uint32_t u = __float_as_uint(x);
    uint16_t h;
    if ((u & 0x7fffffffu) > 0x7f800000u) {
      h = static_cast<uint16_t>((u >> 16) | 0x40u);
    } else {
      h = static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
    }
    static_cast<uint16_t*>(base)[i] = h;
  }
};

// ------------------------------------------------- cross-lane reductions --

template <int CTRL>
__device__ inline float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i within each 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i within each 16 lanes

// Sum over each aligned group of W lanes; every lane of the group gets it.
// After the quad steps all four lanes of a quad hold the same value, so the
// mirror steps (which pair each lane with one in the other quad / half-row)
// complete the butterfly.
template <int W>
__device__ inline float group_sum(float x) {
  if constexpr (W >= 2) x += dpp_f<kDppQuadXor1>(x);
  if constexpr (W >= 4) x += dpp_f<kDppQuadXor2>(x);
  if constexpr (W >= 8) x += dpp_f<kDppHalfMirror>(x);
  if constexpr (W >= 16) x += dpp_f<kDppMirror>(x);
  if constexpr (W >= 32) x += __shfl_xor(x, 16);
  if constexpr (W >= 64) x += __shfl_xor(x, 32);
  return x;
}

// ------------------------------------------------------------ decode attn --

struct DecodeParams {
  const char* k;
  const char* v;
  int64_t sb, sh, st;          // cache strides in bytes
  const int32_t* seq_lens;
  const char* q;               // [B, H_q, D] cache dtype, contiguous
  float* ws_o;                 // [B, H_q, S, D]
  float* ws_ml;                // [B, H_q, S, 2]
  void* out;                   // [B, H_q, D]
  uint32_t* status;
  int32_t batch, n_q, n_kv, group, n_hblk, max_len, n_pending, n_splits;
  float scale_log2;            // softmax scale * log2(e)
};

__device__ inline int tokens_attended(const DecodeParams& p, int b, bool* clamped, bool* bad) {
  int n = p.seq_lens[b];
  *bad = n < 0;
  if (n < 0) n = 0;
  n += p.n_pending;
  *clamped = n > p.max_len;
  if (n > p.max_len) n = p.max_len;
  return n;
}

// Merge two online-softmax states (log2 domain); empty states have m = -inf.
__device__ inline void merge_state(float& m, float& l, float* a, float m2, float l2, const float* a2, int n) {
  const float mn = fmaxf(m, m2);
  const float ref = (mn == -INFINITY) ? 0.f : mn;
  const float c1 = exp2f(m - ref);
  const float c2 = exp2f(m2 - ref);
  l = l * c1 + l2 * c2;
  for (int e = 0; e < n; ++e) a[e] = a[e] * c1 + a2[e] * c2;
  m = mn;
}

template <typename ET, int D, int GB>
__global__ __launch_bounds__(256) void decode_split_kernel(const DecodeParams p) {
  constexpr int EPL = ET::kPerVec;        // elements per lane per row
  constexpr int LPR = D / EPL;            // lanes per row
  constexpr int RPP = 64 / LPR;           // rows per wave pass
  constexpr int NW = 4;                   // waves per workgroup
  constexpr int U = (GB >= 8) ? 2 : 4;    // passes per tile (rescale once per tile)
  static_assert(LPR >= 1 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "row must split into 16-byte lane slices");

  __shared__ float sm_a[NW][GB][D];
  __shared__ float sm_ml[NW][GB][2];

  int bid = blockIdx.x;
  const int split = bid % p.n_splits;
  bid /= p.n_splits;
  const int hb = bid % p.n_hblk;
  const int unit = bid / p.n_hblk;
  const int b = unit / p.n_kv;
  const int g = unit - b * p.n_kv;

  bool clamped, bad;
  const int n = tokens_attended(p, b, &clamped, &bad);
  const int chunk = (n + p.n_splits - 1) / p.n_splits;
  const int t0 = split * chunk;
  if (t0 >= n) return;                    // also n == 0; the merge skips this split
  const int t1 = min(t0 + chunk, n);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane / LPR;             // which row of the pass
  const int li = lane % LPR;              // which 16-byte slice of the row

  const int h_first = g * p.group + hb * GB;
  float qf[GB][EPL];
#pragma unroll
  for (int j = 0; j < GB; ++j) {
    if (hb * GB + j < p.group) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(
          p.q + ((static_cast<int64_t>(b) * p.n_q + h_first + j) * D + li * EPL) * ET::kBytes);
      ET::unpack(raw, qf[j]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[j][e] *= p.scale_log2;
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[j][e] = 0.f;
    }
  }

  float m[GB], l[GB], acc[GB][EPL];
#pragma unroll
  for (int j = 0; j < GB; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[j][e] = 0.f;
  }

  const char* kb = p.k + b * p.sb + g * p.sh + li * 16;
  const char* vb = p.v + b * p.sb + g * p.sh + li * 16;

  // Uniform trip count for the whole wave; rows past t1 are masked per lane group.
  for (int base = t0 + wave * RPP; base < t1; base += NW * RPP * U) {
    u32x4 kr[U], vr[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = base + u * NW * RPP + grp;
      ok[u] = r < t1;
      if (ok[u]) {
        kr[u] = *reinterpret_cast<const u32x4*>(kb + static_cast<int64_t>(r) * p.st);
        vr[u] = *reinterpret_cast<const u32x4*>(vb + static_cast<int64_t>(r) * p.st);
      } else {
        kr[u] = u32x4{0u, 0u, 0u, 0u};
        vr[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    float s[GB][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[EPL];
      ET::unpack(kr[u], kf);
#pragma unroll
      for (int j = 0; j < GB; ++j) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) d = fmaf(qf[j][e], kf[e], d);
        d = group_sum<LPR>(d);
        s[j][u] = ok[u] ? d : -INFINITY;
      }
    }
    float vf[U][EPL];
#pragma unroll
    for (int u = 0; u < U; ++u) ET::unpack(vr[u], vf[u]);
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      float mt = s[j][0];
#pragma unroll
      for (int u = 1; u < U; ++u) mt = fmaxf(mt, s[j][u]);
      const float mn = fmaxf(m[j], mt);
      const float ref = (mn == -INFINITY) ? 0.f : mn;
      const float corr = exp2f(m[j] - ref);
      float pu[U];
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        pu[u] = exp2f(s[j][u] - ref);
        ps += pu[u];
      }
      l[j] = l[j] * corr + ps;
      m[j] = mn;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float a = acc[j][e] * corr;
#pragma unroll
        for (int u = 0; u < U; ++u) a = fmaf(pu[u], vf[u][e], a);
        acc[j][e] = a;
      }
    }
  }

  // Merge the RPP lane groups of this wave (lanes li, li+LPR, li+2*LPR, ...).
#pragma unroll
  for (int off = LPR; off < 64; off *= 2) {
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      const float m2 = __shfl_xor(m[j], off);
      const float l2 = __shfl_xor(l[j], off);
      float a2[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) a2[e] = __shfl_xor(acc[j][e], off);
      merge_state(m[j], l[j], acc[j], m2, l2, a2, EPL);
    }
  }
  if (lane < LPR) {
#pragma unroll
    for (int j = 0; j < GB; ++j) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_a[wave][j][li * EPL + e] = acc[j][e];
      if (lane == 0) {
        sm_ml[wave][j][0] = m[j];
        sm_ml[wave][j][1] = l[j];
      }
    }
  }
  __syncthreads();

  // Merge the NW waves and write this split's partial for each valid head.
  for (int t = threadIdx.x; t < GB * D; t += blockDim.x) {
    const int j = t / D;
    const int d = t - j * D;
    if (hb * GB + j >= p.group) continue;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mm = fmaxf(mm, sm_ml[w][j][0]);
    const float ref = (mm == -INFINITY) ? 0.f : mm;
    float ll = 0.f, aa = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float c = exp2f(sm_ml[w][j][0] - ref);
      ll += sm_ml[w][j][1] * c;
      aa += sm_a[w][j][d] * c;
    }
    const int64_t row = (static_cast<int64_t>(b) * p.n_q + h_first + j) * p.n_splits + split;
    p.ws_o[row * D + d] = aa;
    if (d == 0) {
      p.ws_ml[row * 2] = mm;
      p.ws_ml[row * 2 + 1] = ll;
    }
  }
}

// One workgroup per (sequence, query head): merge the active splits' partials
// (log-sum-exp over the per-split maxima) and write the normalised output.
template <typename OT>
__global__ __launch_bounds__(256) void decode_merge_kernel(const DecodeParams p, int D) {
  const int b = blockIdx.x / p.n_q;
  const int h = blockIdx.x - b * p.n_q;
  bool clamped, bad;
  const int n = tokens_attended(p, b, &clamped, &bad);
  if (h == 0 && threadIdx.x == 0 && p.status != nullptr && (clamped || bad))
    atomicOr(p.status, (clamped ? KVC_DEVERR_CAPACITY : 0u) | (bad ? KVC_DEVERR_BADLEN : 0u));
  const int64_t orow = (static_cast<int64_t>(b) * p.n_q + h) * D;
  if (n <= 0) {
    for (int d = threadIdx.x; d < D; d += blockDim.x) OT::store(p.out, orow + d, 0.f);
    return;
  }
  const int chunk = (n + p.n_splits - 1) / p.n_splits;
  const int ns = (n + chunk - 1) / chunk;
  const int64_t row0 = (static_cast<int64_t>(b) * p.n_q + h) * p.n_splits;
  float mm = -INFINITY;
  for (int i = 0; i < ns; ++i) mm = fmaxf(mm, p.ws_ml[(row0 + i) * 2]);
  float ll = 0.f;
  for (int i = 0; i < ns; ++i) ll += p.ws_ml[(row0 + i) * 2 + 1] * exp2f(p.ws_ml[(row0 + i) * 2] - mm);
  const float inv = 1.f / ll;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float a = 0.f;
    for (int i = 0; i < ns; ++i) a += p.ws_o[(row0 + i) * D + d] * exp2f(p.ws_ml[(row0 + i) * 2] - mm);
    OT::store(p.out, orow + d, a * inv);
  }
}

// ------------------------------------------------------------- dispatch --

typedef void (*SplitKernel)(const DecodeParams);

template <typename ET, int D>
SplitKernel pick_gb(int gb) {
  switch (gb) {
    case 1: return decode_split_kernel<ET, D, 1>;
    case 2: return decode_split_kernel<ET, D, 2>;
    case 4: return decode_split_kernel<ET, D, 4>;
    default: return decode_split_kernel<ET, D, 8>;
  }
}

template <typename ET>
SplitKernel pick_d(int d, int gb) {
  switch (d) {
    case 4: if constexpr (ET::kBytes * 4 >= 16) return pick_gb<ET, 4>(gb); else return nullptr;
    case 8: return pick_gb<ET, 8>(gb);
    case 16: return pick_gb<ET, 16>(gb);
    case 32: return pick_gb<ET, 32>(gb);
    case 64: return pick_gb<ET, 64>(gb);
    case 128: return pick_gb<ET, 128>(gb);
    case 256: return pick_gb<ET, 256>(gb);
    default: return nullptr;
  }
}

SplitKernel pick_split_kernel(int dtype, int d, int gb) {
  switch (dtype) {
    case KVC_F32: return pick_d<F32T>(d, gb);
    case KVC_F16: return pick_d<F16T>(d, gb);
    case KVC_BF16: return pick_d<BF16T>(d, gb);
    default: return nullptr;
  }
}

kvc_status_t launch_copy(const kvc_cache_t* c, const int32_t* seq_lens, const void* ks, const void* vs,
                         int64_t sb, int64_t sh, int64_t st, int32_t t_new, uint32_t* status,
                         hipStream_t stream) {
  const int s = kvc::elem_bytes(c->dtype);
  CopyParams p;
  p.kc = static_cast<char*>(c->k);
  p.vc = static_cast<char*>(c->v);
  p.cb = c->stride_b * s;
  p.ch = c->stride_h * s;
  p.ct = c->stride_t * s;
  p.ks = static_cast<const char*>(ks);
  p.vs = static_cast<const char*>(vs);
  p.sb = sb * s;
  p.sh = sh * s;
  p.st = st * s;
  p.seq_lens = seq_lens;
  p.status = status;
  p.batch = c->batch;
  p.n_kv = c->n_kv_heads;
  p.max_len = c->max_len;
  p.t_new = t_new;
  const int64_t src_strides[3] = {p.sb, p.sh, p.st};
  const int vb = kvc::copy_vector_bytes(c, ks, vs, src_strides, 3);
  p.vecs_per_row = static_cast<int32_t>((static_cast<int64_t>(c->head_dim) * s) / vb);
  p.total = static_cast<int64_t>(c->batch) * c->n_kv_heads * t_new * p.vecs_per_row;
  if (p.total == 0) return KVC_OK;
  const int threads = 256;
  int64_t blocks = (p.total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;   // grid-stride loop covers the rest
  const dim3 grid(static_cast<unsigned>(blocks)), block(threads);
  switch (vb) {
    case 16: hipLaunchKernelGGL(copy_rows_kernel<16>, grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL(copy_rows_kernel<8>, grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL(copy_rows_kernel<4>, grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL(copy_rows_kernel<2>, grid, block, 0, stream, p); break;
  }
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

}  // namespace

// ------------------------------------------------------------ C ABI calls --

extern "C" kvc_status_t kvc_append(const kvc_cache_t* cache, const int32_t* seq_lens, const void* k_new,
                                   const void* v_new, int64_t new_stride_b, int64_t new_stride_h,
                                   uint32_t* dev_status, hipStream_t stream) {
  kvc_status_t st = kvc::check_cache(cache, false);
  if (st != KVC_OK) return st;
  if (cache->batch == 0) return KVC_OK;
  if (seq_lens == nullptr || k_new == nullptr || v_new == nullptr) return KVC_ERR_NULL;
  if (new_stride_b < 0 || new_stride_h < 0) return KVC_ERR_SHAPE;
  if (cache->n_kv_heads > 1 && new_stride_h < cache->head_dim) return KVC_ERR_SHAPE;
  const int s = kvc::elem_bytes(cache->dtype);
  if (reinterpret_cast<uintptr_t>(k_new) % s || reinterpret_cast<uintptr_t>(v_new) % s) return KVC_ERR_ALIGN;
  return launch_copy(cache, seq_lens, k_new, v_new, new_stride_b, new_stride_h, 0, 1, dev_status, stream);
}

extern "C" kvc_status_t kvc_prefill_fill(const kvc_cache_t* cache, const int32_t* seq_lens, const void* k,
                                         const void* v, int64_t src_stride_b, int64_t src_stride_h,
                                         int64_t src_stride_t, int32_t t_new, uint32_t* dev_status,
                                         hipStream_t stream) {
  kvc_status_t st = kvc::check_cache(cache, false);
  if (st != KVC_OK) return st;
  if (t_new < 0) return KVC_ERR_SHAPE;
  if (cache->batch == 0 || t_new == 0) return KVC_OK;
  if (seq_lens == nullptr || k == nullptr || v == nullptr) return KVC_ERR_NULL;
  if (src_stride_b < 0 || src_stride_h < 0 || src_stride_t < 0) return KVC_ERR_SHAPE;
  if (t_new > 1 && src_stride_t < cache->head_dim) return KVC_ERR_SHAPE;
  const int s = kvc::elem_bytes(cache->dtype);
  if (reinterpret_cast<uintptr_t>(k) % s || reinterpret_cast<uintptr_t>(v) % s) return KVC_ERR_ALIGN;
  return launch_copy(cache, seq_lens, k, v, src_stride_b, src_stride_h, src_stride_t, t_new, dev_status, stream);
}

extern "C" kvc_status_t kvc_decode_attn(const kvc_cache_t* cache, const int32_t* seq_lens, int32_t n_pending,
                                        const void* q, int32_t n_q_heads, float scale, void* out,
                                        int32_t out_dtype, void* workspace, size_t workspace_bytes,
                                        int32_t n_splits, uint32_t* dev_status, hipStream_t stream) {
  kvc_status_t st = kvc::check_cache(cache, true);
  if (st != KVC_OK) return st;
  if (n_q_heads <= 0 || n_q_heads % cache->n_kv_heads != 0) return KVC_ERR_GQA;
  if (n_pending < 0 || n_splits < 0) return KVC_ERR_SHAPE;
  if (out_dtype != KVC_F32 && out_dtype != cache->dtype) return KVC_ERR_DTYPE;
  if (!kvc::decode_head_dim_supported(cache->head_dim, cache->dtype)) return KVC_ERR_UNSUPPORTED;
  if (cache->batch == 0) return KVC_OK;
  if (seq_lens == nullptr || q == nullptr || out == nullptr) return KVC_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(q) % 16) return KVC_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(out) % kvc::elem_bytes(out_dtype)) return KVC_ERR_ALIGN;
  const int32_t splits = n_splits > 0 ? n_splits : kvc::auto_splits(cache, n_q_heads);
  const size_t need = kvc::workspace_bytes(cache, n_q_heads, splits);
  if (workspace == nullptr || workspace_bytes < need) return KVC_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 16) return KVC_ERR_ALIGN;

  const int s = kvc::elem_bytes(cache->dtype);
  const int group = n_q_heads / cache->n_kv_heads;
  const int gb = kvc::heads_per_block(group);
  DecodeParams p;
  p.k = static_cast<const char*>(cache->k);
  p.v = static_cast<const char*>(cache->v);
  p.sb = cache->stride_b * s;
  p.sh = cache->stride_h * s;
  p.st = cache->stride_t * s;
  p.seq_lens = seq_lens;
  p.q = static_cast<const char*>(q);
  p.ws_o = static_cast<float*>(workspace);
  p.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                     kvc::workspace_ml_offset(cache, n_q_heads, splits));
  p.out = out;
  p.status = dev_status;
  p.batch = cache->batch;
  p.n_q = n_q_heads;
  p.n_kv = cache->n_kv_heads;
  p.group = group;
  p.n_hblk = kvc::head_blocks(group);
  p.max_len = cache->max_len;
  p.n_pending = n_pending;
  p.n_splits = splits;
  p.scale_log2 = scale * 1.44269504088896340736f;  // log2(e)

  SplitKernel k = pick_split_kernel(cache->dtype, cache->head_dim, gb);
  if (k == nullptr) return KVC_ERR_UNSUPPORTED;
  const int64_t wgs = static_cast<int64_t>(cache->batch) * cache->n_kv_heads * p.n_hblk * splits;
  if (wgs > 0x7fffffffll) return KVC_ERR_SHAPE;
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(wgs)), dim3(256), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return KVC_ERR_HIP;
  const dim3 mgrid(static_cast<unsigned>(cache->batch * n_q_heads));
  const dim3 mblock(cache->head_dim >= 256 ? 256 : (cache->head_dim >= 64 ? cache->head_dim : 64));
  switch (out_dtype) {
    case KVC_F32: hipLaunchKernelGGL(decode_merge_kernel<F32T>, mgrid, mblock, 0, stream, p, cache->head_dim); break;
    case KVC_F16: hipLaunchKernelGGL(decode_merge_kernel<F16T>, mgrid, mblock, 0, stream, p, cache->head_dim); break;
    default: hipLaunchKernelGGL(decode_merge_kernel<BF16T>, mgrid, mblock, 0, stream, p, cache->head_dim); break;
  }
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

extern "C" kvc_status_t kvc_seq_lens_advance(int32_t* seq_lens, int32_t batch, int32_t n, hipStream_t stream) {
  if (batch < 0) return KVC_ERR_SHAPE;
  if (batch == 0) return KVC_OK;
  if (seq_lens == nullptr) return KVC_ERR_NULL;
  hipLaunchKernelGGL(advance_kernel, dim3((batch + 255) / 256), dim3(256), 0, stream, seq_lens, batch, n);
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}
