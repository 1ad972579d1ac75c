// HIP kernels for gfx950 (CDNA4) and the C-ABI entry points that launch them.
//
// Append / prefill fill: a bit-exact copy of new K/V rows into their slots of
// the preallocated cache (course notes "第 1 周 · Day 4" §3.1, the update of
// the preallocated KVCache; glossary "KV 缓存", path B).
//
// Decode attention: one query per head attends every cached token (textbook
// "11.7 KV Cache" §2.2 single-step decode). It is HBM-bound by construction
// (textbook §1.1 and course notes §1.5: about one FLOP per byte), so the
// kernel is organised around streaming K/V exactly once, in one launch:
//   * the T axis of every (sequence, KV head) is cut into n_splits chunks,
//     one 256-thread workgroup per chunk (and per block of <= 8 query heads);
//   * K/V tiles are read through buffer resources whose range ends at the
//     last row to stream (rows past it read as zero), with a register ring
//     keeping the next tiles' loads in flight;
//   * every K/V row is fetched once for all query heads of its group (course
//     notes §3.4: query head j reads KV head floor(j/(h/G)); no copy);
//   * 16-bit caches run on the matrix cores: 16 rows x (up to) 16 heads of
//     scores per v_mfma_f32_16x16x32 chain, weights through LDS to the row
//     layout of V, and P.V on v_mfma_f32_4x4x1_16b_f32 (fp32 weights) for
//     4+ heads; fp32 caches take a vector-ALU path with 2-way dot products
//     and DPP reductions;
//   * the softmax is online in the log2 domain with a lazily moved reference:
//     it only moves when a score exceeds it by more than 2^8, so the
//     accumulators are rarely rescaled (exact in real arithmetic, bounded
//     exponentials in fp32);
//   * with several splits, every split but the last publishes its partial
//     (reference, sum, unnormalised output) in the workspace and raises a
//     ready flag; the last split's workgroup waits for those flags, merges
//     the partials in split order (bit-identical results run to run) and
//     writes the normalised output, then leaves the flags at zero;
//   * kvc_decode_step additionally takes the step's k_t, v_t: the workgroup
//     whose chunk holds slot T_b reads that row from k_t/v_t and writes it
//     into the cache, so append and attention share the launch.
#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

#include "kvc.h"
#include "kvc_internal.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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
  // paged cache (table != null): cb is the page stride; slot t of sequence b
  // is row t & (page_size - 1) of page table[b * table_stride + (t >> page_shift)]
  const int32_t* table;
  int32_t table_stride, page_shift, n_pages;

  // ring cache (ring != 0): token number pos + t goes to slot (pos + t) % max_len;
  // of a block longer than the ring only its last max_len rows are written
  int32_t ring;
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
    if (p.ring) {
      if (pos < 0) {
        if (h == 0 && t == 0 && vv == 0 && p.status != nullptr) atomicOr(p.status, KVC_DEVERR_BADLEN);
        continue;
      }
      if (t < p.t_new - p.max_len) continue;    // overwritten by a later row of the same block
      const int slot = static_cast<int>((static_cast<int64_t>(pos) + t) % p.max_len);
      const int64_t src = b * p.sb + h * p.sh + t * p.st + static_cast<int64_t>(vv) * VB;
      const int64_t dst = b * p.cb + h * p.ch + static_cast<int64_t>(slot) * p.ct + static_cast<int64_t>(vv) * VB;
      *reinterpret_cast<V*>(p.kc + dst) = *reinterpret_cast<const V*>(p.ks + src);
      *reinterpret_cast<V*>(p.vc + dst) = *reinterpret_cast<const V*>(p.vs + src);
      continue;
    }
    if (pos < 0 || pos > p.max_len - p.t_new) {
      if (h == 0 && t == 0 && vv == 0 && p.status != nullptr)
        atomicOr(p.status, pos < 0 ? (KVC_DEVERR_BADLEN | KVC_DEVERR_CAPACITY) : KVC_DEVERR_CAPACITY);
      continue;
    }
    const int64_t src = b * p.sb + h * p.sh + t * p.st + static_cast<int64_t>(vv) * VB;
    int64_t dst;
    if (p.table != nullptr) {
      const int slot = pos + t;
      const int pg = p.table[static_cast<int64_t>(b) * p.table_stride + (slot >> p.page_shift)];
      if (pg < 0 || pg >= p.n_pages) {
        if (h == 0 && vv == 0 && p.status != nullptr) atomicOr(p.status, KVC_DEVERR_PAGE);
        continue;
      }
      dst = pg * p.cb + h * p.ch + static_cast<int64_t>(slot & ((1 << p.page_shift) - 1)) * p.ct +
            static_cast<int64_t>(vv) * VB;
    } else {
      dst = b * p.cb + h * p.ch + static_cast<int64_t>(pos + t) * p.ct + static_cast<int64_t>(vv) * VB;
    }
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
  // q.k over this lane's 4 elements
  __device__ static inline float dot(const u32x4 q, const u32x4 k, float d) {
#pragma unroll
    for (int i = 0; i < 4; ++i) d = fmaf(__uint_as_float(q[i]), __uint_as_float(k[i]), d);
    return d;
  }
  __device__ static inline void store(void* base, int64_t i, float x) { static_cast<float*>(base)[i] = x; }
};

struct F16T {
  static constexpr bool kIsF16 = true;
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
  // q.k over this lane's 8 elements: four 2-way fp16 dot products, fp32 sum.
  // (The whole vector is bit-cast once: casting single lanes of the uint
  // vector inside a loop was compiled to four uses of lane 0.)
  // C += A * B on 16x16x32 tiles; each lane passes its 8-element slices of A and B.
  __device__ static inline f32x4 mfma16(const u32x4 a, const u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c,
                                                  0, 0, 0);
  }
  __device__ static inline float dot(const u32x4 q, const u32x4 k, float d) {
    const half8_t a = __builtin_bit_cast(half8_t, q);
    const half8_t b = __builtin_bit_cast(half8_t, k);
    d = __builtin_amdgcn_fdot2(a.s01, b.s01, d, false);
    d = __builtin_amdgcn_fdot2(a.s23, b.s23, d, false);
    d = __builtin_amdgcn_fdot2(a.s45, b.s45, d, false);
    return __builtin_amdgcn_fdot2(a.s67, b.s67, d, false);
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
  static constexpr bool kIsF16 = false;
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;
  __device__ static inline void unpack(const u32x4 r, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(r[i] << 16);
      f[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
  }
  // q.k over this lane's 8 elements: four 2-way bf16 dot products, fp32 sum
  __device__ static inline f32x4 mfma16(const u32x4 a, const u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  }
  __device__ static inline float dot(const u32x4 q, const u32x4 k, float d) {
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, q);
    const bf16x8_t b = __builtin_bit_cast(bf16x8_t, k);
    d = __builtin_amdgcn_fdot2_f32_bf16(a.s01, b.s01, d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(a.s23, b.s23, d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(a.s45, b.s45, d, false);
    return __builtin_amdgcn_fdot2_f32_bf16(a.s67, b.s67, d, false);
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

constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i within each 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i within each 16 lanes

// Sum over each aligned group of W lanes; every lane of the group gets it.
// After the quad steps all four lanes of a quad hold the same value, so the
// mirror steps (which pair each lane with one in the other quad / half-row)
// complete the butterfly.
// The same butterfly on N independent values, one step across all of them
// at a time, so no DPP op reads the result of the VALU op just before it.
template <int W, int N>
__device__ inline void group_sum_n(float (&x)[N]) {
  if constexpr (W >= 2) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f<kDppQuadXor1>(x[i]);
  }
  if constexpr (W >= 4) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f<kDppQuadXor2>(x[i]);
  }
  if constexpr (W >= 8) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f<kDppHalfMirror>(x[i]);
  }
  if constexpr (W >= 16) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f<kDppMirror>(x[i]);
  }
  if constexpr (W >= 32) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += __shfl_xor(x[i], 16);
  }
  if constexpr (W >= 64) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += __shfl_xor(x[i], 32);
  }
}

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

// Maximum / sum over each aligned group of 16 lanes (a DPP row); every lane
// of the group gets the result.
__device__ inline float row16_max(float x) {
  x = fmaxf(x, dpp_f<kDppQuadXor1>(x));
  x = fmaxf(x, dpp_f<kDppQuadXor2>(x));
  x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
  return fmaxf(x, dpp_f<kDppMirror>(x));
}
__device__ inline float lane_value(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// ------------------------------------------------------------ decode attn --

struct DecodeParams {
  char* k;                     // cache; written only by the fused append
  char* v;
  int64_t sb, sh, st;          // cache strides in bytes
  const int32_t* seq_lens;
  const char* q;               // [B, H_q, D] cache dtype, contiguous
  const char* k_new;           // fused append source [B, H_kv, D] or null
  const char* v_new;
  int64_t nsb, nsh;            // its strides in bytes
  uint32_t* ws_flag;           // [B * H_kv * n_hblk, flag_stride] ready flags; a row's last word is its epoch
  float* ws_o;                 // [B, H_q, S, D]
  float* ws_ml;                // [B, H_q, S, 2]
  void* out;                   // [B, H_q, D]
  uint32_t* status;
  int32_t batch, n_q, n_kv, group, n_hblk, max_len, n_pending, n_splits, out_f32;
  // Block of new queries (kvc_block_attn): t_q queries per sequence, query i
  // attending slots 0..seq_lens[b] + i. The t_q * group (query, head) pairs
  // of a KV head play the role of its query heads; pair v is query v / group
  // of head v % group. Decode has t_q = 1 and block = 0.
  int32_t t_q, block;
  // Paged cache (table != null): sb is the page stride, and the 16-row tile
  // starting at slot r lives in page table[b * table_stride + (r >> page_shift)].
  const int32_t* table;
  int32_t table_stride, page_shift, n_pages;
  // Ring cache (ring != 0): max_len slots hold the most recent max_len
  // tokens, token number t in slot t % max_len; decode attends
  // min(seq_lens[b] + n_pending, max_len) slots.
  int32_t ring;
  // Quantised cache (8-bit codes): fp32 scales per token of K and of V,
  // [B, H_kv, T_max] with byte strides ssb, ssh and 4 bytes per token.
  char* k_scale;                 // written only by the fused append
  char* v_scale;
  int64_t ssb, ssh;
  float scale_log2;            // softmax scale * log2(e)
  int32_t merge_spins;         // bound on the split merge's wait for ready flags (polls)
  int32_t flag_stride;         // words per flag row (>= n_splits)
  int32_t* lens_next;          // kvc_decode_step_advance: seq_lens[b] + 1 written here, or null
};

struct SeqInfo {
  int n;           // tokens attended
  int append_row;  // slot the fused append writes, or -1
  int newest;      // slot of the newest attended token (ring caches; else n - 1)
  uint32_t flags;  // KVC_DEVERR_* bits
};

__device__ inline SeqInfo seq_info(const DecodeParams& p, int c0) {
  SeqInfo si;
  si.flags = 0;
  const int c = c0 < 0 ? 0 : c0;
  if (c0 < 0) si.flags |= KVC_DEVERR_BADLEN;
  si.append_row = -1;
  // lengths plus new tokens are summed in 64 bits: a length near 2^31 is a
  // capacity case, not a wrapped negative count
  const int add = p.k_new != nullptr ? 1 : (p.block ? p.t_q : p.n_pending);
  const int64_t n64 = static_cast<int64_t>(c) + add;
  if (p.ring) {                   // sliding window: no capacity limit, the ring wraps
    if (c0 >= 0 && p.k_new != nullptr) si.append_row = c0 % p.max_len;
    const int n = c0 < 0 ? 0 : static_cast<int>(min(n64, static_cast<int64_t>(p.max_len)));
    si.n = n;
    si.newest = c0 < 0 ? -1 : static_cast<int>((n64 - 1) % p.max_len);
    return si;
  }
  if (p.block) {                  // the whole block must fit: else flagged, zero rows
    if (c0 >= 0 && n64 > p.max_len) si.flags |= KVC_DEVERR_CAPACITY;
    si.n = (c0 < 0 || n64 > p.max_len) ? 0 : static_cast<int>(n64);
    si.newest = si.n - 1;
    return si;
  }
  if (p.k_new != nullptr) {
    if (c0 >= 0 && c0 < p.max_len) si.append_row = c0;
    else si.flags |= KVC_DEVERR_CAPACITY;
  }
  int n = static_cast<int>(min(n64, static_cast<int64_t>(p.max_len)));
  if (n64 > p.max_len) si.flags |= KVC_DEVERR_CAPACITY;
  if (c0 < 0) n = 0;               // a negative length: a zero row, nothing attended
  si.n = n;
  si.newest = n - 1;
  return si;
}

template <typename ET>
__device__ inline void store_out(const DecodeParams& p, int64_t idx, float x) {
  if (p.out_f32) F32T::store(p.out, idx, x);
  else ET::store(p.out, idx, x);
}

// Byte offset of slot `row` of (sequence b, KV head g) in the cache or page
// pool, or -1 when its page-table entry is not in the pool.
__device__ inline int64_t slot_offset(const DecodeParams& p, int b, int g, int row) {
  if (p.table == nullptr) return b * p.sb + g * p.sh + static_cast<int64_t>(row) * p.st;
  const int pg = p.table[static_cast<int64_t>(b) * p.table_stride + (row >> p.page_shift)];
  if (pg < 0 || pg >= p.n_pages) return -1;
  return pg * p.sb + g * p.sh + static_cast<int64_t>(row & ((1 << p.page_shift) - 1)) * p.st;
}
__device__ inline void flag(const DecodeParams& p, uint32_t bits) {
  if (p.status != nullptr) atomicOr(p.status, bits);
}

// Row of q and out ([B, t_q, H_q, D], token-major) of pair v of KV head g.
__device__ inline int64_t pair_row(const DecodeParams& p, int b, int g, int v) {
  const int i = v / p.group;
  return (static_cast<int64_t>(b) * p.t_q + i) * p.n_q + g * p.group + (v - i * p.group);
}
// Slots pair v may attend are [0, limit): seq_lens[b] + i + 1 for a block
// query i, and n for every head in decode.
__device__ inline int pair_limit(const DecodeParams& p, int n, int v) {
  return p.block ? n - p.t_q + v / p.group + 1 : n;
}

// exp2 of a non-positive-or-bounded argument; -inf gives 0 (hardware v_exp_f32)
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Merge two online-softmax states (log2 domain, reference r, sum l,
// unnormalised accumulators a); an empty state has r = -inf and l = a = 0.
__device__ inline void merge_state(float& r, float& l, float* a, float r2, float l2, const float* a2, int n) {
  const float mn = fmaxf(r, r2);
  const float c1 = (r == -INFINITY) ? 0.f : fast_exp2(r - mn);
  const float c2 = (r2 == -INFINITY) ? 0.f : fast_exp2(r2 - mn);
  l = l * c1 + l2 * c2;
  for (int e = 0; e < n; ++e) a[e] = a[e] * c1 + a2[e] * c2;
  r = mn;
}

// Buffer resource (V#) over [base, base + bytes): loads past the end return
// zero and stores past it are dropped (hardware range check). Word 3 is the
// gfx9-family raw-buffer configuration (32-bit data format, no swizzle).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
// Values every lane of the wave holds alike, moved to scalar registers so
// buffer resources built from them need no per-lane handling.
// (The builtin returns a signed int: each half is taken back to uint32_t
// before widening, or a low word with bit 31 set would sign-extend into the
// high word and corrupt the address.)
__device__ inline uint32_t uniform_u32(uint32_t x) { return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(x)); }
__device__ inline const char* uniform_ptr(const char* q) {
  const uint64_t a = reinterpret_cast<uint64_t>(q);
  const uint64_t lo = uniform_u32(static_cast<uint32_t>(a));
  const uint64_t hi = uniform_u32(static_cast<uint32_t>(a >> 32));
  return reinterpret_cast<const char*>(lo | (hi << 32));
}
// Cache policy of the split exchange (partials, ready flags): device scope
// (16: write-through, miss in the per-XCD L2) unless set otherwise in
// kvc_internal.h.
constexpr int kXchg = KVC_XCHG_POLICY;
// Scope of the epoch's read at entry: the exchange's own (an item's
// workgroups share one XCD's L2 with the default placement and exchange)
constexpr int kEpochScope = KVC_XCHG_POLICY == 0 ? __HIP_MEMORY_SCOPE_WORKGROUP : __HIP_MEMORY_SCOPE_AGENT;
// Cache policy of the K/V stream: every row is read once per launch, so the
// loads carry the non-temporal hint (`nt`). Measured on MI355X (same box,
// interleaved runs) it streams 6-7 % faster than the default policy on every
// decode workload.
constexpr int kStream = 2;

__device__ inline u32x4 buf_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, kStream));
}
__device__ inline u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(off), 0, kStream));
}
__device__ inline u32x4 buf_load_xchg(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, kXchg));
}
__device__ inline void buf_store_xchg(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, x), r,
                                         static_cast<int>(off), 0, kXchg);
}

// 8-bit cache codes (KQ = 1: OCP E4M3, KQ = 2: int8). Every code's value has
// at most 8 significant bits, so widening it to fp16, bf16 or fp32 is exact;
// the scales are applied to scores and weights, not here.
constexpr int kQuantFp8 = 1;
constexpr int kQuantInt8 = 2;

// Codes in bytes 2*HI, 2*HI+1 of w, as two fp32 values.
template <int KQ, bool HI>
__device__ inline void code_pair_f32(uint32_t w, float& a, float& b) {
  if constexpr (KQ == kQuantFp8) {
    const auto f = __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
    a = f[0];
    b = f[1];
  } else {
    a = static_cast<float>(static_cast<int32_t>(w << (HI ? 8 : 24)) >> 24);
    b = static_cast<float>(static_cast<int32_t>(w << (HI ? 0 : 16)) >> 24);
  }
}

// The same two codes as two packed values of the query's 16-bit type.
template <int KQ, typename ET, bool HI>
__device__ inline uint32_t code_pair_16(uint32_t w) {
  if constexpr (KQ == kQuantFp8 && ET::kIsF16) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
  } else {
    float a, b;
    code_pair_f32<KQ, HI>(w, a, b);
    if constexpr (ET::kIsF16) {
      return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
    } else {   // bf16: the high half of an fp32 value with at most 8 significant bits
      return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
    }
  }
}

// Eight codes (two dwords) as the 8-element MFMA operand of the query's type.
template <int KQ, typename ET>
__device__ inline u32x4 codes8_16(uint32_t w0, uint32_t w1) {
  return u32x4{code_pair_16<KQ, ET, false>(w0), code_pair_16<KQ, ET, true>(w0), code_pair_16<KQ, ET, false>(w1),
               code_pair_16<KQ, ET, true>(w1)};
}

// Eight codes as fp32 values, in order.
template <int KQ>
__device__ inline void codes8_f32(const u32x2 r, float* f) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    code_pair_f32<KQ, false>(r[i], f[4 * i], f[4 * i + 1]);
    code_pair_f32<KQ, true>(r[i], f[4 * i + 2], f[4 * i + 3]);
  }
}

// fp32 -> OCP E4M3 byte: round to nearest even, saturate at +-448, NaN -> 0x7F.
__device__ inline uint32_t e4m3_from_f32(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t au = u & 0x7fffffffu;
  if (au > 0x7f800000u) return 0x7Fu;                  // NaN
  const float a = __uint_as_float(au);
  if (a >= 448.f) return sign | 0x7Eu;
  if (a < 0.015625f) {                                 // below 2^-6: multiples of 2^-9
    // a * 512 is exact; rint rounds ties to even; 8 is the code of 2^-6
    return sign | static_cast<uint32_t>(__builtin_rintf(a * 512.f));
  }
  uint32_t e = (au >> 23) - 120u;                      // biased E4M3 exponent (bias 7), 1..15
  const uint32_t mant = au & 0x7fffffu;
  uint32_t m = (mant + 0x7ffffu + ((mant >> 20) & 1u)) >> 20;   // 3 bits, ties to even; 8 carries
  if (m == 8u) {
    e += 1u;
    m = 0u;
  }
  const uint32_t code = (e << 3) | m;
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

template <typename IT>
__device__ inline float load_elem(const char* row, int i) {
  if constexpr (IT::kBytes == 4) return reinterpret_cast<const float*>(row)[i];
  else if constexpr (IT::kIsF16) return static_cast<float>(reinterpret_cast<const _Float16*>(row)[i]);
  else return __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(row)[i]) << 16);
}

// Quantise one row of D values held by a wave (lane l: elements
// [l*E, l*E + E), E = D/64) as the format defines: amax by a wave-wide
// maximum, scale = amax / QMAX and each code from x / scale, both fp32
// divisions (correctly rounded). Returns the scale (0 for a row of zeros) and
// the lane's E code bytes packed little-endian. Every lane of the wave must
// take part.
template <typename IT, int KQ, int D>
__device__ inline float quant_row(const char* src, int lane, uint32_t& packed) {
  constexpr int E = D / 64;
  constexpr float kQmax = KQ == kQuantFp8 ? 448.f : 127.f;
  float x[E];
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    x[e] = load_elem<IT>(src, lane * E + e);
    amax = fmaxf(amax, fabsf(x[e]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float scale = amax / kQmax;
  packed = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    uint32_t c = 0u;
    if (amax > 0.f) {
      const float y = x[e] / scale;
      if constexpr (KQ == kQuantFp8) {
        c = e4m3_from_f32(y);
      } else {
        c = static_cast<uint32_t>(static_cast<int32_t>(fminf(fmaxf(__builtin_rintf(y), -127.f), 127.f))) & 0xffu;
      }
    }
    packed |= c << (8 * e);
  }
  return amax > 0.f ? scale : 0.f;
}

// E code bytes of one lane, little-endian, to dst.
template <int E>
__device__ inline void store_codes(char* dst, uint32_t packed) {
  if constexpr (E == 1) *reinterpret_cast<uint8_t*>(dst) = static_cast<uint8_t>(packed);
  else if constexpr (E == 2) *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(packed);
  else *reinterpret_cast<uint32_t*>(dst) = packed;
}

// Tuning constants (measured on MI355X): waves per decode workgroup, row
// passes per register tile, and tiles of loads kept in flight ahead of the
// one being computed.
#ifndef KVC_WAVES
#define KVC_WAVES 4
#endif
#ifndef KVC_TILE_PASSES
#define KVC_TILE_PASSES 2
#endif
#ifndef KVC_PREFETCH
#define KVC_PREFETCH 2
#endif
#ifndef KVC_OCCUPANCY
#define KVC_OCCUPANCY 4
#endif
#ifndef KVC_MFMA_PREFETCH   // matrix-core path: one tile ahead measured 2-4 % faster than two
#define KVC_MFMA_PREFETCH 1
#endif
#ifndef KVC_MFMA_OCCUPANCY
#define KVC_MFMA_OCCUPANCY 2
#endif

// 16-bit caches whose rows are whole 32-element slices take the matrix-core
// path (scores on 16x16x32 MFMA, and P.V on 4x4x1 MFMA for 4+ heads).
template <typename ET, int D>
constexpr bool decode_uses_mfma() { return ET::kBytes == 2 && D % 32 == 0; }

// Workgroups each CU should hold at once, which sets the VGPR budget
// (512 / workgroups per SIMD).
template <typename ET, int D, int GB, int KQ = 0>
constexpr int decode_min_wgs() {
  if constexpr (KQ != 0 || decode_uses_mfma<ET, D>()) return (GB > 4 || D > 128) ? 1 : KVC_MFMA_OCCUPANCY;
  return (ET::kBytes == 2 && GB <= 4) ? KVC_OCCUPANCY : 1;
}

// ET: the type of q and out (and of the cache, KQ = 0); KQ != 0: a cache of
// 8-bit codes with per-token scales (see the format helpers above).
template <typename ET, int D, int GB, int KQ = 0>
__global__ __launch_bounds__(KVC_WAVES * 64, (decode_min_wgs<ET, D, GB, KQ>())) void decode_kernel(
    const DecodeParams p) {
  constexpr bool kQuant = KQ != 0;
  // One field from each 64-byte line of the parameters, read here: all the
  // lines are requested in the first round trip, and later reads of the
  // parameters hit the scalar cache instead of waiting in turn. Measured on
  // MI355X with many workgroups per CU (ragged_long) a few per cent faster.
  asm volatile("" ::"s"(p.k), "s"(p.v_new), "s"(p.batch), "s"(p.scale_log2));
  // Cache elements per lane of a row in the V layout: one 16-byte slice, or
  // 8 bytes of 8-bit codes (so the fp32 accumulators per lane stay 8 per head).
  constexpr int EPL = kQuant ? 8 : ET::kPerVec;
  constexpr int VSL = kQuant ? 8 : 16;     // bytes per lane slice of a row
  constexpr int LPR = D / EPL;            // lanes per row
  constexpr int RPP = 64 / LPR;           // rows per wave pass
  constexpr int NW = KVC_WAVES;           // waves per workgroup
  constexpr int U = (RPP >= 4) ? KVC_TILE_PASSES : 4;   // passes per tile
  constexpr int TS = NW * RPP * U;        // rows per workgroup tile
  constexpr int D4 = D / 4;               // float4 columns of an output row
  constexpr float kLazy = 8.f;            // reference moves only past ref + 8 (log2 domain)
  // Reference of a state that has seen no row: finite, so exp2(score - ref)
  // of a masked (-inf) score is exp2(-inf) = 0 rather than NaN, and far
  // below any finite score, so exp2(kEmpty - ref) is 0 once a row is seen.
  constexpr float kEmpty = -1e30f;
  static_assert(LPR >= 1 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "row must split into 16-byte lane slices");

  constexpr bool kMfma = kQuant || decode_uses_mfma<ET, D>();
  static_assert(!kQuant || (ET::kBytes == 2 && D % 64 == 0), "8-bit caches: 16-bit queries, D a multiple of 64");
  constexpr int NQ = (GB + 3) / 4;         // quads of query heads (matrix-core path)

  // Matrix-core path with up to 4 heads: one softmax reference per wave, so
  // the wave's lane groups are summed through LDS (32 KB at most) instead of
  // merged with cross-lane shuffles.
  constexpr bool kLdsMerge = kMfma && GB <= 4;
  __shared__ float sm_a[kLdsMerge ? 1 : NW][GB][D];
  __shared__ float sm_acc[kLdsMerge ? NW : 1][kLdsMerge ? RPP : 1][GB][kLdsMerge ? D : 1];
  __shared__ float sm_ml[NW][GB][2];
  __shared__ float sm_p[kMfma ? NW : 1][16][4 * NQ];   // softmax weights, score layout -> V layout
  // 8-bit caches, fused append: the new row's K and V codes, staged so that
  // they can be read in the score layout (K) and the row layout (V)
  __shared__ __align__(16) uint8_t sm_x[kQuant ? 2 : 1][kQuant ? D : 16];

  // Workgroup ids go round-robin over the 8 XCDs (id mod 8). Every
  // workgroup of a (sequence, KV head) unit takes an id with the same residue
  // mod 8, so the unit's splits and head blocks run on one XCD: the head
  // blocks read the same K/V rows through one L2, and the splits exchange
  // their partials through it. On its XCD a unit's workgroups take
  // consecutive slots, head blocks innermost, then splits, so the merging
  // split (the last) has the highest id of its item. The grid is padded to a
  // multiple of 8 units.
  const int xcd = blockIdx.x & 7;
  const int r8 = blockIdx.x >> 3;
  const int hb = r8 % p.n_hblk;
#if KVC_XCD_COLOCATE
  const int rest = r8 / p.n_hblk;
  const int split = rest % p.n_splits;
  const int unit = (rest / p.n_splits) * 8 + xcd;
  if (unit >= p.batch * p.n_kv) return;             // grid padding
#else
  const int w_item = (r8 / p.n_hblk) * 8 + xcd;
  if (w_item >= p.batch * p.n_kv * p.n_splits) return;   // grid padding
  const int split = w_item % p.n_splits;
  const int unit = w_item / p.n_splits;
#endif
  const int b = unit / p.n_kv;
  const int g = unit - b * p.n_kv;
  // The sequence's length, then the item's epoch (word S - 1 of its flags:
  // no split publishes there), requested in that order so that the wait
  // for the length does not also wait for the epoch, which is used only
  // after the stream. A publisher raises its flag to epoch + 1; the merger
  // waits for exactly that value and then advances the epoch, so flags
  // never need clearing and a flag raised after a merge gave up waiting
  // (KVC_DEVERR_SYNC) cannot be taken for the next call's. With the item's
  // workgroups on one XCD the epoch is read from that XCD's L2, where the
  // previous call's merger (on the same XCD) left it.
  const int c0 = p.seq_lens[b];
  asm volatile("" ::: "memory");
  const int64_t item = static_cast<int64_t>(unit) * p.n_hblk + hb;
  uint32_t* const flags = p.ws_flag + item * p.flag_stride;
  uint32_t epoch = 0u;
  if (p.n_splits > 1) epoch = __hip_atomic_load(flags + p.flag_stride - 1, __ATOMIC_RELAXED, kEpochScope);

  const SeqInfo si = seq_info(p, c0);
  // kvc_decode_step_advance (the last layer of a step): the next step's
  // lengths, written by one workgroup per sequence into another array, so no
  // workgroup of this launch reads a changed length
  if (p.lens_next != nullptr && g == 0 && split == 0 && hb == 0 && threadIdx.x == 0)
    p.lens_next[b] = c0 + 1;
  if (si.flags != 0 && g == 0 && hb == 0 && split == 0 && threadIdx.x == 0 && p.status != nullptr)
    atomicOr(p.status, si.flags);
  const int n = si.n;
  const int gv = p.group * p.t_q;                  // (query, head) pairs of this KV head
  const int v_first = hb * GB;                     // first pair of this block
  const int nh = min(GB, gv - v_first);            // valid pairs in this block
  if (n <= 0) {                                      // empty sequence: zero rows
    if (split == 0)
      for (int t = threadIdx.x; t < nh * D; t += blockDim.x)
        store_out<ET>(p, pair_row(p, b, g, v_first + t / D) * D + t % D, 0.f);
    return;
  }
  // The newest attended row is folded in apart from the stream (below), so
  // the chunks share out the other n - 1 rows: equal whole 16-row tiles (a
  // tile never straddles two pages), the last active split also holding row
  // n - 1. ns splits are active.
  const int chunk = max(16, ((n - 1 + p.n_splits - 1) / p.n_splits + 15) & ~15);
  const int ns = n > 1 ? min(p.n_splits, (n - 1 + chunk - 1) / chunk) : 1;
  if (split >= ns) return;                           // inactive split: not counted in ns
  const int t0 = split * chunk;
  const int t1 = split == ns - 1 ? n : t0 + chunk;

  const int lane = threadIdx.x & 63;
  // wave index as a scalar: loop bounds derived from it are wave-uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane / LPR;             // which row of the pass
  const int li = lane % LPR;              // which 16-byte slice of the row

  float ref[GB], l[GB], acc[GB][EPL];
#pragma unroll
  for (int j = 0; j < GB; ++j) {
    ref[j] = kEmpty;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[j][e] = 0.f;
  }

  const int64_t unit_off = b * p.sb + g * p.sh;
  // The last attended row (n - 1) is folded in after the streaming loop, as
  // one extra tile held in registers, by the workgroup whose chunk holds it;
  // that workgroup streams only [t0, n - 1) from the cache. With the fused
  // append that row is the new token: it comes from k_new/v_new and the
  // workgroup of the first head block writes it into the cache, so nothing
  // waits on the copy and no workgroup reads slot T_b from the cache in this
  // launch. Both entry points thus add the same rows in the same order, and
  // kvc_decode_step matches kvc_append + kvc_decode_attn bit for bit.
  const int arow = si.append_row;
  const int xrow = si.newest;
  const bool has_x = xrow >= t0 && xrow < t1;
  const bool x_new = has_x && arow == xrow;
  // Rows streamed from the cache: [t0, t_end) (a scalar, like every loop
  // bound below). A wrapped ring's newest slot can sit inside the chunk: then
  // the chunk is streamed as two segments, [t0, newest) and (newest, t1), so
  // that no tile ever needs a mask for that slot.
  int t_end = __builtin_amdgcn_readfirstlane(has_x ? xrow : t1);
  const int n_seg = (p.ring != 0 && has_x && xrow != t1 - 1) ? 2 : 1;
  const int seg1_lo = __builtin_amdgcn_readfirstlane(xrow + 1);
  u32x4 nk = u32x4{0u, 0u, 0u, 0u}, nv = u32x4{0u, 0u, 0u, 0u};
  // The row's K in the matrix-core layout (lanes l with l % 16 == 0 hold
  // 16-byte slice 4m + l / 16 for MFMA m), requested here with the rest of
  // the row so that no load waits after the streaming loop.
  constexpr int NXK = kMfma ? (kQuant ? D / 64 : D / 32) : 1;
  u32x4 xk[NXK];
#pragma unroll
  for (int m = 0; m < NXK; ++m) xk[m] = u32x4{0u, 0u, 0u, 0u};
  float xks = 0.f, xvs = 0.f;                   // scales of the folded row (8-bit caches)
  // The row's loads (and, for a new row on an 8-bit cache, its
  // quantisation), issued by each path after its first tiles' loads.
  auto load_x_row = [&]() {
    if (has_x && wave == 0) {
      const char* krow;
      const char* vrow;
      if (x_new) {
        const int64_t noff = b * p.nsb + g * p.nsh;
        krow = p.k_new + noff;
        vrow = p.v_new + noff;
      } else {
        const int64_t xo = slot_offset(p, b, g, xrow);
        krow = xo < 0 ? nullptr : p.k + xo;
        vrow = xo < 0 ? nullptr : p.v + xo;
        if (xo < 0 && lane == 0) flag(p, KVC_DEVERR_PAGE);
      }
      if (krow != nullptr) {
        if constexpr (kQuant) {                  // 8 code bytes of V (K is loaded in the MFMA layout)
          if (!x_new) {                          // (a new row is quantised below)
            const u32x2 w = *reinterpret_cast<const u32x2*>(vrow + li * VSL);
            nv = u32x4{w[0], w[1], 0u, 0u};
          }
        } else {
          nk = *reinterpret_cast<const u32x4*>(krow + li * VSL);
          nv = *reinterpret_cast<const u32x4*>(vrow + li * VSL);
        }
        if constexpr (kMfma) {
          if ((!kQuant || !x_new) && (lane & 15) == 0) {   // (a new 8-bit row's codes come through LDS)
#pragma unroll
            for (int m = 0; m < NXK; ++m) xk[m] = *reinterpret_cast<const u32x4*>(krow + (4 * m + (lane >> 4)) * 16);
          }
        }
      }
    }
    if constexpr (kQuant) {
      if (has_x && wave == 0) {
        if (x_new) {
          // The step's new row, quantised as kvc_quant_append does (the same
          // device function), so the fused step matches append + decode bit
          // for bit; its codes go through LDS to the K and V layouts.
          const int64_t noff = b * p.nsb + g * p.nsh;
          uint32_t xkc, xvc;                     // this lane's code bytes of the new row
          xks = quant_row<ET, KQ, D>(p.k_new + noff, lane, xkc);
          xvs = quant_row<ET, KQ, D>(p.v_new + noff, lane, xvc);
          store_codes<D / 64>(reinterpret_cast<char*>(&sm_x[0][lane * (D / 64)]), xkc);
          store_codes<D / 64>(reinterpret_cast<char*>(&sm_x[1][lane * (D / 64)]), xvc);
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          __builtin_amdgcn_wave_barrier();
          const u32x2 w = *reinterpret_cast<const u32x2*>(&sm_x[1][li * VSL]);
          nv = u32x4{w[0], w[1], 0u, 0u};
          // the first head block also writes the row into the cache: no
          // workgroup of this launch reads that slot from memory
          if (hb == 0) {
            const int64_t ao = slot_offset(p, b, g, arow);
            store_codes<D / 64>(p.k + ao + lane * (D / 64), xkc);
            store_codes<D / 64>(p.v + ao + lane * (D / 64), xvc);
            if (lane == 0) {
              const int64_t so = b * p.ssb + g * p.ssh + static_cast<int64_t>(arow) * 4;
              *reinterpret_cast<float*>(p.k_scale + so) = xks;
              *reinterpret_cast<float*>(p.v_scale + so) = xvs;
            }
          }
        } else {
          const int64_t so = b * p.ssb + g * p.ssh + static_cast<int64_t>(xrow) * 4;
          xks = *reinterpret_cast<const float*>(p.k_scale + so);
          xvs = *reinterpret_cast<const float*>(p.v_scale + so);
        }
      }
    }
  };

  // K/V of this unit through buffer resources built per tile on the scalar
  // unit: base = the tile's first row, range = up to row t_end, so rows of a
  // tile past t_end read as zero (and are masked), every load is
  // unconditional, nothing past the streamed range can be read, and the lanes'
  // offsets are loop constants (no vector address arithmetic in the loop).
  const uint32_t st = static_cast<uint32_t>(p.st);
  const char* kunit = p.k + unit_off;
  const char* vunit = p.v + unit_off;
  const float sc = p.scale_log2;

  if constexpr (kMfma) {
    //------------------------------------------------------------------------
    // Matrix-core path. A wave takes 16 consecutive rows per tile. Scores
    // S[h][r] = q_h . K_r come from NM MFMAs 16x16x32 with q as A (row = head,
    // lanes l%16) and K as B (column = row r = l%16): lane l loads 16 bytes,
    // slice 4m + l/16, of row l%16 for the m-th MFMA, and q is loaded with the
    // same slice order, so the sum runs over all D elements. Lane l then holds
    // S[4(l/16) + t][l%16] in register t: the scores of row l%16 for heads
    // 4(l/16)..+3. Padded heads (no query) and masked rows start from -inf in
    // the accumulator, so their weights are exactly 0.
    // The running reference is one value per head for the whole wave. The
    // weights go through LDS to the row layout of V (LPR lanes per row, 16
    // bytes each), where P.V runs on 4x4x1 MFMAs for 4+ heads (block b =
    // lanes 4b..4b+3, all of one row: A = the weight of head 4q + l%4, B = V
    // element e of lane l, C = the head quad's outputs for that column) or on
    // the vector ALU for 1-2 heads.
    // 8-bit caches: a lane's 16-byte load of a K row holds 16 codes, which
    // feed two MFMAs after widening to q's type (load i, lane group kq:
    // elements 64i + 16kq .. +16; the first 8 go to MFMA 2i, the rest to
    // MFMA 2i+1, and q is loaded in that order). The scores are scaled by the
    // row's K scale before the masks, and each weight is multiplied by its
    // row's V scale on its way to LDS (the row sums use the unscaled weights).
    constexpr int NM = D / 32;                // score MFMAs per tile
    constexpr int NKL = kQuant ? NM / 2 : NM;  // 16-byte K loads per lane per tile
    using VT = std::conditional_t<kQuant, u32x2, u32x4>;   // a lane's slice of a V row
    constexpr int NP = 16 / RPP;              // V row passes per tile
    constexpr int TSM = NW * 16;              // rows per workgroup tile
    constexpr int NBM = KVC_MFMA_PREFETCH + 1;
    const int r16 = lane & 15;                // score row of this lane
    const int kq = lane >> 4;                 // its slice group, and its head quad in the scores

    uint32_t koff[NKL], voffm[NP];
#pragma unroll
    for (int m = 0; m < NKL; ++m) koff[m] = static_cast<uint32_t>(r16) * st + static_cast<uint32_t>(4 * m + kq) * 16u;
#pragma unroll
    for (int u = 0; u < NP; ++u)
      voffm[u] = static_cast<uint32_t>(u * RPP + grp) * st + static_cast<uint32_t>(li * VSL);

    // Paged caches: a wave's tiles start at slots wbase0 + k * TSM. Lane j
    // of `pidv` holds the page of tile (k & ~63) + j, loaded 64 tiles at a
    // time with one vector load, and a tile's page is taken with readlane, so
    // no page-table read waits in front of the tile loads.
    const bool paged = p.table != nullptr;
    const int wbase0 = t0 + wave * 16;
    int pidv = -1, pid_block = -1;
    auto tile_page = [&](int base) {
      const int k = (base - wbase0) / TSM;    // wave-uniform tile index
      if ((k >> 6) != pid_block) {
        pid_block = k >> 6;
        const int row = wbase0 + ((pid_block << 6) + lane) * TSM;
        pidv = -1;
        if (row < t_end) pidv = p.table[static_cast<int64_t>(b) * p.table_stride + (row >> p.page_shift)];
      }
      return __builtin_amdgcn_readlane(pidv, k & 63);
    };
    // the scales of this unit's rows (8-bit caches), 4 bytes per token
    const int64_t sunit = b * p.ssb + g * p.ssh;
    auto load_tile = [&](int base_any, u32x4 (&K)[NKL], VT (&V)[NP], float& KS, float& VS) {
      const int base = __builtin_amdgcn_readfirstlane(base_any);
      const int rows_left = t_end - base;
      uint32_t range = rows_left > 0 ? static_cast<uint32_t>(rows_left) * st : 0u;
      int64_t boff = unit_off + static_cast<int64_t>(base) * st;
      if (paged) {                            // the tile's 16 rows lie in one page
        boff = 0;
        if (rows_left > 0) {
          const int pg = tile_page(base);
          range = static_cast<uint32_t>(min(rows_left, 16)) * st;
          if (pg < 0 || pg >= p.n_pages) {    // not in the pool: read zeros, report
            range = 0u;
            if (lane == 0) flag(p, KVC_DEVERR_PAGE);
          } else {
            boff = pg * p.sb + g * p.sh + static_cast<int64_t>(base & ((1 << p.page_shift) - 1)) * st;
          }
        }
      }
      const __amdgpu_buffer_rsrc_t krs = make_rsrc(uniform_ptr(p.k + boff), range);
      const __amdgpu_buffer_rsrc_t vrs = make_rsrc(uniform_ptr(p.v + boff), range);
#pragma unroll
      for (int m = 0; m < NKL; ++m) K[m] = buf_load(krs, koff[m]);
#pragma unroll
      for (int u = 0; u < NP; ++u) {
        if constexpr (kQuant) V[u] = buf_load8(vrs, voffm[u]);
        else V[u] = buf_load(vrs, voffm[u]);
      }
      if constexpr (kQuant) {                 // row r16's scales; rows past t_end read as 0
        const uint32_t srange = rows_left > 0 ? static_cast<uint32_t>(rows_left) * 4u : 0u;
        const int64_t soff = sunit + static_cast<int64_t>(base) * 4;
        const __amdgpu_buffer_rsrc_t ksr = make_rsrc(uniform_ptr(p.k_scale + soff), srange);
        const __amdgpu_buffer_rsrc_t vsr = make_rsrc(uniform_ptr(p.v_scale + soff), srange);
        KS = __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(ksr, r16 * 4, 0, kStream)));
        VS = __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(vsr, r16 * 4, 0, kStream)));
      }
    };

    // The first tiles' loads leave first: they need only the split's rows,
    // and the query and newest-row loads and the per-pair setup below then
    // run while those loads are in flight instead of ahead of them.
    u32x4 KB[NBM][NKL];
    VT VB[NBM][NP];
    float KSB[NBM], VSB[NBM];
    const int base0 = __builtin_amdgcn_readfirstlane(t0 + wave * 16);
    const int n_tiles0 = base0 < t_end ? (t_end - base0 + TSM - 1) / TSM : 0;
    if constexpr (kQuant) load_x_row();       // (a new 8-bit row is quantised: its wait stays ahead of the tiles)
    if (n_tiles0 > 0) {
#pragma unroll
      for (int r = 0; r < NBM - 1; ++r) load_tile(base0 + r * TSM, KB[r], VB[r], KSB[r], VSB[r]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!kQuant) load_x_row();

    u32x4 qa[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      qa[m] = u32x4{0u, 0u, 0u, 0u};
      const int qe = kQuant ? 64 * (m >> 1) + 16 * kq + 8 * (m & 1) : (4 * m + kq) * EPL;   // first element
      if (r16 < nh)
        qa[m] = *reinterpret_cast<const u32x4*>(p.q + (pair_row(p, b, g, v_first + r16) * D + qe) * ET::kBytes);
    }
    float hbias[4];                           // 0 where (lane, register) is a real head's score
#pragma unroll
    for (int t = 0; t < 4; ++t) hbias[t] = (kq < NQ && 4 * kq + t < nh) ? 0.f : -INFINITY;
    int plim[4];                              // slot limit of the pair in (lane, register t)
#pragma unroll
    for (int t = 0; t < 4; ++t) plim[t] = pair_limit(p, n, v_first + 4 * kq + t);
    const bool block = p.block != 0;
    float refh[4 * NQ];                       // wave-uniform reference per head
#pragma unroll
    for (int h = 0; h < 4 * NQ; ++h) refh[h] = kEmpty;
    float lsum[4] = {0.f, 0.f, 0.f, 0.f};    // per-lane sums, score layout
    f32x4 accq[GB >= 4 ? NQ : 1][EPL];       // 4x4x1 outputs: register i = head 4q + i
#pragma unroll
    for (int q = 0; q < (GB >= 4 ? NQ : 1); ++q)
#pragma unroll
      for (int e = 0; e < EPL; ++e) accq[q][e] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto lane_ref = [&](int t) { return (NQ > 1 && kq == 1) ? refh[4 + t] : refh[t]; };

    const f32x4 hb4 = f32x4{hbias[0], hbias[1], hbias[2], hbias[3]};
    // rows_left: rows of this tile to attend (all 16 unless it is the last);
    // row0: the tile's first slot, for the per-pair limits of a query block
    // KS, VS: this lane's row's K and V scales (8-bit caches)
    auto compute = [&](const u32x4 (&K)[NKL], const VT (&V)[NP], float KS, float VS, int rows_left, int row0) {
      f32x4 sv;
      if constexpr (kQuant) {
        sv = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < NM; ++m)
          sv = ET::mfma16(qa[m], codes8_16<KQ, ET>(K[m >> 1][2 * (m & 1)], K[m >> 1][2 * (m & 1) + 1]), sv);
        const float f = KS * sc;              // K scale and softmax scale (log2 domain)
#pragma unroll
        for (int t = 0; t < 4; ++t) sv[t] = fmaf(sv[t], f, hbias[t]);
      } else {
        sv = ET::mfma16(qa[0], K[0], hb4);
#pragma unroll
        for (int m = 1; m < NM; ++m) sv = ET::mfma16(qa[m], K[m], sv);
      }
      if (rows_left < 16) {                   // wave-uniform: only a last, partial tile
#pragma unroll
        for (int t = 0; t < 4; ++t) sv[t] = r16 < rows_left ? sv[t] : -INFINITY;
      }
      if (block) {                            // lower-right causal mask of a query block
#pragma unroll
        for (int t = 0; t < 4; ++t) sv[t] = row0 + r16 < plim[t] ? sv[t] : -INFINITY;
      }
      float w[4], rl[4];
      bool need = false;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        w[t] = kQuant ? sv[t] : sv[t] * sc;   // log2-domain score
        rl[t] = lane_ref(t);
        need = need || (w[t] > rl[t] + kLazy);
      }
      if (__any(need)) {                      // wave-uniform, rarely taken after the first tile
        float mx[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) mx[t] = row16_max(w[t]);
#pragma unroll
        for (int h = 0; h < 4 * NQ; ++h) {
          const float mh = lane_value(mx[h & 3], 16 * (h >> 2));
          const float nr = mh > refh[h] + kLazy ? mh : refh[h];
          const float c = fast_exp2(refh[h] - nr);   // 0 while the reference is still empty
          refh[h] = nr;
          if (kq == (h >> 2)) lsum[h & 3] *= c;
          if constexpr (GB >= 4) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) accq[h >> 2][e][h & 3] *= c;
          } else if (h < GB) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] *= c;
          }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) rl[t] = lane_ref(t);
      }
      f32x4 pw;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        pw[t] = fast_exp2(w[t] - rl[t]);
        lsum[t] += pw[t];
      }
      if constexpr (kQuant) pw *= VS;         // V scale of this lane's row
      if (kq < NQ) *reinterpret_cast<f32x4*>(&sm_p[wave][r16][4 * kq]) = pw;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int u = 0; u < NP; ++u) {
        const int r = u * RPP + grp;          // row of this lane in pass u
        float vf[EPL];
        if constexpr (kQuant) codes8_f32<KQ>(V[u], vf);
        else ET::unpack(V[u], vf);
        if constexpr (GB >= 4) {
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            const float a = sm_p[wave][r][4 * q + (lane & 3)];
#pragma unroll
            for (int e = 0; e < EPL; ++e) accq[q][e] = __builtin_amdgcn_mfma_f32_4x4x1f32(a, vf[e], accq[q][e], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int j = 0; j < GB; ++j) {
            const float a = sm_p[wave][r][j];
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[j][e] = fmaf(a, vf[e], acc[j][e]);
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
    };

    // The last attended row, as row 0 of one more tile. Wave 0 folds it in
    // right after its first streamed tile, while its next tiles are still in
    // flight, rather than after the loop, where the wave would run it alone.
    bool x_done = false;
    auto fold_x = [&]() {
      // The row's registers are made opaque here: otherwise the compiler
      // hoists their selects and conversions ahead of the streaming loop,
      // and its wait for the row's loads there holds back the first tiles'.
      asm volatile("" : "+v"(nv));
#pragma unroll
      for (int m = 0; m < NXK; ++m) asm volatile("" : "+v"(xk[m]));
      u32x4 K[NKL];
      VT V[NP];
      static_assert(NKL == NXK, "x-row K slices");
#pragma unroll
      for (int m = 0; m < NKL; ++m) {
        K[m] = xk[m];
        if (kQuant && x_new) K[m] = r16 == 0 ? *reinterpret_cast<const u32x4*>(&sm_x[0][(4 * m + kq) * 16])
                                             : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < NP; ++u) {
        if constexpr (kQuant) V[u] = (u == 0 && grp == 0) ? u32x2{nv[0], nv[1]} : u32x2{0u, 0u};
        else V[u] = (u == 0 && grp == 0) ? nv : u32x4{0u, 0u, 0u, 0u};
      }
      compute(K, V, r16 == 0 ? xks : 0.f, r16 == 0 ? xvs : 0.f, 1, xrow);
      x_done = true;
    };

    // (a second segment occurs on contiguous ring caches only, so the page
    // lookup, which counts tiles from t0, never sees one)
    for (int seg = 0; seg < n_seg; ++seg) {
      if (seg == 1) t_end = t1;
      int base = seg == 0 ? base0 : __builtin_amdgcn_readfirstlane(seg1_lo + wave * 16);
      const int n_tiles = seg == 0 ? n_tiles0 : (base < t_end ? (t_end - base + TSM - 1) / TSM : 0);
      if (n_tiles > 0) {
        if (seg == 1) {                       // (seg 0's first tiles were requested above)
#pragma unroll
          for (int r = 0; r < NBM - 1; ++r) load_tile(base + r * TSM, KB[r], VB[r], KSB[r], VSB[r]);
        }
        bool done = false;
        for (int it = 0; !done; it += NBM) {
#pragma unroll
          for (int r = 0; r < NBM; ++r) {     // unrolled: ring slots are compile-time
            const int nr = (r + NBM - 1) % NBM;
            load_tile(base + (NBM - 1) * TSM, KB[nr], VB[nr], KSB[nr], VSB[nr]);
            // the next tile's loads leave before any wait on this tile's
            __builtin_amdgcn_sched_barrier(0);
            compute(KB[r], VB[r], KSB[r], VSB[r], __builtin_amdgcn_readfirstlane(t_end - base), base);
            if (!x_done && has_x && wave == 0) fold_x();
            base += TSM;
            if (it + r + 1 >= n_tiles) {
              done = true;
              break;
            }
          }
        }
      }
    }
    if (!x_done && has_x && wave == 0) fold_x();   // (wave 0 streamed no tile)
    // Wave totals in the common layout: one reference per head (the same in
    // every lane), the weight sum in lane group 0 only (the lane-group merge
    // below adds the groups), accumulators as acc[head][element].
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float x = lsum[t];
      x += dpp_f<kDppQuadXor1>(x);
      x += dpp_f<kDppQuadXor2>(x);
      x += dpp_f<kDppHalfMirror>(x);
      lsum[t] = x + dpp_f<kDppMirror>(x);
    }
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      ref[j] = refh[j];
      const float lt = lane_value(lsum[j & 3], 16 * (j >> 2));
      l[j] = grp == 0 ? lt : 0.f;
      if constexpr (GB >= 4) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] = accq[j >> 2][e][j & 3];
      }
    }
  } else {
  //--------------------------------------------------------------------------
  // Vector-ALU path (fp32 caches, and rows that are not whole 32-element
  // slices): every lane holds its 16-byte slice of q for each head of the
  // block, and a row's LPR lanes reduce their partial dot products with DPP.
  load_x_row();
  u32x4 qv[GB];
#pragma unroll
  for (int j = 0; j < GB; ++j) {
    if (j < nh) {
      qv[j] = *reinterpret_cast<const u32x4*>(p.q + (pair_row(p, b, g, v_first + j) * D + li * EPL) * ET::kBytes);
    } else {
      qv[j] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  uint32_t voff[U];
#pragma unroll
  for (int u = 0; u < U; ++u)
    voff[u] = static_cast<uint32_t>(u * NW * RPP + grp) * st + static_cast<uint32_t>(li) * 16u;

  auto load_tile = [&](int base_any, u32x4 (&K)[U], u32x4 (&V)[U]) {
    const int base = __builtin_amdgcn_readfirstlane(base_any);
    const int rows_left = t_end - base;
    const uint32_t range = rows_left > 0 ? static_cast<uint32_t>(rows_left) * st : 0u;
    const int64_t boff = static_cast<int64_t>(base) * st;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(uniform_ptr(kunit + boff), range);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(uniform_ptr(vunit + boff), range);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      K[u] = buf_load(krs, voff[u]);
      V[u] = buf_load(vrs, voff[u]);
    }
  };

  // One tile of U rows per lane group. bias[u] is 0 for a row to attend and
  // -inf for a masked one: it seeds the dot product, so a masked row's score
  // is -inf, drops out of the maximum and gets weight exp2(-inf) = 0 with no
  // per-head masking (its K and V read as zero through the range check).
  // The order (all scores, then all weights, then V one row at a time) keeps
  // few temporaries live next to the buffered tiles.
  int vlim[GB];                                // slot limit of each pair (query blocks)
#pragma unroll
  for (int j = 0; j < GB; ++j) vlim[j] = pair_limit(p, n, v_first + j);
  const bool block = p.block != 0;
  // row_at[u]: this lane's slot in pass u (for the per-pair limits of a block)
  auto compute_rows = [&](const u32x4 (&K)[U], const u32x4 (&V)[U], const float (&bias)[U], const int (&row_at)[U]) {
    float w[GB][U];
#pragma unroll
    for (int j = 0; j < GB; ++j)
#pragma unroll
      for (int u = 0; u < U; ++u)
        w[j][u] = ET::dot(qv[j], K[u], (block && row_at[u] >= vlim[j]) ? -INFINITY : bias[u]);
    group_sum_n<LPR>(reinterpret_cast<float (&)[GB * U]>(w));
#pragma unroll
    for (int j = 0; j < GB; ++j) {
#pragma unroll
      for (int u = 0; u < U; ++u) w[j][u] *= sc;   // log2-domain score
      float mt = w[j][0];
#pragma unroll
      for (int u = 1; u < U; ++u) mt = fmaxf(mt, w[j][u]);   // tile maximum (-inf if all masked)
      const bool need = mt > ref[j] + kLazy;
      if (__any(need)) {                      // wave-uniform branch, rarely taken after the first tile
        const float nr = need ? mt : ref[j];
        const float c = fast_exp2(ref[j] - nr);   // 0 while ref is still the empty value
        l[j] *= c;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] *= c;
        ref[j] = nr;
      }
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        w[j][u] = fast_exp2(w[j][u] - ref[j]);   // exactly 1 for the row that set ref
        ps += w[j][u];
      }
      l[j] += ps;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[EPL];
      ET::unpack(V[u], vf);
#pragma unroll
      for (int j = 0; j < GB; ++j)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] = fmaf(w[j][u], vf[e], acc[j][e]);
    }
  };

  // row of pass u relative to the tile's first row, per lane (loop invariant)
  int rel_row[U];
#pragma unroll
  for (int u = 0; u < U; ++u) rel_row[u] = u * NW * RPP + grp;

  auto compute_tile = [&](int base, const u32x4 (&K)[U], const u32x4 (&V)[U]) {
    const int rows_left = __builtin_amdgcn_readfirstlane(t_end - base);   // scalar
    float bias[U];
    int row_at[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      row_at[u] = base + rel_row[u];
      bias[u] = rel_row[u] < rows_left ? 0.f : -INFINITY;
    }
    compute_rows(K, V, bias, row_at);
  };

  // Register ring of NB tiles: NB - 1 tiles of loads in flight behind the
  // one being computed. `base` is this wave's first row of a tile
  // (wave-uniform); tiles past t_end read as zeros and are never computed.
  for (int seg = 0; seg < n_seg; ++seg) {
    if (seg == 1) t_end = t1;
    constexpr int NB = KVC_PREFETCH + 1;
    int base = __builtin_amdgcn_readfirstlane((seg == 0 ? t0 : seg1_lo) + wave * RPP);
    const int n_tiles = base < t_end ? (t_end - base + TS - 1) / TS : 0;
    if (n_tiles > 0) {
      u32x4 KB[NB][U], VB[NB][U];
#pragma unroll
      for (int r = 0; r < NB - 1; ++r) load_tile(base + r * TS, KB[r], VB[r]);
      bool done = false;
      for (int it = 0; !done; it += NB) {
#pragma unroll
        for (int r = 0; r < NB; ++r) {       // unrolled: ring slots are compile-time
          load_tile(base + (NB - 1) * TS, KB[(r + NB - 1) % NB], VB[(r + NB - 1) % NB]);
          compute_tile(base, KB[r], VB[r]);
          base += TS;
          if (it + r + 1 >= n_tiles) {
            done = true;
            break;
          }
        }
      }
    }
  }
  if (has_x && wave == 0) {                    // the last attended row: lane group 0, pass 0
    u32x4 K[U], V[U];
    float bias[U];
    int row_at[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      K[u] = u == 0 ? nk : u32x4{0u, 0u, 0u, 0u};
      V[u] = u == 0 ? nv : u32x4{0u, 0u, 0u, 0u};
      bias[u] = (u == 0 && grp == 0) ? 0.f : -INFINITY;
      row_at[u] = xrow;
    }
    compute_rows(K, V, bias, row_at);
  }
  }   // vector-ALU path

  if (!kQuant && has_x && wave == 0 && x_new && hb == 0 && grp == 0) {   // fused append: write the new row
    const int64_t ao = slot_offset(p, b, g, arow);
    if (ao >= 0) {
      *reinterpret_cast<u32x4*>(p.k + ao + li * 16) = nk;
      *reinterpret_cast<u32x4*>(p.v + ao + li * 16) = nv;
    } else if (lane == 0) {
      flag(p, KVC_DEVERR_PAGE);
    }
  }

  if constexpr (kLdsMerge) {
#pragma unroll
    for (int j = 0; j < GB; ++j)
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *reinterpret_cast<f32x4*>(&sm_acc[wave][grp][j][li * EPL + e]) =
            f32x4{acc[j][e], acc[j][e + 1], acc[j][e + 2], acc[j][e + 3]};
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < GB; ++j) {
        sm_ml[wave][j][0] = ref[j];
        sm_ml[wave][j][1] = l[j];
      }
    }
  } else {
  // Merge the RPP lane groups of this wave (lanes li, li+LPR, li+2*LPR, ...).
#pragma unroll
  for (int off = LPR; off < 64; off *= 2) {
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      const float r2 = __shfl_xor(ref[j], off);
      const float l2 = __shfl_xor(l[j], off);
      float a2[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) a2[e] = __shfl_xor(acc[j][e], off);
      merge_state(ref[j], l[j], acc[j], r2, l2, a2, EPL);
    }
  }
  if (lane < LPR) {
#pragma unroll
    for (int j = 0; j < GB; ++j) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_a[wave][j][li * EPL + e] = acc[j][e];
      if (lane == 0) {
        sm_ml[wave][j][0] = ref[j];
        sm_ml[wave][j][1] = l[j];
      }
    }
  }
  }
  __syncthreads();

  // Merge the NW waves: each thread takes (head, four output columns) items.
  constexpr int TPT = (GB * D4 + NW * 64 - 1) / (NW * 64);   // items per thread
  float aa[TPT][4], rv[TPT], lv[TPT];
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int t = threadIdx.x + i * NW * 64;
    const int j = t / D4;
    const int d = (t - j * D4) * 4;
    rv[i] = kEmpty;
    lv[i] = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) aa[i][e] = 0.f;
    if (t >= nh * D4) continue;
    float rr = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) rr = fmaxf(rr, sm_ml[w][j][0]);
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float rw = sm_ml[w][j][0];
      const float c = (rw == -INFINITY) ? 0.f : fast_exp2(rw - rr);
      lv[i] += sm_ml[w][j][1] * c;
      if constexpr (kLdsMerge) {
        f32x4 sg = *reinterpret_cast<const f32x4*>(&sm_acc[w][0][j][d]);
#pragma unroll
        for (int g2 = 1; g2 < RPP; ++g2) sg += *reinterpret_cast<const f32x4*>(&sm_acc[w][g2][j][d]);
#pragma unroll
        for (int e = 0; e < 4; ++e) aa[i][e] += sg[e] * c;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) aa[i][e] += sm_a[w][j][d + e] * c;
      }
    }
    rv[i] = rr;
  }
  auto write_out = [&]() {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int t = threadIdx.x + i * NW * 64;
      if (t >= nh * D4) continue;
      const int j = t / D4;
      const int d = (t - j * D4) * 4;
      const float inv = 1.f / lv[i];
      const int64_t orow = pair_row(p, b, g, v_first + j) * D + d;
#pragma unroll
      for (int e = 0; e < 4; ++e) store_out<ET>(p, orow + e, aa[i][e] * inv);
    }
  };
  if (ns == 1) {                                   // a single active split: done
    write_out();
    return;
  }

  // Several splits. The last active split merges; the others publish their
  // partial (reference, sum, unnormalised output), wait for the stores to
  // complete and raise their split's ready flag to epoch + 1. The merging
  // workgroup waits for the other splits' flags, folds the partials in,
  // writes the output and advances the item's epoch for the next call. It
  // has the highest workgroup id of its item, and a workgroup that publishes
  // never waits, so with workgroups dispatched in id order on each XCD every
  // awaited workgroup is dispatched and finishes; the wait is bounded all the
  // same.
  // partial rows: [B, H_kv * pairs, S] (for decode, [B, H_q, S])
  const int64_t prow0 = ((static_cast<int64_t>(b) * p.n_kv + g) * gv + v_first) * p.n_splits;
  const __amdgpu_buffer_rsrc_t ors = make_rsrc(p.ws_o + prow0 * D, static_cast<uint32_t>(nh * p.n_splits * D * 4));
  const __amdgpu_buffer_rsrc_t mrs = make_rsrc(p.ws_ml + prow0 * 2, static_cast<uint32_t>(nh * p.n_splits * 2 * 4));
  const __amdgpu_buffer_rsrc_t frs = make_rsrc(flags, static_cast<uint32_t>(p.flag_stride * 4));
  // first use of the epoch: its load (issued at entry) is waited for here,
  // not in front of the stream
  asm volatile("" : "+v"(epoch));
  if (split != ns - 1) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int t = threadIdx.x + i * NW * 64;
      if (t >= nh * D4) continue;
      const int j = t / D4;
      const int d = (t - j * D4) * 4;
      const uint32_t row = static_cast<uint32_t>(j * p.n_splits + split);
      buf_store_xchg(ors, (row * D + d) * 4u,
                         u32x4{__float_as_uint(aa[i][0]), __float_as_uint(aa[i][1]), __float_as_uint(aa[i][2]),
                               __float_as_uint(aa[i][3])});
      if (d == 0) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(rv[i]), mrs, static_cast<int>(row * 8u), 0, kXchg);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lv[i]), mrs, static_cast<int>(row * 8u + 4u), 0, kXchg);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0)
      __builtin_amdgcn_raw_buffer_store_b32(epoch + 1u, frs, static_cast<int>(split * 4), 0, kXchg);
    return;
  }

  // The merging workgroup: wait for the other splits' flags to reach this
  // call's value (epoch + 1).
  for (int k = threadIdx.x; k < ns - 1; k += blockDim.x) {
    int spins = 0;
    for (;;) {
#if KVC_XCHG_L2_POLL
      // (a compare-and-swap that writes back what it finds: an atomic, so it
      // is performed in L2 and returns L2's value; an idempotent add or load
      // would be turned into a load the CU's L1 may serve)
      uint32_t f = epoch + 1u;
      __hip_atomic_compare_exchange_strong(flags + k, &f, epoch + 1u, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_WORKGROUP);
#else
      const uint32_t f = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(frs, k * 4, 0, kXchg));
#endif
      if (f == epoch + 1u) break;
      if (++spins > p.merge_spins) {             // never expected: flag the call, do not hang
        if (p.status != nullptr) atomicOr(p.status, KVC_DEVERR_SYNC);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      asm volatile("" ::: "memory");
    }
  }
  __syncthreads();
  // Fold all splits in split order, eight per round trip, this workgroup's own
  // (last) split taken from registers, so the order, and with it every output
  // bit, is the same on every run. The other splits' (reference,
  // sum) pairs and partial outputs are requested together (unconditional
  // loads: rows past the split count read another head's data or, past the
  // region, zeros, and are weighted 0), then merged with a running reference.
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int t = threadIdx.x + i * NW * 64;
    if (t >= nh * D4) continue;
    const int j = t / D4;
    const int d = (t - j * D4) * 4;
    const uint32_t row0 = static_cast<uint32_t>(j * p.n_splits);
    float mm = -INFINITY, ll = 0.f, am[4] = {0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < ns; i0 += 8) {
      float rb[8], lb[8];
      u32x4 ob[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t row = row0 + static_cast<uint32_t>(i0 + k);
        rb[k] = __uint_as_float(static_cast<uint32_t>(
            __builtin_amdgcn_raw_buffer_load_b32(mrs, static_cast<int>(row * 8u), 0, kXchg)));
        lb[k] = __uint_as_float(static_cast<uint32_t>(
            __builtin_amdgcn_raw_buffer_load_b32(mrs, static_cast<int>(row * 8u + 4u), 0, kXchg)));
        ob[k] = buf_load_xchg(ors, (row * D + d) * 4u);
      }
      bool use[8];
      float bm = -INFINITY;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        use[k] = i0 + k < ns;
        if (i0 + k == split) {                 // own split: from registers
          rb[k] = rv[i];
          lb[k] = lv[i];
          ob[k] = u32x4{__float_as_uint(aa[i][0]), __float_as_uint(aa[i][1]), __float_as_uint(aa[i][2]),
                        __float_as_uint(aa[i][3])};
        }
        bm = use[k] ? fmaxf(bm, rb[k]) : bm;
      }
      const float nm = fmaxf(mm, bm);
      const float c = (mm == -INFINITY) ? 0.f : fast_exp2(mm - nm);
      ll *= c;
#pragma unroll
      for (int e = 0; e < 4; ++e) am[e] *= c;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float w = use[k] ? fast_exp2(rb[k] - nm) : 0.f;
        ll = fmaf(use[k] ? lb[k] : 0.f, w, ll);
#pragma unroll
        for (int e = 0; e < 4; ++e) am[e] = fmaf(use[k] ? __uint_as_float(ob[k][e]) : 0.f, w, am[e]);
      }
      mm = nm;
    }
    lv[i] = ll;
#pragma unroll
    for (int e = 0; e < 4; ++e) aa[i][e] = am[e];
  }
  write_out();
  // the next call on this workspace waits for flags of epoch + 2
  if (threadIdx.x == 0)
    __builtin_amdgcn_raw_buffer_store_b32(epoch + 1u, frs, static_cast<int>((p.flag_stride - 1) * 4), 0, kXchg);
}

// ------------------------------------------------------------- dispatch --

typedef void (*DecodeKernel)(const DecodeParams);

template <typename ET, int D>
DecodeKernel pick_gb(int gb) {
  switch (gb) {
    case 1: return decode_kernel<ET, D, 1>;
    case 2: return decode_kernel<ET, D, 2>;
    case 4: return decode_kernel<ET, D, 4>;
    default: return decode_kernel<ET, D, 8>;
  }
}

template <typename ET>
DecodeKernel pick_d(int d, int gb) {
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

DecodeKernel pick_decode_kernel(int dtype, int d, int gb) {
  switch (dtype) {
    case KVC_F32: return pick_d<F32T>(d, gb);
    case KVC_F16: return pick_d<F16T>(d, gb);
    case KVC_BF16: return pick_d<BF16T>(d, gb);
    default: return nullptr;
  }
}

template <typename ET, int D, int KQ>
DecodeKernel pick_gb_quant(int gb) {
  switch (gb) {
    case 1: return decode_kernel<ET, D, 1, KQ>;
    case 2: return decode_kernel<ET, D, 2, KQ>;
    case 4: return decode_kernel<ET, D, 4, KQ>;
    default: return decode_kernel<ET, D, 8, KQ>;
  }
}

template <typename ET, int KQ>
DecodeKernel pick_d_quant(int d, int gb) {
  switch (d) {
    case 64: return pick_gb_quant<ET, 64, KQ>(gb);
    case 128: return pick_gb_quant<ET, 128, KQ>(gb);
    case 256: return pick_gb_quant<ET, 256, KQ>(gb);
    default: return nullptr;
  }
}

// Decode over 8-bit codes: q (and out) fp16 or bf16.
DecodeKernel pick_quant_kernel(int format, int q_dtype, int d, int gb) {
  const bool fp8 = format == KVC_QFMT_FP8_E4M3;
  if (q_dtype == KVC_F16) return fp8 ? pick_d_quant<F16T, kQuantFp8>(d, gb) : pick_d_quant<F16T, kQuantInt8>(d, gb);
  if (q_dtype == KVC_BF16) return fp8 ? pick_d_quant<BF16T, kQuantFp8>(d, gb) : pick_d_quant<BF16T, kQuantInt8>(d, gb);
  return nullptr;
}

// Workgroups of a decode launch over `units` (sequence, KV head) units: see
// the id mapping at the top of decode_kernel.
int64_t decode_grid(int64_t units, int32_t splits, int32_t n_hblk) {
#if KVC_XCD_COLOCATE
  return (units + 7) / 8 * 8 * splits * n_hblk;
#else
  return (units * splits + 7) / 8 * 8 * n_hblk;
#endif
}

// ------------------------------------------------ quantised append / fill --

struct QuantParams {
  char* kc;                  // codes
  char* vc;
  char* ks;                  // scales
  char* vs;
  int64_t cb, ch, ct;        // code strides in bytes
  int64_t ssb, ssh;          // scale strides in bytes (4 bytes per token)
  const char* src_k;         // new rows [B, H_kv, T_new, D] of the input type
  const char* src_v;
  int64_t sb, sh, st;        // their strides in bytes
  const int32_t* seq_lens;
  uint32_t* status;
  int32_t batch, n_kv, max_len, t_new;
};

// One wave per new row (K rows, then V rows): lane l holds elements
// [l*E, l*E + E). amax over the row by a wave-wide maximum, scale = amax /
// QMAX and each code from x / scale, both fp32 divisions (correctly rounded),
// then E code bytes per lane and the scale from lane 0.
template <typename IT, int KQ, int D>
__global__ __launch_bounds__(256) void quant_rows_kernel(const QuantParams p) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t rows = static_cast<int64_t>(p.batch) * p.n_kv * p.t_new;
  const int64_t n_waves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  for (int64_t r = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6; r < 2 * rows; r += n_waves) {
    const bool is_v = r >= rows;
    const int64_t rr = is_v ? r - rows : r;
    const int i = static_cast<int>(rr % p.t_new);
    const int64_t bg = rr / p.t_new;
    const int g = static_cast<int>(bg % p.n_kv);
    const int b = static_cast<int>(bg / p.n_kv);
    const int pos = p.seq_lens[b];
    if (pos < 0 || static_cast<int64_t>(pos) + p.t_new > p.max_len) {   // whole sequence skipped
      if (lane == 0 && !is_v && g == 0 && i == 0 && p.status != nullptr)
        atomicOr(p.status, pos < 0 ? KVC_DEVERR_BADLEN : KVC_DEVERR_CAPACITY);
      continue;
    }
    const char* src = (is_v ? p.src_v : p.src_k) + b * p.sb + g * p.sh + static_cast<int64_t>(i) * p.st;
    uint32_t packed;
    const float scale = quant_row<IT, KQ, D>(src, lane, packed);
    const int slot = pos + i;
    store_codes<E>((is_v ? p.vc : p.kc) + b * p.cb + g * p.ch + static_cast<int64_t>(slot) * p.ct + lane * E, packed);
    if (lane == 0)
      *reinterpret_cast<float*>((is_v ? p.vs : p.ks) + b * p.ssb + g * p.ssh + static_cast<int64_t>(slot) * 4) = scale;
  }
}

typedef void (*QuantKernel)(const QuantParams);

template <typename IT, int KQ>
QuantKernel pick_quant_rows_d(int d) {
  switch (d) {
    case 64: return quant_rows_kernel<IT, KQ, 64>;
    case 128: return quant_rows_kernel<IT, KQ, 128>;
    case 256: return quant_rows_kernel<IT, KQ, 256>;
    default: return nullptr;
  }
}

template <int KQ>
QuantKernel pick_quant_rows_t(int in_dtype, int d) {
  switch (in_dtype) {
    case KVC_F32: return pick_quant_rows_d<F32T, KQ>(d);
    case KVC_F16: return pick_quant_rows_d<F16T, KQ>(d);
    case KVC_BF16: return pick_quant_rows_d<BF16T, KQ>(d);
    default: return nullptr;
  }
}

kvc_status_t launch_quant_rows(const kvc_qcache_t* c, const int32_t* seq_lens, const void* k, const void* v,
                               int64_t sb, int64_t sh, int64_t st, int32_t t_new, uint32_t* status,
                               hipStream_t stream, bool check_only = false) {
  kvc_status_t rc = kvc::check_qcache(c, false);
  if (rc != KVC_OK) return rc;
  if (t_new < 0) return KVC_ERR_SHAPE;
  if (c->batch == 0 || t_new == 0) return KVC_OK;
  if (seq_lens == nullptr || k == nullptr || v == nullptr) return KVC_ERR_NULL;
  if (sb < 0 || sh < 0 || st < 0) return KVC_ERR_SHAPE;
  if (t_new > 1 && st < c->head_dim) return KVC_ERR_SHAPE;
  const int s = kvc::elem_bytes(c->in_dtype);
  if (reinterpret_cast<uintptr_t>(k) % s || reinterpret_cast<uintptr_t>(v) % s) return KVC_ERR_ALIGN;
  const QuantKernel kern = c->format == KVC_QFMT_FP8_E4M3 ? pick_quant_rows_t<kQuantFp8>(c->in_dtype, c->head_dim)
                                                          : pick_quant_rows_t<kQuantInt8>(c->in_dtype, c->head_dim);
  if (kern == nullptr) return KVC_ERR_UNSUPPORTED;
  QuantParams p;
  p.kc = static_cast<char*>(c->k);
  p.vc = static_cast<char*>(c->v);
  p.ks = reinterpret_cast<char*>(c->k_scale);
  p.vs = reinterpret_cast<char*>(c->v_scale);
  p.cb = c->stride_b;
  p.ch = c->stride_h;
  p.ct = c->stride_t;
  p.ssb = c->scale_stride_b * 4;
  p.ssh = c->scale_stride_h * 4;
  p.src_k = static_cast<const char*>(k);
  p.src_v = static_cast<const char*>(v);
  p.sb = sb * s;
  p.sh = sh * s;
  p.st = st * s;
  p.seq_lens = seq_lens;
  p.status = status;
  p.batch = c->batch;
  p.n_kv = c->n_kv_heads;
  p.max_len = c->max_len;
  p.t_new = t_new;
  const int64_t waves = 2 * static_cast<int64_t>(c->batch) * c->n_kv_heads * t_new;
  int64_t blocks = (waves + 3) / 4;             // 4 waves per 256-thread block
  if (blocks > 65536) blocks = 65536;           // the wave loop covers the rest
  if (check_only) return KVC_OK;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, p);
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

// k_new != nullptr: the fused step (the new rows quantised into slot
// seq_lens[b] by the workgroup that attends them; n_pending must be 1).
kvc_status_t launch_quant_decode(const kvc_qcache_t* c, const int32_t* seq_lens, int32_t n_pending, const void* q,
                                 int32_t n_q_heads, float scale, void* out, int32_t out_dtype, void* workspace,
                                 size_t workspace_bytes, int32_t n_splits, uint32_t* dev_status,
                                 hipStream_t stream, const void* k_new = nullptr, const void* v_new = nullptr,
                                 int64_t new_stride_b = 0, int64_t new_stride_h = 0, bool check_only = false) {
  kvc_status_t rc = kvc::check_qcache(c, true);
  if (rc != KVC_OK) return rc;
  if (n_q_heads <= 0 || n_q_heads % c->n_kv_heads != 0) return KVC_ERR_GQA;
  if (n_pending < 0 || n_splits < 0 || n_splits > KVC_MAX_SPLITS) return KVC_ERR_SHAPE;
  if (out_dtype != KVC_F32 && out_dtype != c->in_dtype) return KVC_ERR_DTYPE;
  const float scale_log2 = scale * 1.44269504088896340736f;  // log2(e)
  if (!(scale > 0.f) || !(scale_log2 < INFINITY)) return KVC_ERR_UNSUPPORTED;
  if (c->batch == 0) return KVC_OK;
  if (seq_lens == nullptr || q == nullptr || out == nullptr) return KVC_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(q) % 16) return KVC_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(out) % kvc::elem_bytes(out_dtype)) return KVC_ERR_ALIGN;
  if ((static_cast<int64_t>(c->max_len) + 2048) * c->stride_t > 0x7fffffffll) return KVC_ERR_SHAPE;
  const int s_in = kvc::elem_bytes(c->in_dtype);
  if (k_new != nullptr) {
    if (v_new == nullptr) return KVC_ERR_NULL;
    if (new_stride_b < 0 || new_stride_h < 0) return KVC_ERR_SHAPE;
    if (c->n_kv_heads > 1 && new_stride_h < c->head_dim) return KVC_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(k_new) % s_in || reinterpret_cast<uintptr_t>(v_new) % s_in) return KVC_ERR_ALIGN;
  }
  const kvc_cache_t view = kvc::qcache_view(c);
  // Groups of 16+ query heads (MQA, wide GQA) run on the wide-group kernel's
  // 8-bit mode, which reads each KV head's codes once per 128 heads; the
  // decode kernel's head blocks of 8 would read them once per block. (A
  // fused append is not part of that mode: kvc_quant_decode_step then
  // enqueues the append and this call.)
  const bool wide = k_new == nullptr && kvc::quant_routes_wide(c, n_q_heads);
  const int32_t splits = n_splits > 0 ? n_splits : kvc::auto_splits(&view, n_q_heads, wide);
  const size_t need = kvc::workspace_bytes(&view, n_q_heads, splits);
  if (workspace == nullptr || workspace_bytes < need) return KVC_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 16) return KVC_ERR_ALIGN;
  const int group = n_q_heads / c->n_kv_heads;
  if (wide) {
    const kvc::WsRegions wr = kvc::workspace_regions(&view, n_q_heads, splits, workspace);
    kvc::WideQuant wq;
    wq.format = c->format;
    wq.q_dtype = c->in_dtype;
    wq.k_scale = c->k_scale;
    wq.v_scale = c->v_scale;
    wq.scale_stride_b = c->scale_stride_b;
    wq.scale_stride_h = c->scale_stride_h;
    return kvc::launch_wide(&view, seq_lens, n_pending, nullptr, nullptr, 0, 0, 0, q, n_q_heads, 0, scale_log2, out,
                            out_dtype, wr, splits, nullptr, dev_status, stream, check_only, &wq);
  }
  const DecodeKernel k = pick_quant_kernel(c->format, c->in_dtype, c->head_dim, kvc::heads_per_block(group));
  if (k == nullptr) return KVC_ERR_UNSUPPORTED;

  DecodeParams p = {};
  p.k = static_cast<char*>(c->k);
  p.v = static_cast<char*>(c->v);
  p.sb = c->stride_b;
  p.sh = c->stride_h;
  p.st = c->stride_t;
  p.seq_lens = seq_lens;
  p.q = static_cast<const char*>(q);
  p.k_new = static_cast<const char*>(k_new);
  p.v_new = static_cast<const char*>(v_new);
  p.nsb = new_stride_b * s_in;
  p.nsh = new_stride_h * s_in;
  const kvc::WsRegions wr = kvc::workspace_regions(&view, n_q_heads, splits, workspace);
  p.ws_flag = wr.flags;
  p.flag_stride = wr.flag_stride;
  p.ws_o = wr.o;
  p.ws_ml = wr.ml;
  p.lens_next = nullptr;
  p.out = out;
  p.status = dev_status;
  p.batch = c->batch;
  p.n_q = n_q_heads;
  p.n_kv = c->n_kv_heads;
  p.group = group;
  p.n_hblk = kvc::head_blocks(group);
  p.max_len = c->max_len;
  p.n_pending = n_pending;
  p.n_splits = splits;
  p.out_f32 = out_dtype == KVC_F32 ? 1 : 0;
  p.t_q = 1;
  p.block = 0;
  p.table = nullptr;
  p.ring = 0;
  p.k_scale = reinterpret_cast<char*>(c->k_scale);
  p.v_scale = reinterpret_cast<char*>(c->v_scale);
  p.ssb = c->scale_stride_b * 4;
  p.ssh = c->scale_stride_h * 4;
  p.scale_log2 = scale_log2;
  p.merge_spins = kvc::merge_spin_limit();
  const int64_t wgs = decode_grid(static_cast<int64_t>(c->batch) * c->n_kv_heads, splits, p.n_hblk);
  if (wgs > 0x7fffffffll) return KVC_ERR_SHAPE;
  if (check_only) return KVC_OK;
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(wgs)), dim3(KVC_WAVES * 64), 0, stream, p);
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

kvc_status_t launch_copy(const kvc_cache_t* c, const int32_t* seq_lens, const void* ks, const void* vs,
                         int64_t sb, int64_t sh, int64_t st, int32_t t_new, uint32_t* status,
                         hipStream_t stream, const kvc::PageInfo* pg = nullptr, bool ring = false) {
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
  p.table = pg != nullptr ? pg->table : nullptr;
  p.table_stride = pg != nullptr ? pg->table_stride : 0;
  p.page_shift = pg != nullptr ? pg->page_shift : 0;
  p.n_pages = pg != nullptr ? pg->n_pages : 0;
  p.ring = ring ? 1 : 0;
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

// Shared by kvc_decode_attn (k_new == nullptr) and kvc_decode_step.
kvc_status_t launch_decode(const kvc_cache_t* cache, const int32_t* seq_lens, int32_t n_pending, const void* k_new,
                           const void* v_new, int64_t new_stride_b, int64_t new_stride_h, const void* q,
                           int32_t n_q_heads, float scale, void* out, int32_t out_dtype, void* workspace,
                           size_t workspace_bytes, int32_t n_splits, uint32_t* dev_status, hipStream_t stream,
                           int32_t t_q, const kvc::PageInfo* pg = nullptr, bool ring = false,
                           int32_t* lens_next = nullptr, kvc::RegionsFn regions_fn = nullptr,
                           int64_t new_stride_t = 0, bool check_only = false) {
  kvc_status_t st = kvc::check_cache(cache, true);
  if (st != KVC_OK) return st;
  if (n_q_heads <= 0 || n_q_heads % cache->n_kv_heads != 0) return KVC_ERR_GQA;
  // t_q > 0: a block of t_q queries per sequence; the (query, head) pairs are
  // handled as t_q * n_q_heads virtual heads. t_q == 0: single-query decode.
  if (t_q < 0 || static_cast<int64_t>(n_q_heads) * (t_q > 0 ? t_q : 1) > (1 << 24)) return KVC_ERR_SHAPE;
  const int32_t tq = t_q > 0 ? t_q : 1;
  const int32_t n_qv = n_q_heads * tq;
  if (n_pending < 0 || n_splits < 0 || n_splits > KVC_MAX_SPLITS) return KVC_ERR_SHAPE;
  if (out_dtype != KVC_F32 && out_dtype != cache->dtype) return KVC_ERR_DTYPE;
  if (!kvc::decode_head_dim_supported(cache->head_dim, cache->dtype)) return KVC_ERR_UNSUPPORTED;
  // Masked rows enter as -inf scores before scaling: a positive finite scale
  // keeps them -inf (and keeps the order of scores for the running maximum).
  const float scale_log2 = scale * 1.44269504088896340736f;  // log2(e)
  if (!(scale > 0.f) || !(scale_log2 < INFINITY)) return KVC_ERR_UNSUPPORTED;
  if (cache->batch == 0) return KVC_OK;
  if (seq_lens == nullptr || q == nullptr || out == nullptr) return KVC_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(q) % 16) return KVC_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(out) % kvc::elem_bytes(out_dtype)) return KVC_ERR_ALIGN;
  const int s = kvc::elem_bytes(cache->dtype);
  if (k_new != nullptr) {
    if (v_new == nullptr) return KVC_ERR_NULL;
    if (new_stride_b < 0 || new_stride_h < 0) return KVC_ERR_SHAPE;
    if (cache->n_kv_heads > 1 && new_stride_h < cache->head_dim) return KVC_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(k_new) % 16 || reinterpret_cast<uintptr_t>(v_new) % 16 ||
        (new_stride_b * s) % 16 || (new_stride_h * s) % 16)
      return KVC_ERR_ALIGN;
    if (t_q > 0) {                               // a fused fill: the block's rows, on the wide-group kernel only
      if (new_stride_t < 0 || (t_q > 1 && new_stride_t < cache->head_dim)) return KVC_ERR_SHAPE;
      if ((new_stride_t * s) % 16) return KVC_ERR_ALIGN;
      if (pg != nullptr || ring || !kvc::routes_wide(cache, n_qv)) return KVC_ERR_UNSUPPORTED;
    }
  }
  // The kernels address one (sequence, KV head) slice of K/V with 32-bit
  // byte offsets (plus up to two tiles past the end, read back as zeros).
  if ((static_cast<int64_t>(cache->max_len) + 2048) * cache->stride_t * s > 0x7fffffffll) return KVC_ERR_SHAPE;
  // 16-bit caches with 8..512 (query, head) pairs per KV head run on the
  // wide-group kernel (K/V streamed once per 128 pairs, both products on the
  // matrix cores): contiguous caches, and paged and ring caches in decode.
  const bool wide = kvc::routes_wide(cache, n_qv) && ((pg == nullptr && !ring) || t_q == 0);
  const int32_t splits = n_splits > 0 ? n_splits : kvc::auto_splits(cache, n_qv, wide);
  kvc::WsRegions wr;
  if (regions_fn != nullptr) {                   // exchange space the caller of this function lays out
    st = regions_fn(cache, n_qv, splits, &wr);
    if (st != KVC_OK) return st;
  } else {
    const size_t need = kvc::workspace_bytes(cache, n_qv, splits);
    if (workspace == nullptr || workspace_bytes < need) return KVC_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 16) return KVC_ERR_ALIGN;
    wr = kvc::workspace_regions(cache, n_qv, splits, workspace);
  }

  const int group = n_q_heads / cache->n_kv_heads;
  // A block of 8 or more queries with at least 32 (query, head) pairs per KV
  // head that the wide-group kernel does not take (more than 128 pairs, or
  // more than kWideMaxBlock queries) goes to the matrix-core prefill kernel,
  // which reads each query head's K/V once for all its queries; within the
  // wide kernel's range that kernel is faster (it reads each KV head's K/V
  // once for all pairs: gqa_8b verify blocks of 8, 16 and 32 queries 1.8x,
  // 1.6x and 1.2x, mha_7b blocks of 32 and 64 queries 4.7x and 3.8x), and
  // below 32 pairs the decode kernels are. The workspace contract stays the
  // same (checked above); n_splits is then unused.
  if (t_q >= 8 && group * t_q >= 32 && !(wide && t_q <= kvc::kWideMaxBlock) && pg == nullptr && !ring &&
      k_new == nullptr && kvc::prefill_supported(cache->dtype, cache->head_dim))
    return kvc::launch_prefill(cache, seq_lens, t_q, q, n_q_heads, scale, out, out_dtype, dev_status, stream,
                               check_only);
  if (wide)
    return kvc::launch_wide(cache, seq_lens, n_pending, k_new, v_new, new_stride_b, new_stride_h, new_stride_t, q,
                            n_q_heads, t_q, scale_log2, out, out_dtype, wr, splits, lens_next, dev_status, stream,
                            check_only, nullptr, pg, ring);
  const int gb = kvc::heads_per_block(group * tq);
  DecodeParams p;
  p.k = static_cast<char*>(cache->k);
  p.v = static_cast<char*>(cache->v);
  p.sb = cache->stride_b * s;
  p.sh = cache->stride_h * s;
  p.st = cache->stride_t * s;
  p.seq_lens = seq_lens;
  p.q = static_cast<const char*>(q);
  p.k_new = static_cast<const char*>(k_new);
  p.v_new = static_cast<const char*>(v_new);
  p.nsb = new_stride_b * s;
  p.nsh = new_stride_h * s;
  p.ws_flag = wr.flags;
  p.flag_stride = wr.flag_stride;
  p.ws_o = wr.o;
  p.ws_ml = wr.ml;
  p.lens_next = lens_next;
  p.out = out;
  p.status = dev_status;
  p.batch = cache->batch;
  p.n_q = n_q_heads;
  p.n_kv = cache->n_kv_heads;
  p.group = group;
  p.n_hblk = kvc::head_blocks(group * tq);
  p.max_len = cache->max_len;
  p.n_pending = n_pending;
  p.n_splits = splits;
  p.out_f32 = out_dtype == KVC_F32 ? 1 : 0;
  p.scale_log2 = scale_log2;
  p.t_q = tq;
  p.block = t_q > 0 ? 1 : 0;
  p.table = pg != nullptr ? pg->table : nullptr;
  p.table_stride = pg != nullptr ? pg->table_stride : 0;
  p.page_shift = pg != nullptr ? pg->page_shift : 0;
  p.n_pages = pg != nullptr ? pg->n_pages : 0;
  p.ring = ring ? 1 : 0;
  // paged caches are read by the matrix-core path only (16-row tiles)
  if (pg != nullptr && !(s == 2 && cache->head_dim % 32 == 0)) return KVC_ERR_UNSUPPORTED;

  DecodeKernel k = pick_decode_kernel(cache->dtype, cache->head_dim, gb);
  if (k == nullptr) return KVC_ERR_UNSUPPORTED;
  p.merge_spins = kvc::merge_spin_limit();
  const int64_t wgs = decode_grid(static_cast<int64_t>(cache->batch) * cache->n_kv_heads, splits, p.n_hblk);
  if (wgs > 0x7fffffffll) return KVC_ERR_SHAPE;
  if (check_only) return KVC_OK;
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(wgs)), dim3(KVC_WAVES * 64), 0, stream, p);
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
  return launch_decode(cache, seq_lens, n_pending, nullptr, nullptr, 0, 0, q, n_q_heads, scale, out, out_dtype,
                       workspace, workspace_bytes, n_splits, dev_status, stream, 0);
}

extern "C" kvc_status_t kvc_decode_step(const kvc_cache_t* cache, const int32_t* seq_lens, const void* k_new,
                                        const void* v_new, int64_t new_stride_b, int64_t new_stride_h,
                                        const void* q, int32_t n_q_heads, float scale, void* out,
                                        int32_t out_dtype, void* workspace, size_t workspace_bytes,
                                        int32_t n_splits, uint32_t* dev_status, hipStream_t stream) {
  if (k_new == nullptr || v_new == nullptr) {
    kvc_status_t st = kvc::check_cache(cache, true);
    if (st != KVC_OK) return st;
    if (cache->batch > 0) return KVC_ERR_NULL;
  }
  return launch_decode(cache, seq_lens, 1, k_new, v_new, new_stride_b, new_stride_h, q, n_q_heads, scale, out,
                       out_dtype, workspace, workspace_bytes, n_splits, dev_status, stream, 0);
}

extern "C" kvc_status_t kvc_decode_step_advance(const kvc_cache_t* cache, const int32_t* seq_lens,
                                                int32_t* seq_lens_next, const void* k_new, const void* v_new,
                                                int64_t new_stride_b, int64_t new_stride_h, const void* q,
                                                int32_t n_q_heads, float scale, void* out, int32_t out_dtype,
                                                void* workspace, size_t workspace_bytes, int32_t n_splits,
                                                uint32_t* dev_status, hipStream_t stream) {
  if (cache != nullptr && cache->batch > 0) {
    if (k_new == nullptr || v_new == nullptr || seq_lens_next == nullptr) return KVC_ERR_NULL;
    // the two length arrays must not overlap: the launch reads one and writes the other
    const int32_t* a = seq_lens;
    const int32_t* e = seq_lens_next;
    if (a != nullptr && e < a + cache->batch && a < e + cache->batch) return KVC_ERR_SHAPE;
  }
  return launch_decode(cache, seq_lens, 1, k_new, v_new, new_stride_b, new_stride_h, q, n_q_heads, scale, out,
                       out_dtype, workspace, workspace_bytes, n_splits, dev_status, stream, 0, nullptr, false,
                       seq_lens_next);
}

kvc_status_t kvc::decode_step_in_regions(const kvc_cache_t* cache, const int32_t* seq_lens, const void* k_new,
                                         const void* v_new, int64_t new_stride_b, int64_t new_stride_h,
                                         const void* q, int32_t n_q_heads, float scale, void* out, int32_t out_dtype,
                                         int32_t n_splits, uint32_t* dev_status, hipStream_t stream,
                                         RegionsFn regions_fn) {
  return launch_decode(cache, seq_lens, 1, k_new, v_new, new_stride_b, new_stride_h, q, n_q_heads, scale, out,
                       out_dtype, nullptr, 0, n_splits, dev_status, stream, 0, nullptr, false, nullptr, regions_fn);
}

extern "C" kvc_status_t kvc_block_attn(const kvc_cache_t* cache, const int32_t* seq_lens, int32_t t_q, const void* q,
                                       int32_t n_q_heads, float scale, void* out, int32_t out_dtype, void* workspace,
                                       size_t workspace_bytes, int32_t n_splits, uint32_t* dev_status,
                                       hipStream_t stream) {
  if (cache == nullptr) return KVC_ERR_NULL;
  if (t_q <= 0) return KVC_ERR_SHAPE;
  return launch_decode(cache, seq_lens, 0, nullptr, nullptr, 0, 0, q, n_q_heads, scale, out, out_dtype, workspace,
                       workspace_bytes, n_splits, dev_status, stream, t_q);
}

extern "C" kvc_status_t kvc_block_step(const kvc_cache_t* cache, const int32_t* seq_lens, int32_t t_q,
                                       const void* k_new, const void* v_new, int64_t new_stride_b,
                                       int64_t new_stride_h, int64_t new_stride_t, const void* q, int32_t n_q_heads,
                                       float scale, void* out, int32_t out_dtype, void* workspace,
                                       size_t workspace_bytes, int32_t n_splits, uint32_t* dev_status,
                                       hipStream_t stream) {
  if (cache == nullptr) return KVC_ERR_NULL;
  if (t_q <= 0) return KVC_ERR_SHAPE;
  kvc_status_t st = kvc::check_cache(cache, false);
  if (st != KVC_OK) return st;
  if (cache->batch > 0 && (k_new == nullptr || v_new == nullptr)) return KVC_ERR_NULL;
  if (new_stride_b < 0 || new_stride_h < 0 || new_stride_t < 0) return KVC_ERR_SHAPE;
  if (t_q > 1 && new_stride_t < cache->head_dim) return KVC_ERR_SHAPE;
  const int s = kvc::elem_bytes(cache->dtype);
  if (reinterpret_cast<uintptr_t>(k_new) % s || reinterpret_cast<uintptr_t>(v_new) % s) return KVC_ERR_ALIGN;
  // One launch where the wide-group kernel serves the block (it folds the
  // block's rows in from k_new/v_new and writes them into the cache): 16-byte
  // aligned rows, and the rows within what its threads copy in one pass.
  const bool gqa_ok = n_q_heads > 0 && n_q_heads % cache->n_kv_heads == 0;
  const bool aligned = reinterpret_cast<uintptr_t>(k_new) % 16 == 0 && reinterpret_cast<uintptr_t>(v_new) % 16 == 0 &&
                       (new_stride_b * s) % 16 == 0 && (new_stride_h * s) % 16 == 0 && (new_stride_t * s) % 16 == 0;
  if (gqa_ok && aligned && kvc::routes_wide(cache, static_cast<int32_t>(n_q_heads * t_q)) &&
      static_cast<int64_t>(t_q) * (cache->head_dim / 8) <= 512)
    return launch_decode(cache, seq_lens, 0, k_new, v_new, new_stride_b, new_stride_h, q, n_q_heads, scale, out,
                         out_dtype, workspace, workspace_bytes, n_splits, dev_status, stream, t_q, nullptr, false,
                         nullptr, nullptr, new_stride_t);
  // Otherwise the fill, then the attention; the attention's checks run
  // first, so that a call that fails enqueues nothing.
  st = launch_decode(cache, seq_lens, 0, nullptr, nullptr, 0, 0, q, n_q_heads, scale, out, out_dtype, workspace,
                     workspace_bytes, n_splits, dev_status, stream, t_q, nullptr, false, nullptr, nullptr, 0, true);
  if (st != KVC_OK || cache->batch == 0) return st;
  st = launch_copy(cache, seq_lens, k_new, v_new, new_stride_b, new_stride_h, new_stride_t, t_q, dev_status, stream);
  if (st != KVC_OK) return st;
  return launch_decode(cache, seq_lens, 0, nullptr, nullptr, 0, 0, q, n_q_heads, scale, out, out_dtype, workspace,
                       workspace_bytes, n_splits, dev_status, stream, t_q);
}

extern "C" kvc_status_t kvc_seq_lens_advance(int32_t* seq_lens, int32_t batch, int32_t n, hipStream_t stream) {
  if (batch < 0) return KVC_ERR_SHAPE;
  if (batch == 0) return KVC_OK;
  if (seq_lens == nullptr) return KVC_ERR_NULL;
  hipLaunchKernelGGL(advance_kernel, dim3((batch + 255) / 256), dim3(256), 0, stream, seq_lens, batch, n);
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

// ------------------------------------------------------------ paged cache --

extern "C" kvc_status_t kvc_paged_append(const kvc_paged_cache_t* cache, const int32_t* seq_lens,
                                         const void* k_new, const void* v_new, int64_t new_stride_b,
                                         int64_t new_stride_h, uint32_t* dev_status, hipStream_t stream) {
  kvc_cache_t view;
  kvc::PageInfo info;
  kvc_status_t st = kvc::paged_view(cache, false, &view, &info);
  if (st != KVC_OK) return st;
  st = kvc::check_cache(&view, false);
  if (st != KVC_OK) return st;
  if (view.batch == 0) return KVC_OK;
  if (seq_lens == nullptr || k_new == nullptr || v_new == nullptr) return KVC_ERR_NULL;
  if (new_stride_b < 0 || new_stride_h < 0) return KVC_ERR_SHAPE;
  if (view.n_kv_heads > 1 && new_stride_h < view.head_dim) return KVC_ERR_SHAPE;
  const int s = kvc::elem_bytes(view.dtype);
  if (reinterpret_cast<uintptr_t>(k_new) % s || reinterpret_cast<uintptr_t>(v_new) % s) return KVC_ERR_ALIGN;
  return launch_copy(&view, seq_lens, k_new, v_new, new_stride_b, new_stride_h, 0, 1, dev_status, stream, &info);
}

extern "C" kvc_status_t kvc_paged_prefill_fill(const kvc_paged_cache_t* cache, const int32_t* seq_lens,
                                               const void* k, const void* v, int64_t src_stride_b,
                                               int64_t src_stride_h, int64_t src_stride_t, int32_t t_new,
                                               uint32_t* dev_status, hipStream_t stream) {
  kvc_cache_t view;
  kvc::PageInfo info;
  kvc_status_t st = kvc::paged_view(cache, false, &view, &info);
  if (st != KVC_OK) return st;
  st = kvc::check_cache(&view, false);
  if (st != KVC_OK) return st;
  if (t_new < 0) return KVC_ERR_SHAPE;
  if (view.batch == 0 || t_new == 0) return KVC_OK;
  if (seq_lens == nullptr || k == nullptr || v == nullptr) return KVC_ERR_NULL;
  if (src_stride_b < 0 || src_stride_h < 0 || src_stride_t < 0) return KVC_ERR_SHAPE;
  if (t_new > 1 && src_stride_t < view.head_dim) return KVC_ERR_SHAPE;
  const int s = kvc::elem_bytes(view.dtype);
  if (reinterpret_cast<uintptr_t>(k) % s || reinterpret_cast<uintptr_t>(v) % s) return KVC_ERR_ALIGN;
  return launch_copy(&view, seq_lens, k, v, src_stride_b, src_stride_h, src_stride_t, t_new, dev_status, stream,
                     &info);
}

extern "C" kvc_status_t kvc_paged_decode_attn(const kvc_paged_cache_t* cache, const int32_t* seq_lens,
                                              int32_t n_pending, const void* q, int32_t n_q_heads, float scale,
                                              void* out, int32_t out_dtype, void* workspace,
                                              size_t workspace_bytes, int32_t n_splits, uint32_t* dev_status,
                                              hipStream_t stream) {
  kvc_cache_t view;
  kvc::PageInfo info;
  const kvc_status_t st = kvc::paged_view(cache, true, &view, &info);
  if (st != KVC_OK) return st;
  return launch_decode(&view, seq_lens, n_pending, nullptr, nullptr, 0, 0, q, n_q_heads, scale, out, out_dtype,
                       workspace, workspace_bytes, n_splits, dev_status, stream, 0, &info);
}

extern "C" kvc_status_t kvc_paged_decode_step(const kvc_paged_cache_t* cache, const int32_t* seq_lens,
                                              const void* k_new, const void* v_new, int64_t new_stride_b,
                                              int64_t new_stride_h, const void* q, int32_t n_q_heads, float scale,
                                              void* out, int32_t out_dtype, void* workspace,
                                              size_t workspace_bytes, int32_t n_splits, uint32_t* dev_status,
                                              hipStream_t stream) {
  kvc_cache_t view;
  kvc::PageInfo info;
  const kvc_status_t st = kvc::paged_view(cache, true, &view, &info);
  if (st != KVC_OK) return st;
  if (view.batch > 0 && (k_new == nullptr || v_new == nullptr)) return KVC_ERR_NULL;
  return launch_decode(&view, seq_lens, 1, k_new, v_new, new_stride_b, new_stride_h, q, n_q_heads, scale, out,
                       out_dtype, workspace, workspace_bytes, n_splits, dev_status, stream, 0, &info);
}

// ------------------------------------------------------------- ring cache --

extern "C" kvc_status_t kvc_ring_append(const kvc_cache_t* cache, const int32_t* seq_lens, const void* k_new,
                                        const void* v_new, int64_t new_stride_b, int64_t new_stride_h,
                                        uint32_t* dev_status, hipStream_t stream) {
  kvc_status_t st = kvc::check_cache(cache, false);
  if (st != KVC_OK) return st;
  if (cache->batch == 0) return KVC_OK;
  if (cache->max_len <= 0) return KVC_ERR_SHAPE;
  if (seq_lens == nullptr || k_new == nullptr || v_new == nullptr) return KVC_ERR_NULL;
  if (new_stride_b < 0 || new_stride_h < 0) return KVC_ERR_SHAPE;
  if (cache->n_kv_heads > 1 && new_stride_h < cache->head_dim) return KVC_ERR_SHAPE;
  const int s = kvc::elem_bytes(cache->dtype);
  if (reinterpret_cast<uintptr_t>(k_new) % s || reinterpret_cast<uintptr_t>(v_new) % s) return KVC_ERR_ALIGN;
  return launch_copy(cache, seq_lens, k_new, v_new, new_stride_b, new_stride_h, 0, 1, dev_status, stream, nullptr,
                     true);
}

extern "C" kvc_status_t kvc_ring_prefill_fill(const kvc_cache_t* cache, const int32_t* seq_lens, const void* k,
                                              const void* v, int64_t src_stride_b, int64_t src_stride_h,
                                              int64_t src_stride_t, int32_t t_new, uint32_t* dev_status,
                                              hipStream_t stream) {
  kvc_status_t st = kvc::check_cache(cache, false);
  if (st != KVC_OK) return st;
  if (t_new < 0) return KVC_ERR_SHAPE;
  if (cache->batch == 0 || t_new == 0) return KVC_OK;
  if (cache->max_len <= 0) return KVC_ERR_SHAPE;
  if (seq_lens == nullptr || k == nullptr || v == nullptr) return KVC_ERR_NULL;
  if (src_stride_b < 0 || src_stride_h < 0 || src_stride_t < 0) return KVC_ERR_SHAPE;
  if (t_new > 1 && src_stride_t < cache->head_dim) return KVC_ERR_SHAPE;
  const int s = kvc::elem_bytes(cache->dtype);
  if (reinterpret_cast<uintptr_t>(k) % s || reinterpret_cast<uintptr_t>(v) % s) return KVC_ERR_ALIGN;
  return launch_copy(cache, seq_lens, k, v, src_stride_b, src_stride_h, src_stride_t, t_new, dev_status, stream,
                     nullptr, true);
}

extern "C" kvc_status_t kvc_ring_decode_attn(const kvc_cache_t* cache, const int32_t* seq_lens, int32_t n_pending,
                                             const void* q, int32_t n_q_heads, float scale, void* out,
                                             int32_t out_dtype, void* workspace, size_t workspace_bytes,
                                             int32_t n_splits, uint32_t* dev_status, hipStream_t stream) {
  if (cache != nullptr && cache->batch > 0 && cache->max_len <= 0) return KVC_ERR_SHAPE;
  return launch_decode(cache, seq_lens, n_pending, nullptr, nullptr, 0, 0, q, n_q_heads, scale, out, out_dtype,
                       workspace, workspace_bytes, n_splits, dev_status, stream, 0, nullptr, true);
}

extern "C" kvc_status_t kvc_ring_decode_step(const kvc_cache_t* cache, const int32_t* seq_lens, const void* k_new,
                                             const void* v_new, int64_t new_stride_b, int64_t new_stride_h,
                                             const void* q, int32_t n_q_heads, float scale, void* out,
                                             int32_t out_dtype, void* workspace, size_t workspace_bytes,
                                             int32_t n_splits, uint32_t* dev_status, hipStream_t stream) {
  if (cache != nullptr && cache->batch > 0 && cache->max_len <= 0) return KVC_ERR_SHAPE;
  if (cache != nullptr && cache->batch > 0 && (k_new == nullptr || v_new == nullptr)) return KVC_ERR_NULL;
  return launch_decode(cache, seq_lens, 1, k_new, v_new, new_stride_b, new_stride_h, q, n_q_heads, scale, out,
                       out_dtype, workspace, workspace_bytes, n_splits, dev_status, stream, 0, nullptr, true);
}

// -------------------------------------------------------- quantised cache --

extern "C" kvc_status_t kvc_quant_append(const kvc_qcache_t* cache, const int32_t* seq_lens, const void* k_new,
                                         const void* v_new, int64_t new_stride_b, int64_t new_stride_h,
                                         uint32_t* dev_status, hipStream_t stream) {
  return launch_quant_rows(cache, seq_lens, k_new, v_new, new_stride_b, new_stride_h, 0, 1, dev_status, stream);
}

extern "C" kvc_status_t kvc_quant_prefill_fill(const kvc_qcache_t* cache, const int32_t* seq_lens, const void* k,
                                               const void* v, int64_t src_stride_b, int64_t src_stride_h,
                                               int64_t src_stride_t, int32_t t_new, uint32_t* dev_status,
                                               hipStream_t stream) {
  return launch_quant_rows(cache, seq_lens, k, v, src_stride_b, src_stride_h, src_stride_t, t_new, dev_status,
                           stream);
}

extern "C" kvc_status_t kvc_quant_decode_attn(const kvc_qcache_t* cache, const int32_t* seq_lens, int32_t n_pending,
                                              const void* q, int32_t n_q_heads, float scale, void* out,
                                              int32_t out_dtype, void* workspace, size_t workspace_bytes,
                                              int32_t n_splits, uint32_t* dev_status, hipStream_t stream) {
  return launch_quant_decode(cache, seq_lens, n_pending, q, n_q_heads, scale, out, out_dtype, workspace,
                             workspace_bytes, n_splits, dev_status, stream);
}

extern "C" kvc_status_t kvc_quant_decode_step(const kvc_qcache_t* cache, const int32_t* seq_lens, const void* k_new,
                                              const void* v_new, int64_t new_stride_b, int64_t new_stride_h,
                                              const void* q, int32_t n_q_heads, float scale, void* out,
                                              int32_t out_dtype, void* workspace, size_t workspace_bytes,
                                              int32_t n_splits, uint32_t* dev_status, hipStream_t stream) {
  if (cache != nullptr && cache->batch > 0 && (k_new == nullptr || v_new == nullptr)) return KVC_ERR_NULL;
  if (cache != nullptr && cache->batch > 0 && kvc::check_qcache(cache, true) == KVC_OK &&
      kvc::quant_routes_wide(cache, n_q_heads)) {
    // On the wide-group kernel: the append, then the attention (every host
    // check of both first), so the result is that of the two separate calls.
    if (new_stride_b < 0 || new_stride_h < 0) return KVC_ERR_SHAPE;
    if (cache->n_kv_heads > 1 && new_stride_h < cache->head_dim) return KVC_ERR_SHAPE;
    kvc_status_t st = launch_quant_decode(cache, seq_lens, 1, q, n_q_heads, scale, out, out_dtype, workspace,
                                          workspace_bytes, n_splits, dev_status, stream, nullptr, nullptr, 0, 0,
                                          true);
    if (st != KVC_OK) return st;
    st = launch_quant_rows(cache, seq_lens, k_new, v_new, new_stride_b, new_stride_h, 0, 1, dev_status, stream, true);
    if (st != KVC_OK) return st;
    st = launch_quant_rows(cache, seq_lens, k_new, v_new, new_stride_b, new_stride_h, 0, 1, dev_status, stream);
    if (st != KVC_OK) return st;
    return launch_quant_decode(cache, seq_lens, 1, q, n_q_heads, scale, out, out_dtype, workspace, workspace_bytes,
                               n_splits, dev_status, stream);
  }
  return launch_quant_decode(cache, seq_lens, 1, q, n_q_heads, scale, out, out_dtype, workspace, workspace_bytes,
                             n_splits, dev_status, stream, k_new, v_new, new_stride_b, new_stride_h);
}
