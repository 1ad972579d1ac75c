// Device helpers shared by the matrix-core attention kernels (prefill and
// wide-group decode): 16-bit element traits for v_mfma_f32_16x16x32 and the
// split of fp32 weights into two 16-bit parts, buffer resources, and the key
// order of a transposed-V row in LDS. Device code only; include inside an
// anonymous namespace of a .hip file.
#ifndef KVC_TILE_H_
#define KVC_TILE_H_

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// 16-bit cache element types: the matrix-core product, the split of two
// fp32 weights into high and low 16-bit parts (packed two to a word, first
// weight in the low half), and the output store.
struct Bf16P {
  __device__ static inline f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  }
  // hi keeps the top 16 bits of each weight (a bf16 value), lo the top 16
  // bits of the exact remainder: hi + lo carries 16 of the 24 bits. (The
  // byte permute takes bytes 2-3 of each word: 0x07060302 over {p1, p0}.)
  __device__ static inline void split(float p0, float p1, uint32_t& hi, uint32_t& lo) {
    const uint32_t u0 = __float_as_uint(p0), u1 = __float_as_uint(p1);
    const float r0 = p0 - __uint_as_float(u0 & 0xffff0000u);
    const float r1 = p1 - __uint_as_float(u1 & 0xffff0000u);
    hi = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
    lo = __builtin_amdgcn_perm(__float_as_uint(r1), __float_as_uint(r0), 0x07060302u);
  }
  // fp32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN
  __device__ static inline uint16_t bits(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
  }
  __device__ static inline void store(void* base, int64_t i, float x) { static_cast<uint16_t*>(base)[i] = bits(x); }
};

struct F16P {
  __device__ static inline f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c,
                                                  0, 0, 0);
  }
  // hi = fp16(p) rounded toward zero, lo = fp16(p - hi) likewise; the
  // remainder is exact in fp32 (one packed conversion per pair)
  __device__ static inline void split(float p0, float p1, uint32_t& hi, uint32_t& lo) {
    const half2_t h = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(p0, p1));
    const float r0 = p0 - static_cast<float>(h[0]), r1 = p1 - static_cast<float>(h[1]);
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(r0, r1));
  }
  // fp32 -> fp16 bits, round to nearest even (the fp32 value is pinned
  // first, so the conversion is one rounding of it)
  __device__ static inline uint16_t bits(float x) {
    asm volatile("" : "+v"(x));
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
  __device__ static inline void store(void* base, int64_t i, float x) { static_cast<uint16_t*>(base)[i] = bits(x); }
};

// Buffer resource over [base, base + bytes): loads past the end return zero.
__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ inline u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0));
}
// The slot of key kk (0..31) of a 32-key chunk in a transposed-V row. The
// score product leaves lane group g (lanes 16g .. 16g+15) with keys 4g..4g+3
// of each 16-key block; the output product takes 8 consecutive slots per
// lane group, so slots 8g..8g+7 hold keys 4g..4g+3 and 16+4g..16+4g+3.
__device__ inline int vt_slot(int kk) { return 8 * ((kk & 15) >> 2) + (kk & 3) + 4 * (kk >> 4); }


// K and V tiles in LDS (the prefill and wide-group kernels) sit as stored
// (row-major, no padding), with the 16-byte chunks of row r permuted by
// chunk ^ tile_swz(r): the score product's K
// reads (8 consecutive rows at one chunk) and the output product's
// transposing V reads (4 consecutive rows, two chunks each) then fall on
// distinct banks.
__device__ inline int tile_swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Four 16-bit elements of column d0 + i from four consecutive rows, into
// lane i of each 16-lane group (ds_read_b64_tr_b16): lane s of the group
// points at elements d0 + 4 (s % 4) .. + 3 of row s / 4.
__device__ inline u32x2 lds_read_tr(const char* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                       (__attribute__((address_space(3))) i16x4*)(const_cast<char*>(p))));
}

// Buffer descriptor words (base, 16-bit stride 0, byte range, raw format) in
// scalar registers, for the LDS loads below.
__device__ inline u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a))),
               static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32) & 0xffffu)),
               static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(bytes)), 0x00020000u};
}

// The LDS address of a __shared__ array (for M0 below).
#define KVC_LDS_ADDR(arr) \
  static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)(arr)))

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes at
// voff land at LDS address lds + 16 l (buffer_load_dwordx4 ... lds, the
// address in M0); offsets past the range write zeros. Written as inline assembly so
// that the compiler does not take later LDS reads of other buffers for
// reads of this load's destination and wait for every load in flight
// before them; the caller waits (s_waitcnt vmcnt) before reading the data.
// kNt: the non-temporal hint (rows read once).
template <bool kNt>
__device__ inline void lds_load16(const u32x4& rs, uint32_t voff, uint32_t lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  if constexpr (kNt)
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(rs), "s"(m0)
                 : "memory");
  else
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "s"(m0)
                 : "memory");
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// the wave are outstanding (the other counters left alone)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

#endif  // KVC_TILE_H_
