// Decode attention for wide groups: many query heads per KV head (MQA, wide
// GQA) or, for a block of new queries, many (query, head) pairs per KV head,
// on the CDNA4 matrix cores, with each KV head's K/V streamed from HBM once
// for all of them.
//
// Grouping query heads onto fewer KV heads saves cache bytes, not FLOPs
// (course notes "第 1 周 · Day 4" §2.2 and §2.5), and the saving only reaches
// the decode step if the shared K/V rows are read once for the whole group,
// through the head map rather than by copying heads (glossary "KV 缓存",
// "从教学代码到生产实现还差什么"). With 64 query heads on one KV head a
// decode step does 64 FLOPs per cache byte, past what the vector ALU
// sustains at HBM rate, so both products run on v_mfma_f32_16x16x32:
//   * one 512-thread workgroup (8 waves) per (sequence, KV head, split of
//     the T axis); the split's K/V rows go from memory straight into LDS
//     (buffer loads with the LDS destination) in tiles of 64 keys, as stored
//     with the 16-byte chunks of each row permuted, through a ring of four
//     tile buffers, so three tiles are in flight while one is computed;
//   * each wave owns column blocks of 16 (query, head) pairs and half of each
//     tile's keys; scores are computed transposed, S^T = K Q^T, so a lane
//     holds the scores of one pair and the online softmax (a lazily moved
//     reference, as in the other decode kernel) stays in its registers;
//   * the output is accumulated transposed, O^T += V^T P^T, V^T read from the
//     row-major tile with the transposing LDS reads; each fp32 weight is
//     split into two 16-bit parts (hi + lo, about 16 significant bits) so the
//     product keeps the weights' precision; accumulation fp32;
//   * the newest attended row is folded in by the last split as a tile of its
//     own (from k_new/v_new in the fused step, which also writes it into the
//     cache), so kvc_decode_step and kvc_append + kvc_decode_attn add the same
//     rows in the same order;
//   * splits publish (reference, sum, unnormalised output) per pair; 3 to 32
//     splits share the merge (each split merges a slice of the unit's pairs
//     once all have published, the last to arrive takes what no split
//     claimed), 2 or more than 32 splits merge in the last split, in split
//     order either way; every split of a unit runs on one XCD.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "kvc.h"
#include "kvc_internal.h"

namespace {

#include "kvc_tile.h"

constexpr int kWTile = 64;       // keys per LDS tile
constexpr int kXchgW = KVC_XCHG_POLICY;
// Split counts for which the merge is spread over the splits (at two, the
// last split's merge with ready flags measured 2 % faster)
constexpr int kSpreadMin = 3;
constexpr int kSpreadMax = kvc::kWideSpreadMax;
static_assert(kSpreadMax <= 32, "one lane of a wave per slice, claims in 32 bits");
// Scope of the spread merge's atomics: a unit's splits share one XCD's L2
// (workgroup placement), where atomics are performed; otherwise the device.
constexpr int kSyncScope =
    (KVC_XCD_COLOCATE && KVC_LOCAL_EXCHANGE) ? __HIP_MEMORY_SCOPE_WORKGROUP : __HIP_MEMORY_SCOPE_AGENT;

// The 8-bit mode (KQ = 1: OCP E4M3 codes, KQ = 2: int8 codes, each with one
// fp32 scale per token and KV head). Every code's value has at most 8
// significant bits, so widening it to the queries' 16-bit type is exact; the
// scales are applied to the scores (K) and to the weights in the weighted
// sum (V), in fp32.
constexpr int kWQFp8 = 1;
constexpr int kWQInt8 = 2;
// Codes in bytes 2 HI, 2 HI + 1 of w as two packed 16-bit values.
template <int KQ, bool kF16, bool HI>
__device__ inline uint32_t wcode_pair16(uint32_t w) {
  float a, b;
  if constexpr (KQ == kWQFp8) {
    const auto f = __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
    a = f[0];
    b = f[1];
  } else {
    a = static_cast<float>(static_cast<int32_t>(w << (HI ? 8 : 24)) >> 24);
    b = static_cast<float>(static_cast<int32_t>(w << (HI ? 0 : 16)) >> 24);
  }
  if constexpr (kF16) return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
  else return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);   // bf16: the exact high half
}
// Eight codes as one 16-byte chunk of eight 16-bit values, in order.
template <int KQ, bool kF16>
__device__ inline u32x4 wcodes8(u32x2 c) {
  return u32x4{wcode_pair16<KQ, kF16, false>(c[0]), wcode_pair16<KQ, kF16, true>(c[0]),
               wcode_pair16<KQ, kF16, false>(c[1]), wcode_pair16<KQ, kF16, true>(c[1])};
}

#ifndef KVC_WIDE_BUFFERS
#define KVC_WIDE_BUFFERS 4       // LDS tile buffers: the tiles in flight behind the one computed, plus it
#endif

struct WideParams {
  char* k;                       // cache; written only by the fused append
  char* v;
  int64_t sb, sh, st;            // cache strides in bytes
  const int32_t* seq_lens;
  const char* q;                 // [B, t_q, H_q, D] (decode: t_q = 1)
  const char* k_new;             // fused append source [B, H_kv, D] (a block: [B, H_kv, t_q, D]) or null
  const char* v_new;
  int64_t nsb, nsh, nst;         // its strides in bytes (nst: between a block's rows)
  uint32_t* ws_flag;             // [B * H_kv * n_hblk, flag_stride]: pair block pb uses head block pb's row
  uint32_t* ws_sync;             // [B * H_kv * n_pb, kWideSyncWords]: arrival count and slice claims of the spread merge
  float* ws_o;                   // per unit and pair block [S][D / 16][its pairs][16]: see pofs in the kernel
  float* ws_ml;                  // [B, H_kv * pairs, S, 2]
  void* out;                     // like q; fp32 or the cache dtype
  uint32_t* status;
  int32_t batch, n_q, n_kv, group, n_hblk, max_len, n_pending, n_splits, out_f32;
  int32_t n_pb;                  // pair blocks per unit (kWidePairBlock pairs each, the last the rest)
  int32_t t_q, block;            // block of t_q queries (lower-right causal mask), or decode (block = 0)
  int32_t out_vec;               // out is 16-byte aligned: four elements per store
  float scale_log2;              // softmax scale * log2(e)
  int32_t merge_spins;           // bound on the merge's wait for ready flags (polls)
  int32_t flag_stride;           // words per flag row (>= n_splits); the last is the epoch
  int32_t* lens_next;            // kvc_decode_step_advance: seq_lens[b] + 1 written here, or null
  const int32_t* table;          // paged mode: page table [B, table_stride] (slot r: page table[b][r >> page_shift])
  int32_t table_stride, page_shift, n_pages;
  const char* k_scale;           // the 8-bit mode: fp32 scales [B, H_kv, T] (token axis contiguous)
  const char* v_scale;
  int64_t ssb, ssh;              // their strides in bytes
};

__device__ inline __amdgpu_buffer_rsrc_t wrsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
template <int kPolicy>
__device__ inline u32x4 wload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, kPolicy));
}
__device__ inline void wstore(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, x), r,
                                         static_cast<int>(off), 0, kXchgW);
}
// Values every lane holds alike, in scalar registers (for buffer resources).
__device__ inline const char* uniform_cptr(const char* q) {
  const uint64_t a = reinterpret_cast<uint64_t>(q);
  const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a)));
  const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32)));
  return reinterpret_cast<const char*>(lo | (hi << 32));
}

// Row of q and out ([B, t_q, H_q, D], token-major) of pair v of KV head g:
// pair v is query v / group of head v % group.
__device__ inline int64_t wpair_row(const WideParams& p, int b, int g, int v) {
  const int i = v / p.group;
  return (static_cast<int64_t>(b) * p.t_q + i) * p.n_q + g * p.group + (v - i * p.group);
}

// ET: Bf16P or F16P (the cache dtype); QB: column blocks of 16 pairs per wave.
//
// Eight waves: wave w takes column blocks (w % 4) + 4j and the half w / 4 of
// every 64-key tile (keys 32 kh .. 32 kh + 31), so two waves of a SIMD work
// side by side on each tile and hide each other's LDS and matrix-core
// latency. The two halves' softmax states are merged through LDS at the end,
// each wave keeping half of the head dim; the split merge then runs on all
// eight waves, each over its (column block, half of D).
// AM: the cache's addressing. 0: contiguous; 1: paged (k and v are page
// pools, sb the page stride; decode only); 2: ring (a sliding window of
// max_len slots, token i in slot i mod max_len; decode only).
template <typename ET, int D, int QB, int KQ = 0, int AM = 0>
__global__ __launch_bounds__(512, 1) void wide_decode_kernel(const WideParams p) {
  constexpr bool kQuant = KQ != 0;       // 8-bit codes and scales (k and v hold codes, one byte each)
  constexpr bool kPaged = AM == 1;
  constexpr bool kRing = AM == 2;
  static_assert(!kQuant || AM == 0, "the 8-bit mode is contiguous");
  constexpr bool kF16 = std::is_same<ET, F16P>::value;
  constexpr int NT = 512;               // threads per workgroup
  constexpr int NC = D / 32;            // 32-element slices of a row (score product depth)
  constexpr int ND = D / 16;            // 16-element output blocks
  constexpr int NDH = ND / 2;           // output blocks of a wave after the halves merge
  constexpr int RB = 2 * D;             // bytes per K or V row in LDS
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int TB = kWTile * RB;       // one K or one V tile
  constexpr int NL = kWTile * CPR / NT;   // 16-byte loads per thread per tile, K and V each
  constexpr int NBUF = KVC_WIDE_BUFFERS;
  // vector-memory loads every wave issues per tile (in the 8-bit mode waves 0
  // and 1 issue one more, the scales: their waits below are then stricter
  // than they need be)
  constexpr int kLoadsPerTile = kQuant ? (D == 128 ? 2 : 1) : 2 * NL;
  constexpr float kLazy = 8.f;          // the reference moves only past ref + 8 (log2 domain)
  // Reference of a pair that has seen no key: finite, so that exp2 of a
  // masked (-inf) score against it is 0 rather than NaN, and far below any
  // score, so the first key seen replaces it (and zeroes its weight).
  constexpr float kEmpty = -1e30f;
  static_assert(D == 64 || D == 128, "head dim 64 or 128");
  static_assert(NL >= 1 && NL * NT == kWTile * CPR && NBUF >= 2, "tile loads");
  constexpr int NDH_ = D / 32;
  // LDS: NBUF tile buffers (a K tile and a V tile each) during the stream,
  // NBUF - 1 of them filling while one is computed; at the end the halves
  // each wave passes its partner ([8 waves][QB][NDH][64 lanes] f32x4) and
  // the references and sums ([8 waves][QB][64 lanes][2]).
  // The 8-bit mode stages the codes instead: NBUF buffers of a K and a V
  // code tile (rows of D bytes, in order) and their K and V scales, and one
  // more K/V tile, the current tile's codes widened, which the products
  // read as they read a 16-bit tile.
  constexpr int kCodeBytes = kWTile * D;                 // one K or V code tile
  constexpr int kScaleBytes = kWTile * 4;                // one tile's K or V scales
  constexpr int kBufBytes = kQuant ? 2 * kCodeBytes + 2 * kScaleBytes : 2 * TB;
  constexpr int kCvt = NBUF * kBufBytes;                 // the widened tile (8-bit mode)
  constexpr int kStreamBytes = kQuant ? kCvt + 2 * TB : NBUF * kBufBytes;
  constexpr int kXoBytes = 8 * QB * NDH_ * 64 * 16;
  constexpr int kXmlBytes = 8 * QB * 64 * 8;
  constexpr int kLds = kStreamBytes > kXoBytes + kXmlBytes ? kStreamBytes : kXoBytes + kXmlBytes;
  __shared__ __attribute__((aligned(16))) char smem[kLds];

  // Workgroup placement: every split of a unit on one XCD (id residue mod 8),
  // the unit's splits in consecutive slots there, the merging split last;
  // the splits of the unit's pair blocks one block after the other.
  const int xcd = blockIdx.x & 7;
  const int r8 = blockIdx.x >> 3;
  const int split = r8 % p.n_splits;
  const int w8 = r8 / p.n_splits;
  const int pb = w8 % p.n_pb;
  const int unit = (w8 / p.n_pb) * 8 + xcd;
  if (unit >= p.batch * p.n_kv) return;              // grid padding
  const int b = unit / p.n_kv;
  const int g = unit - b * p.n_kv;
  // the unit's epoch (see the merge below), requested behind the first
  // tiles' loads and used at the end: the last word of the unit's flag row
  // for the last-split merge, the last word of its merge-word row for the
  // spread merge, each in the row whose words it is compared with
  uint32_t* const flags = p.ws_flag + (static_cast<int64_t>(unit) * p.n_hblk + pb) * p.flag_stride;
  uint32_t* const sync = p.ws_sync + (static_cast<int64_t>(unit) * p.n_pb + pb) * kvc::kWideSyncWords;
  uint32_t* const sync_epoch = sync + (kvc::kWideSyncWords - 1);
  uint32_t epoch = 0u;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cbw = wave & 3;                          // first column block of this wave
  const int kh = wave >> 2;                          // which half of each tile's keys
  const int r16 = lane & 15;
  const int grp = lane >> 4;
  // (query, head) pairs v0 .. v0 + gv - 1 of this KV head's group * t_q;
  // below, v is a pair's index within the block, v0 + v its index in the unit
  const int v0 = pb * kvc::kWidePairBlock;
  const int gv = min(p.group * p.t_q - v0, kvc::kWidePairBlock);
  const int ncb = (gv + 15) / 16;

  // The wave's pairs as B operands of the score product (column = pair r16
  // of column block cbw + 4j, 8 elements 32c + 8grp of its query row),
  // requested first: they do not depend on the sequence's length, so their
  // round trip overlaps the length's. The rows of a unit's pairs lie within
  // t_q * H_q rows of its first one; a lane with no pair reads past the
  // range (zeros).
  const char* const qunit = uniform_cptr(p.q + ((static_cast<int64_t>(b) * p.t_q) * p.n_q + g * p.group) * D * 2);
  const __amdgpu_buffer_rsrc_t qrs = wrsrc(qunit, static_cast<uint32_t>(p.t_q * p.n_q * D * 2));
  u32x4 qf[QB][NC];
  bool cb_on[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const int cb = cbw + 4 * j;
    cb_on[j] = cb < ncb;
    const int v = cb * 16 + r16;
    const int qi = (v0 + v) / p.group;
    const uint32_t qoff = cb_on[j] && v < gv
                              ? static_cast<uint32_t>(((qi * p.n_q + (v0 + v - qi * p.group)) * D + 8 * grp) * 2)
                              : 0x80000000u;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) qf[j][cc] = wload<0>(qrs, qoff + 64u * cc);
  }

  // Rows attended (n), the slot the fused append writes, device-side flags.
  const int c0 = p.seq_lens[b];
  // kvc_decode_step_advance: the next step's lengths, into another array
  if (p.lens_next != nullptr && g == 0 && split == 0 && pb == 0 && threadIdx.x == 0) p.lens_next[b] = c0 + 1;
  const int c = c0 < 0 ? 0 : c0;
  uint32_t dflags = c0 < 0 ? KVC_DEVERR_BADLEN : 0u;
  const int add = p.block ? p.t_q : (p.k_new != nullptr ? 1 : p.n_pending);
  const int64_t n64 = static_cast<int64_t>(c) + add;
  int n, append_row = -1, newest = -1;
  if constexpr (kRing) {                             // no capacity limit: the ring wraps
    if (c0 >= 0 && p.k_new != nullptr) append_row = c0 % p.max_len;
    n = c0 < 0 ? 0 : static_cast<int>(min(n64, static_cast<int64_t>(p.max_len)));
    newest = c0 < 0 ? -1 : static_cast<int>((n64 - 1) % p.max_len);
  } else if (p.block) {                              // the whole block must fit
    if (c0 >= 0 && n64 > p.max_len) dflags |= KVC_DEVERR_CAPACITY;
    n = (c0 < 0 || n64 > p.max_len) ? 0 : static_cast<int>(n64);
    if (p.k_new != nullptr && n > 0) append_row = c0;   // the fused fill writes slots c0 .. c0 + t_q - 1
  } else {
    if (p.k_new != nullptr) {
      if (c0 >= 0 && c0 < p.max_len) append_row = c0;
      else dflags |= KVC_DEVERR_CAPACITY;
    }
    n = static_cast<int>(min(n64, static_cast<int64_t>(p.max_len)));
    if (n64 > p.max_len) dflags |= KVC_DEVERR_CAPACITY;
    if (c0 < 0) n = 0;             // a negative length: a zero row, nothing attended
  }
  if (dflags != 0 && g == 0 && split == 0 && pb == 0 && threadIdx.x == 0 && p.status != nullptr)
    atomicOr(p.status, dflags);
  auto store_out = [&](int64_t idx, float x) {
    if (p.out_f32) static_cast<float*>(p.out)[idx] = x;
    else ET::store(p.out, idx, x);
  };
  if (n <= 0) {                                      // empty sequence: zero rows
    if (split == 0)
      for (int t = threadIdx.x; t < gv * D; t += blockDim.x)
        store_out(wpair_row(p, b, g, v0 + t / D) * D + t % D, 0.f);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // (the query loads)
    return;
  }
  // The T axis in equal whole tiles. The newest rows -- the newest one in
  // decode, the block's own t_q rows for a block -- are folded in apart from
  // the stream, as one more tile, by the last active split: then a fused
  // append (or fill), whose rows come from k_new/v_new, and the separate
  // calls, which read them from the cache, add the same rows in the same
  // order.
  // (Ring: the newest row's slot can be anywhere in [0, n); every slot is
  // streamed and that one masked in the stream, the order of keys being
  // immaterial to the result.)
  const int xrows = p.block ? p.t_q : 1;
  const int streamed = kRing ? n : n - xrows;
  const int chunk = max(kWTile, ((streamed + p.n_splits - 1) / p.n_splits + kWTile - 1) & ~(kWTile - 1));
  const int ns = streamed > 0 ? min(p.n_splits, (streamed + chunk - 1) / chunk) : 1;
  if (split >= ns) {                                 // inactive split
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // (the query loads)
    return;
  }
  const bool spread = ns >= kSpreadMin && ns <= kSpreadMax;   // how the splits merge (below)
  const int t0 = split * chunk;
  const int t_end = split == ns - 1 ? streamed : t0 + chunk;   // rows streamed from the cache: [t0, t_end)
  const bool has_x = split == ns - 1;
  const int xfirst = kRing ? newest : n - xrows;     // the first folded row
  const int skip = kRing ? newest : -1;              // a slot the stream masks
  const bool x_new = has_x && append_row == xfirst;

  // The fused append (or fill): the newest rows into their slots (no
  // workgroup of this launch reads those slots from the cache). Their loads
  // are issued first and their stores after the stream, so that waiting for
  // them holds nothing else back: thread tid takes 16-byte chunk tid % CPR of
  // row tid / CPR (the host keeps xrows * CPR within the workgroup). Every
  // thread runs them: those with nothing to copy see an empty buffer range
  // (loads read zero, stores are dropped), as a load under a branch would
  // make the compiler wait for every load issued before it.
  const int64_t nst = p.block ? p.nst : static_cast<int64_t>(D * 2);   // between the new rows
  const bool x_write = x_new && pb == 0;             // the first pair block writes the rows
  const uint32_t arange = x_write ? static_cast<uint32_t>((xrows - 1) * nst + D * 2) : 0u;
  const uint32_t aoff_new = static_cast<uint32_t>((tid / CPR) * nst + (tid % CPR) * 16);
  const int64_t nrow = b * p.nsb + g * p.nsh;
  const __amdgpu_buffer_rsrc_t kn_rs = wrsrc(uniform_cptr(p.k_new != nullptr ? p.k_new + nrow : p.k), arange);
  const __amdgpu_buffer_rsrc_t vn_rs = wrsrc(uniform_cptr(p.v_new != nullptr ? p.v_new + nrow : p.v), arange);
  const u32x4 kn_row = wload<0>(kn_rs, aoff_new);
  const u32x4 vn_row = wload<0>(vn_rs, aoff_new);

  // Each pair's slot limit (lower-right causal mask of a query block).
  int plim[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const int v = (cbw + 4 * j) * 16 + r16;
    plim[j] = p.block ? n - p.t_q + (v0 + v) / p.group + 1 : n;
  }

  const uint32_t st = static_cast<uint32_t>(p.st);
  const char* kunit = uniform_cptr(p.k + (b * p.sb + g * p.sh));
  const char* vunit = uniform_cptr(p.v + (b * p.sb + g * p.sh));
  // K/V of the streamed rows; rows past t_end read as zero (and are masked)
  const u32x4 krs = rsrc_words(kunit, static_cast<uint32_t>(t_end) * st);
  const u32x4 vrs = rsrc_words(vunit, static_cast<uint32_t>(t_end) * st);

  // Tiles go from memory straight to LDS (buffer loads to LDS: lane l of a
  // load writes the 16 bytes at the load's LDS base + 16 l), with no
  // registers or stores in between: load i of wave w fills chunk positions
  // 64 (NL w + i) + lane of the tile, i.e. row / chunk position
  // (q / CPR, q % CPR), from the row's chunk q % CPR ^ tile_swz(row). Rows
  // past the streamed ones read as zeros (and are masked).
  const uint32_t smem_lds = KVC_LDS_ADDR(smem);
  // Ring mode: row `hole` of the tile (the newest slot, folded in apart)
  // reads as zeros too, whatever the slot holds (a stale or not yet written
  // row: its weight is 0, and 0 times a non-finite value is not).
  auto load_tile_from = [&](const u32x4& kr_, const u32x4& vr_, uint32_t base, int buf, uint32_t rstride,
                            int hole) {
    const uint32_t kb = smem_lds + buf * kBufBytes;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int m = wave * NL + i;
      const int q = m * 64 + lane;
      const int row = q / CPR;
      uint32_t off =
          base + static_cast<uint32_t>(row) * rstride + static_cast<uint32_t>((q % CPR) ^ tile_swz(row)) * 16u;
      if constexpr (kRing) off = row == hole ? 0x80000000u : off;   // past every range (< 2^31 bytes)
      lds_load16<true>(kr_, off, kb + m * 1024);
      lds_load16<true>(vr_, off, kb + TB + m * 1024);
    }
  };
  // The 8-bit mode: code rows base .. (64 rows, rstride bytes apart, D
  // bytes each, in order) and their 64 K and 64 V scales (from byte sbase
  // of the scale resources) into staging buffer buf. D = 128: every thread
  // takes a K and a V chunk; D = 64: waves 0-3 the K chunks, 4-7 the V
  // chunks; lanes 0-15 of waves 0 and 1 the scales, four each. Rows past a
  // resource's range read as zeros.
  auto load_qtile_from = [&](const u32x4& kr_, const u32x4& vr_, const u32x4& ksr_, const u32x4& vsr_,
                             uint32_t base, uint32_t rstride, uint32_t sbase, int buf) {
    constexpr int CPQ = D / 16;                          // 16-byte chunks per code row
    const uint32_t sb0 = smem_lds + buf * kBufBytes;
    if constexpr (D == 128) {
      const int q = wave * 64 + lane;
      const uint32_t off = base + static_cast<uint32_t>(q / CPQ) * rstride + static_cast<uint32_t>(q % CPQ) * 16u;
      lds_load16<true>(kr_, off, sb0 + wave * 1024);
      lds_load16<true>(vr_, off, sb0 + kCodeBytes + wave * 1024);
    } else {
      const int q = (wave & 3) * 64 + lane;
      const uint32_t off = base + static_cast<uint32_t>(q / CPQ) * rstride + static_cast<uint32_t>(q % CPQ) * 16u;
      if (wave < 4) lds_load16<true>(kr_, off, sb0 + wave * 1024);
      else lds_load16<true>(vr_, off, sb0 + kCodeBytes + (wave - 4) * 1024);
    }
    if (wave < 2 && lane < 16)
      lds_load16<true>(wave == 0 ? ksr_ : vsr_, sbase + static_cast<uint32_t>(lane) * 16u,
                       sb0 + 2 * kCodeBytes + wave * kScaleBytes);
  };
  const char* ksunit = nullptr;
  const char* vsunit = nullptr;
  u32x4 ksrs = u32x4{0u, 0u, 0u, 0u}, vsrs = u32x4{0u, 0u, 0u, 0u};
  if constexpr (kQuant) {
    ksunit = uniform_cptr(p.k_scale + (b * p.ssb + g * p.ssh));
    vsunit = uniform_cptr(p.v_scale + (b * p.ssb + g * p.ssh));
    ksrs = rsrc_words(ksunit, static_cast<uint32_t>(t_end) * 4u);
    vsrs = rsrc_words(vsunit, static_cast<uint32_t>(t_end) * 4u);
  }
  // Paged mode: wave w loads rows 8w .. 8w + 7 of a tile (its NL loads of 64
  // chunks), which lie in one page (pages hold 16+ rows, tiles start on a
  // multiple of 64): one buffer resource per wave and tile. Lane j of pidv
  // holds that page for tile (t & ~63) + j, read 64 tiles at a time; a tile's
  // page is taken with readlane. A page outside the pool reads as zeros and
  // is reported.
  int pidv = -1, pid_block = -1;
  auto tile_page = [&](int t) {               // t: wave-uniform
    if ((t >> 6) != pid_block) {
      pid_block = t >> 6;
      const int row = t0 + ((pid_block << 6) + lane) * kWTile + 8 * wave;
      pidv = -1;
      if (row < t_end) pidv = p.table[static_cast<int64_t>(b) * p.table_stride + (row >> p.page_shift)];
    }
    return __builtin_amdgcn_readlane(pidv, t & 63);
  };
  auto load_tile_paged = [&](int t, int buf) {
    const int r0 = t0 + t * kWTile + 8 * wave;  // this wave's first row
    const int left = t_end - r0;
    const int pg = left > 0 ? tile_page(t) : 0;
    const bool bad = left > 0 && (pg < 0 || pg >= p.n_pages);
    if (bad && lane == 0 && p.status != nullptr) atomicOr(p.status, KVC_DEVERR_PAGE);
    const bool ok = left > 0 && !bad;
    const uint32_t range = ok ? static_cast<uint32_t>(min(left, 8)) * st : 0u;
    const int64_t boff =
        ok ? pg * p.sb + g * p.sh + static_cast<int64_t>(r0 & ((1 << p.page_shift) - 1)) * p.st : int64_t{0};
    const u32x4 kr = rsrc_words(p.k + boff, range);
    const u32x4 vr = rsrc_words(p.v + boff, range);
    const uint32_t kb = smem_lds + buf * kBufBytes;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int m = wave * NL + i;
      const int q = m * 64 + lane;
      const int row = q / CPR;                  // 8 wave .. 8 wave + 7
      const uint32_t off =
          static_cast<uint32_t>(row - 8 * wave) * st + static_cast<uint32_t>((q % CPR) ^ tile_swz(row)) * 16u;
      lds_load16<true>(kr, off, kb + m * 1024);
      lds_load16<true>(vr, off, kb + TB + m * 1024);
    }
  };
  // Byte offset of slot `row` of (sequence b, KV head g) in the cache or page
  // pool, or -1 when its page is not in the pool.
  auto slot_offset = [&](int row) -> int64_t {
    if constexpr (kPaged) {
      const int pg = p.table[static_cast<int64_t>(b) * p.table_stride + (row >> p.page_shift)];
      if (pg < 0 || pg >= p.n_pages) return -1;
      return pg * p.sb + g * p.sh + static_cast<int64_t>(row & ((1 << p.page_shift) - 1)) * p.st;
    } else {
      return b * p.sb + g * p.sh + static_cast<int64_t>(row) * p.st;
    }
  };
  auto load_tile = [&](int t, int buf) {
    if constexpr (kPaged)
      load_tile_paged(t, buf);
    else if constexpr (kQuant)
      load_qtile_from(krs, vrs, ksrs, vsrs, static_cast<uint32_t>(t0 + t * kWTile) * st, st,
                      static_cast<uint32_t>(t0 + t * kWTile) * 4u, buf);
    else
      load_tile_from(krs, vrs, static_cast<uint32_t>(t0 + t * kWTile) * st, buf, st, skip - (t0 + t * kWTile));
  };
  // The 8-bit mode: the codes of staging buffer buf widened into the tile the
  // products read (row r's chunk c at chunk position c ^ tile_swz(r), as the
  // 16-bit loads place them); eight threads per row.
  auto convert = [&](int buf) {
    const char* const src = smem + buf * kBufBytes;
    char* const dst = smem + kCvt;
    const int row = tid >> 3, part = tid & 7;
    const int sw = tile_swz(row);
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      const char* const cs = src + kv * kCodeBytes + row * D;
      char* const cd = dst + kv * TB + row * RB;
      if constexpr (D == 128) {              // sixteen codes: chunks 2 part and 2 part + 1
        const u32x4 c = *reinterpret_cast<const u32x4*>(cs + 16 * part);
        *reinterpret_cast<u32x4*>(cd + ((2 * part) ^ sw) * 16) = wcodes8<KQ, kF16>(u32x2{c[0], c[1]});
        *reinterpret_cast<u32x4*>(cd + ((2 * part + 1) ^ sw) * 16) = wcodes8<KQ, kF16>(u32x2{c[2], c[3]});
      } else {                               // eight codes: chunk part
        const u32x2 c = *reinterpret_cast<const u32x2*>(cs + 8 * part);
        *reinterpret_cast<u32x4*>(cd + (part ^ sw) * 16) = wcodes8<KQ, kF16>(c);
      }
    }
  };

  // Per pair: the reference r (log2 domain) the weights are taken against,
  // exp2(score - r). It moves only when a score passes r + 8, so weights stay
  // below 2^8 and the accumulators are rescaled only in those (rare) tiles.
  float mrun[QB], lrun[QB];                 // lrun: this lane's part of the pair's sum
  f32x4 o[QB][ND];                          // O^T: lane holds elements 16db + 4grp + i of pair r16
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    mrun[j] = kEmpty;
    lrun[j] = 0.f;
#pragma unroll
    for (int db = 0; db < ND; ++db) o[j][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float sc = p.scale_log2;

  // This wave's half of one staged tile whose first key is slot tb (keys
  // tb + 32 kh .. + 31); keys at or past lim, or past a pair's own limit,
  // get weight 0. One code path for every tile: the mask costs a compare and
  // a select per score, less than the register copies two paths would need.
  // Per-lane parts of the LDS addresses: K row r16 (+ 32 kh + 16 kk) has
  // its chunk 4 cc + grp at (4 cc + grp) ^ kswz; the transposing V reads
  // take keys 32 kh + 4 grp + r16 / 4 (and + 16), elements 16 db + 4 (r16 % 4)
  // .., i.e. chunk 2 db + (r16 % 4) / 2 at (2 db) ^ vx, byte 8 (r16 % 2).
  const int kswz = tile_swz(r16);
  const int vrow = 4 * grp + (r16 >> 2);
  const int vx = ((r16 & 3) >> 1) ^ tile_swz(vrow);
  const int voff = (32 * kh + vrow) * RB + 8 * (r16 & 1);
  auto compute = [&](int tb, int lim, int buf, int skp) {
    const char* const sk = kQuant ? smem + kCvt : smem + buf * kBufBytes;
    const char* const sv = sk + TB;
    // 8-bit mode: the scales of this lane's keys 32 kh + 16 kk + 4 grp + i
    f32x4 ksc[2], vsc[2];
    if constexpr (kQuant) {
      const float* const scl = reinterpret_cast<const float*>(smem + buf * kBufBytes + 2 * kCodeBytes);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        ksc[kk] = *reinterpret_cast<const f32x4*>(scl + 32 * kh + 16 * kk + 4 * grp);
        vsc[kk] = *reinterpret_cast<const f32x4*>(scl + kWTile + 32 * kh + 16 * kk + 4 * grp);
      }
    }
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      if (!cb_on[j]) continue;                // wave-uniform
      // Every LDS read of the tile is issued first (K rows for the scores,
      // transposed V for the output), so that their latency overlaps the
      // score products and the softmax instead of stalling each product.
      u32x4 ka[2][NC], va[ND];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int cc = 0; cc < NC; ++cc)
          ka[kk][cc] = *reinterpret_cast<const u32x4*>(sk + (32 * kh + 16 * kk + r16) * RB + ((4 * cc + grp) ^ kswz) * 16);
#pragma unroll
      for (int db = 0; db < ND; ++db) {       // V^T rows 16 db + r16, in the weights' key slots
        const char* const vp = sv + voff + ((2 * db) ^ vx) * 16;
        const u32x2 lo4 = lds_read_tr(vp), hi4 = lds_read_tr(vp + 16 * RB);
        va[db] = u32x4{lo4[0], lo4[1], hi4[0], hi4[1]};
      }
      f32x4 s[2];                             // S^T: lane holds keys 32kh + 16kk + 4grp + i of pair r16
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) s[kk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < NC; ++cc)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) s[kk] = ET::mfma(ka[kk][cc], qf[j][cc], s[kk]);
      if constexpr (kQuant) {                 // scores of the codes times the keys' scales
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[kk][i] *= ksc[kk][i];
      }
      // keys at or past lim, or past the pair's own limit, get weight 0: room
      // is how many keys from this lane's first one are still attended (64
      // or more in every tile but the last of a split and a block's tail)
      const int room = min(lim, plim[j]) - tb - (32 * kh + 4 * grp);
      const int hole = skp - tb - (32 * kh + 4 * grp);    // ring: the newest slot, folded in apart
      float mx = -INFINITY;                   // raw scores: the scale is positive
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (kRing) s[kk][i] = (16 * kk + i < room && 16 * kk + i != hole) ? s[kk][i] : -INFINITY;
          else s[kk][i] = 16 * kk + i < room ? s[kk][i] : -INFINITY;
          mx = fmaxf(mx, s[kk][i]);
        }
      if (__any(mx * sc > mrun[j] + kLazy)) {   // wave-uniform; the first tile always
        mx = fmaxf(mx, __shfl_xor(mx, 16));    // the pair's maximum over its four lanes
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float ms = mx * sc;
        const bool up = ms > mrun[j] + kLazy;   // the four lanes of a pair agree
        const float alpha = up ? __builtin_amdgcn_exp2f(mrun[j] - ms) : 1.f;   // 0 from the empty reference
        mrun[j] = up ? ms : mrun[j];
        lrun[j] *= alpha;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[j][db][i] *= alpha;
      }
      const float nr = -mrun[j];
      float e[8];                             // slots 8grp .. 8grp+7 of this wave's 32-key chunk
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        e[jj] = __builtin_amdgcn_exp2f(fmaf(s[jj >> 2][jj & 3], sc, nr));   // masked: 0
        lrun[j] += e[jj];
      }
      if constexpr (kQuant) {                 // the weights of the codes: times the values' scales
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) e[jj] *= vsc[jj >> 2][jj & 3];
      }
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) ET::split(e[2 * w], e[2 * w + 1], hi[w], lo[w]);
      const u32x4 phi = u32x4{hi[0], hi[1], hi[2], hi[3]};
      const u32x4 plo = u32x4{lo[0], lo[1], lo[2], lo[3]};
      // high parts of every block, then low parts: no product waits on the
      // one before it (each block still adds hi, then lo)
#pragma unroll
      for (int db = 0; db < ND; ++db) o[j][db] = ET::mfma(va[db], phi, o[j][db]);
#pragma unroll
      for (int db = 0; db < ND; ++db) o[j][db] = ET::mfma(va[db], plo, o[j][db]);
    }
  };

  // The stream: NBUF LDS buffers, NBUF - 1 tiles in flight while one is
  // computed. A step waits for this wave's loads of tile t (the later tiles'
  // loads may stay in flight), then the barrier: every wave's loads of tile t
  // have landed, and every wave is done with tile t - 1, whose buffer then
  // takes tile t + NBUF - 1. Every pass runs all NBUF steps, their loads
  // included (tiles past the last read zeros and are not computed): the wait
  // counts are fixed only if every step issues the same loads.
  const int n_tiles = (t_end - t0 + kWTile - 1) / kWTile;
  // The query registers, used here so that the compiler waits for their
  // loads once, before the tiles' loads: a wait it placed later would count
  // only the loads it knows of, not the tiles' (inline assembly), and so
  // wait for most of those too. The query loads left at the start of the
  // kernel, so this wait is normally over at once.
#pragma unroll
  for (int j = 0; j < QB; ++j)
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) asm volatile("" ::"v"(qf[j][cc]));
  // the unit's epoch (see the merge), requested ahead of the tiles, so the
  // first tile's wait covers it
  if (ns > 1)
    epoch = __hip_atomic_load(spread ? sync_epoch : flags + p.flag_stride - 1, __ATOMIC_RELAXED,
                              kSyncScope);
#pragma unroll
  for (int r = 0; r < NBUF - 1; ++r) load_tile(r, r);
  for (int it = 0; it < n_tiles; it += NBUF) {
#pragma unroll
    for (int r = 0; r < NBUF; ++r) {          // unrolled: buffers are compile-time
      const int t = it + r;
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((NBUF - 2) * kLoadsPerTile));
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      load_tile(t + NBUF - 1, (r + NBUF - 1) % NBUF);
      if (t < n_tiles) {                      // uniform
        if constexpr (kQuant) {               // the codes widened, then the products
          convert(r);
          __syncthreads();
        }
        compute(t0 + t * kWTile, t_end, r, skip);
      }
    }
  }
  // every load landed and every wave done with the buffers
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  if (has_x) {
    // The newest rows as keys 0 .. xrows - 1 of one more tile: from
    // k_new/v_new in the fused step, else from the cache; the other keys read
    // as zero (the range ends with the last row) and are masked.
    if constexpr (kQuant) {                   // (from the cache: the 8-bit mode has no fused append)
      const char* kx = kunit + static_cast<int64_t>(xfirst) * p.st;
      const char* vx_ = vunit + static_cast<int64_t>(xfirst) * p.st;
      const uint32_t xrange = static_cast<uint32_t>(xrows - 1) * st + D;
      const uint32_t srange = static_cast<uint32_t>(xrows) * 4u;
      load_qtile_from(rsrc_words(kx, xrange), rsrc_words(vx_, xrange), rsrc_words(ksunit + 4 * xfirst, srange),
                      rsrc_words(vsunit + 4 * xfirst, srange), 0u, st, 0u, 0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();
      convert(0);
      __syncthreads();
    } else {
      const char* kx = x_new ? p.k_new + (b * p.nsb + g * p.nsh) : kunit + static_cast<int64_t>(xfirst) * p.st;
      const char* vx_ = x_new ? p.v_new + (b * p.nsb + g * p.nsh) : vunit + static_cast<int64_t>(xfirst) * p.st;
      const uint32_t xstride = x_new ? static_cast<uint32_t>(nst) : st;
      uint32_t xrange = static_cast<uint32_t>(xrows - 1) * xstride + D * 2;
      if constexpr (kPaged) {                 // (decode: one row, in one page)
        if (!x_new) {
          const int64_t xo = slot_offset(xfirst);
          if (xo < 0) {                       // not in the pool: zeros, reported
            xrange = 0u;
            if (tid == 0 && p.status != nullptr) atomicOr(p.status, KVC_DEVERR_PAGE);
          }
          kx = p.k + (xo < 0 ? 0 : xo);
          vx_ = p.v + (xo < 0 ? 0 : xo);
        }
      }
      load_tile_from(rsrc_words(kx, xrange), rsrc_words(vx_, xrange), 0u, 0, xstride, -1);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();
    }
    compute(xfirst, xfirst + xrows, 0, -1);   // (its rows only: in a ring they need not be the last)
  }
  {
    // the fused append's stores (the rows' loads were issued at entry)
    int64_t aoff = static_cast<int64_t>(append_row < 0 ? 0 : append_row) * p.st;
    uint32_t crange = x_write ? static_cast<uint32_t>((xrows - 1) * st + D * 2) : 0u;
    const char* abase_k = kunit;
    const char* abase_v = vunit;
    if constexpr (kPaged) {                   // the new row's page (decode: one row)
      aoff = 0;
      if (x_write) {
        const int64_t so = slot_offset(append_row);
        if (so < 0) {                         // not in the pool: not written, reported
          crange = 0u;
          if (tid == 0 && p.status != nullptr) atomicOr(p.status, KVC_DEVERR_PAGE);
        }
        abase_k = p.k + (so < 0 ? 0 : so);
        abase_v = p.v + (so < 0 ? 0 : so);
      }
    }
    const __amdgpu_buffer_rsrc_t ka_rs = wrsrc(uniform_cptr(abase_k + aoff), crange);
    const __amdgpu_buffer_rsrc_t va_rs = wrsrc(uniform_cptr(abase_v + aoff), crange);
    const int coff = static_cast<int>((tid / CPR) * st + (tid % CPR) * 16);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, kn_row),
                                           ka_rs, coff, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, vn_row),
                                           va_rs, coff, 0, 0);
  }

  // Merge the two key halves of every column block: each wave of a pair
  // (w, w + 4) passes the other the half of the head dim it gives up (LDS,
  // reusing the tile buffers) with its reference and sum; both then hold the
  // merged state of their own half (wave kh keeps blocks NDH kh .. + NDH).
  __syncthreads();                            // every wave is done with the last tile
  float* const xo = reinterpret_cast<float*>(smem);               // [8 waves][QB][NDH][64 lanes][4]
  float* const xml = reinterpret_cast<float*>(smem + kXoBytes);   // [8 waves][QB][64 lanes][2]
  static_assert(NDH == NDH_, "half blocks");
#pragma unroll
  for (int j = 0; j < QB; ++j) {
#pragma unroll
    for (int h = 0; h < NDH; ++h) {          // the other wave's half (indices fixed at compile
      const f32x4 give = kh ? o[j][h] : o[j][NDH + h];   // time: the accumulators stay in registers)
      *reinterpret_cast<f32x4*>(&xo[(((wave * QB + j) * NDH + h) * 64 + lane) * 4]) = give;
    }
    xml[((wave * QB + j) * 64 + lane) * 2] = mrun[j];
    xml[((wave * QB + j) * 64 + lane) * 2 + 1] = lrun[j];
  }
  __syncthreads();
  const int partner = wave ^ 4;
  f32x4 oh[QB][NDH];                          // this wave's half, merged over both key halves
  float mh[QB], lh[QB];                       // merged reference; this lane's part of the sum
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const float m2 = xml[((partner * QB + j) * 64 + lane) * 2];
    const float l2 = xml[((partner * QB + j) * 64 + lane) * 2 + 1];
    const float mm = fmaxf(mrun[j], m2);
    const float c1 = __builtin_amdgcn_exp2f(mrun[j] - mm);   // 0 for an empty half (its reference kEmpty)
    const float c2 = __builtin_amdgcn_exp2f(m2 - mm);
    mh[j] = mm;
    lh[j] = lrun[j] * c1 + l2 * c2;
#pragma unroll
    for (int h = 0; h < NDH; ++h) {
      const f32x4 other = *reinterpret_cast<const f32x4*>(&xo[(((partner * QB + j) * NDH + h) * 64 + lane) * 4]);
      const f32x4 mine = kh ? o[j][NDH + h] : o[j][h];
#pragma unroll
      for (int i = 0; i < 4; ++i) oh[j][h][i] = mine[i] * c1 + other[i] * c2;
    }
  }
  // Totals per pair: the lane groups' sums.
  float lt[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    float l = lh[j];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    lt[j] = l;
  }
  // Four consecutive output elements from element idx: one 16-byte (fp32)
  // or 8-byte (cache dtype, rounded to nearest even) store when out is
  // 16-byte aligned.
  auto store4 = [&](int64_t idx, const f32x4& y) {
    if (p.out_vec && p.out_f32) {
      *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + idx) = y;
    } else if (p.out_vec) {
      const uint32_t w0 = static_cast<uint32_t>(ET::bits(y[0])) | (static_cast<uint32_t>(ET::bits(y[1])) << 16);
      const uint32_t w1 = static_cast<uint32_t>(ET::bits(y[2])) | (static_cast<uint32_t>(ET::bits(y[3])) << 16);
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + idx) = u32x2{w0, w1};
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) store_out(idx + i, y[i]);
    }
  };
  // A lane's four consecutive output elements per block go out in one store
  // (16 bytes of fp32, or 8 of the cache dtype rounded to nearest even)
  // when out is 16-byte aligned.
  auto write_out = [&](int j, const f32x4 (&acc)[NDH], float l) {
    const int v = (cbw + 4 * j) * 16 + r16;
    if (v >= gv) return;
    const float inv = 1.f / l;
    const int64_t row = wpair_row(p, b, g, v0 + v) * D;
#pragma unroll
    for (int h = 0; h < NDH; ++h) {
      const int64_t idx = row + 16 * (NDH * kh + h) + 4 * grp;
      f32x4 y;
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = acc[h][i] * inv;
      store4(idx, y);
    }
  };
  if (ns == 1) {
#pragma unroll
    for (int j = 0; j < QB; ++j)
      if (cb_on[j]) write_out(j, oh[j], lt[j]);
    return;
  }

  // Several splits: as in the other decode kernel, every split but the last
  // publishes its partial (reference, sum, unnormalised output) and raises
  // its ready flag to epoch + 1; the last waits for those flags, folds the
  // partials in split order (its own from registers), writes the output and
  // advances the unit's epoch. It has the highest workgroup id of its unit
  // on the XCD, and a publishing workgroup never waits, so every awaited
  // workgroup is dispatched and finishes; the wait is bounded all the same.
  // This pair block's exchange: gv * S * D partial output floats (in the
  // order pofs gives below) and (reference, sum) pairs [split][pair], the
  // unit's pair blocks one after the other.
  const int64_t ubase = static_cast<int64_t>(unit) * p.n_splits * (p.group * p.t_q) +
                        static_cast<int64_t>(p.n_splits) * v0;
  const __amdgpu_buffer_rsrc_t ors = wrsrc(p.ws_o + ubase * D, static_cast<uint32_t>(gv) * p.n_splits * D * 4u);
  const __amdgpu_buffer_rsrc_t mrs = wrsrc(p.ws_ml + ubase * 2, static_cast<uint32_t>(gv) * p.n_splits * 8u);
  const __amdgpu_buffer_rsrc_t frs = wrsrc(flags, static_cast<uint32_t>(p.flag_stride) * 4u);
  // first use of the epoch: its load (issued with the first tiles) is waited for here,
  // not in front of the stream
  asm volatile("" : "+v"(epoch));
  // Partial outputs of the unit in the registers' order: split k, output
  // block db (16 elements), pair v, 4-element group g4 at 16-byte word
  // ((k ND + db) gv + v) 4 + g4, so one store of a wave (16 pairs x 4
  // groups of one block) covers 1 KB of whole cache lines (a store of half a
  // line would have the cache fetch the other half from memory first).
  auto pofs = [&](int k, int db, int v, int g4) {
    return static_cast<uint32_t>((((k * ND + db) * gv + v) * 4 + g4) * 16);
  };
  // This split's partial into the exchange, complete in L2 when the function
  // returns.
  auto publish = [&]() {
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      const int v = (cbw + 4 * j) * 16 + r16;
      if (!cb_on[j] || v >= gv) continue;
      const uint32_t row = static_cast<uint32_t>(split * gv + v);
#pragma unroll
      for (int h = 0; h < NDH; ++h)
        wstore(ors, pofs(split, NDH * kh + h, v, grp),
               u32x4{__float_as_uint(oh[j][h][0]), __float_as_uint(oh[j][h][1]), __float_as_uint(oh[j][h][2]),
                     __float_as_uint(oh[j][h][3])});
      if (kh == 0 && grp == 0) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(mh[j]), mrs, static_cast<int>(row * 8u), 0, kXchgW);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lt[j]), mrs, static_cast<int>(row * 8u + 4u), 0, kXchgW);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };

  if (spread) {
    // The spread merge: every split publishes its partial and counts itself
    // in; the unit's output is cut into ns slices of (pair, 4 elements)
    // items, and split k merges slice k once all splits have arrived, so
    // the merge's reads and writes are shared by ns workgroups instead of
    // falling on one. A split waits for the others only for a bounded time;
    // the last to arrive waits for nothing and, after its own slice, merges
    // every slice no one has claimed (those of splits that gave up waiting).
    // Per (sequence, KV head), in one row of merge words: an arrival count,
    // which the last arrival returns to zero when it is done, one claim word
    // per slice, raised to epoch + 1 by the one workgroup that merges the
    // slice (an atomic maximum: each slice is written once), and the epoch
    // itself (the row's last word). The last arrival advances the epoch,
    // which also tells splits still waiting that the merge is done. A claim
    // is only ever raised to its own row's epoch + 1 and that epoch then
    // grows, so a claim left by an earlier call, of any geometry, is below
    // this call's value.
    publish();
    __syncthreads();
    uint32_t* const claims = sync + 1;
    __shared__ uint32_t ss[2];
    if (tid == 0) {
      const uint32_t ticket = __hip_atomic_fetch_add(sync, 1u, __ATOMIC_RELAXED, kSyncScope) + 1u;
      uint32_t state = ticket >= static_cast<uint32_t>(ns) ? 2u : 0u;   // 2: last, 1: all arrived, 0: gave up
      for (int spins = 0; state == 0u && spins < p.merge_spins; ++spins) {
        __builtin_amdgcn_s_sleep(1);
        // (exchanges that write back what they find: performed in L2)
        uint32_t c = static_cast<uint32_t>(ns), e = epoch;
        __hip_atomic_compare_exchange_strong(sync, &c, c, __ATOMIC_RELAXED, __ATOMIC_RELAXED, kSyncScope);
        __hip_atomic_compare_exchange_strong(sync_epoch, &e, e, __ATOMIC_RELAXED, __ATOMIC_RELAXED, kSyncScope);
        if (c >= static_cast<uint32_t>(ns)) state = 1u;
        else if (e != epoch) break;            // the merge is done: nothing left to claim
      }
      ss[0] = state;
    }
    __syncthreads();
    const uint32_t state = ss[0];
    // Slice k: items [k I / ns, (k + 1) I / ns) of the I = pairs * D / 4, each
    // a pair's 4 consecutive elements, in the exchange's order (block, pair,
    // group), so a wave's loads cover whole lines; the splits folded in split
    // order, as in the last-split merge. With claim,
    // the slice is claimed first, and the loads of each thread's first item
    // are issued while the claim's answer is on its way.
    auto merge_slice = [&](int k, bool claim) {
      constexpr int R = 8;
      const int items = gv * (D / 4);                  // item: (block db, pair v, group g4), the exchange's order
      const int i1 = (k + 1) * items / ns;
      uint32_t old = 0u;
      if (claim && tid == 0) old = __hip_atomic_fetch_max(claims + k, epoch + 1u, __ATOMIC_RELAXED, kSyncScope);
      u32x4 ob[R];
      u32x2 mlb[R];
      // one round: splits k0 .. k0 + R - 1 of item it (rows past the region,
      // or no item at all, read as zero)
      auto load_round = [&](int it, int k0) {
        const int db = it / (gv * 4), v = (it - db * gv * 4) >> 2, g4 = it & 3;
        const bool any = it < i1;
#pragma unroll
        for (int kk = 0; kk < R; ++kk) {
          const uint32_t row = static_cast<uint32_t>((k0 + kk) * gv + v);
          const uint32_t mo = any ? row * 8u : 0x80000000u;
          const uint32_t oo = any ? pofs(k0 + kk, db, v, g4) : 0x80000000u;
          mlb[kk] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(mrs, static_cast<int>(mo), 0, kXchgW));
          ob[kk] = wload<kXchgW>(ors, oo);
        }
      };
      int it = k * items / ns + tid;
      load_round(it, 0);
      if (claim) {
        if (tid == 0) ss[1] = old < epoch + 1u;
        __syncthreads();
        if (!ss[1]) return;                   // uniform: another workgroup merges this slice
      }
      for (bool pre = true; it < i1; it += NT, pre = false) {
        const int db = it / (gv * 4), v = (it - db * gv * 4) >> 2, g4 = it & 3;
        float mm = -INFINITY, ll = 0.f;
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int k0 = 0; k0 < ns; k0 += R) {
          if (!pre || k0 > 0) load_round(it, k0);
#pragma unroll
          for (int kk = 0; kk < R; ++kk) {
            if (k0 + kk >= ns) break;
            const float r_k = __uint_as_float(mlb[kk][0]), l_k = __uint_as_float(mlb[kk][1]);
            const float nm = fmaxf(mm, r_k);
            const float c1 = mm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mm - nm);
            const float c2 = __builtin_amdgcn_exp2f(r_k - nm);
            ll = ll * c1 + l_k * c2;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = acc[i] * c1 + __uint_as_float(ob[kk][i]) * c2;
            mm = nm;
          }
        }
        const float inv = 1.f / ll;
        f32x4 y;
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = acc[i] * inv;
        store4(wpair_row(p, b, g, v0 + v) * D + 16 * db + 4 * g4, y);
      }
    };
    if (state != 0u) merge_slice(split, true);
    if (state == 2u) {
      // every slice not yet claimed (normally none: the others claimed theirs
      // while this one merged its own), claimed at once, one lane per slice,
      // and merged here
      __syncthreads();
      if (wave == 0) {
        const bool won = lane < ns && lane != split &&
                         __hip_atomic_fetch_max(claims + lane, epoch + 1u, __ATOMIC_RELAXED, kSyncScope) < epoch + 1u;
        const uint64_t m = __ballot(won);
        if (lane == 0) ss[1] = static_cast<uint32_t>(m);
      }
      __syncthreads();
      const uint32_t won = ss[1];
      for (int k = 0; k < ns; ++k)
        if ((won >> k) & 1u) merge_slice(k, false);
      // the count back to zero for the next call, then the epoch advanced
      __syncthreads();
      if (tid == 0) {
        __hip_atomic_store(sync, 0u, __ATOMIC_RELAXED, kSyncScope);
        __hip_atomic_store(sync_epoch, epoch + 1u, __ATOMIC_RELAXED, kSyncScope);
      }
    }
    return;
  }

  // Two splits, or more than the claim mask holds: every split but the last
  // publishes its partial and raises its ready flag to epoch + 1; the last
  // waits for those flags, folds the partials in split order (its own from
  // registers), writes the output and advances the unit's epoch. It has the
  // highest workgroup id of its unit on the XCD, and a publishing workgroup
  // never waits, so every awaited workgroup is dispatched and finishes; the
  // wait is bounded all the same.
  if (split != ns - 1) {
    publish();
    __syncthreads();
    if (tid == 0) __builtin_amdgcn_raw_buffer_store_b32(epoch + 1u, frs, static_cast<int>(split * 4), 0, kXchgW);
    return;
  }
  for (int k = tid; k < ns - 1; k += blockDim.x) {
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
      const uint32_t f = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(frs, k * 4, 0, kXchgW));
#endif
      if (f == epoch + 1u) break;
      if (++spins > p.merge_spins) {           // never expected: flag the call, do not hang
        if (p.status != nullptr) atomicOr(p.status, KVC_DEVERR_SYNC);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      asm volatile("" ::: "memory");
    }
  }
  __syncthreads();
  // Fold the splits in split order, eight (four with two column blocks) per
  // round trip, all their loads in flight together: running reference mm,
  // sum ll and accumulators acc over this wave's (column block, half of the
  // head dim); this workgroup's own split (the last) from registers.
  constexpr int R = QB == 1 ? 8 : 4;
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const int v = (cbw + 4 * j) * 16 + r16;
    if (!cb_on[j]) continue;
    const uint32_t vrow = static_cast<uint32_t>(v < gv ? v : 0);
    float mm = -INFINITY, ll = 0.f;
    f32x4 acc[NDH];
#pragma unroll
    for (int h = 0; h < NDH; ++h) acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < ns; k0 += R) {
      float rb[R], lb[R];
      u32x4 ob[R][NDH];
#pragma unroll
      for (int kk = 0; kk < R; ++kk) {       // rows past the region read as zero
        const uint32_t row = static_cast<uint32_t>((k0 + kk) * gv) + vrow;   // past the region: zeros
        rb[kk] = __uint_as_float(static_cast<uint32_t>(
            __builtin_amdgcn_raw_buffer_load_b32(mrs, static_cast<int>(row * 8u), 0, kXchgW)));
        lb[kk] = __uint_as_float(static_cast<uint32_t>(
            __builtin_amdgcn_raw_buffer_load_b32(mrs, static_cast<int>(row * 8u + 4u), 0, kXchgW)));
#pragma unroll
        for (int h = 0; h < NDH; ++h) ob[kk][h] = wload<kXchgW>(ors, pofs(k0 + kk, NDH * kh + h, vrow, grp));
      }
#pragma unroll
      for (int kk = 0; kk < R; ++kk) {
        const int k = k0 + kk;
        if (k >= ns) break;                    // uniform
        float r_k = rb[kk], l_k = lb[kk];
        if (k == split) {                      // own split: from registers
          r_k = mh[j];
          l_k = lt[j];
#pragma unroll
          for (int h = 0; h < NDH; ++h)
            ob[kk][h] = u32x4{__float_as_uint(oh[j][h][0]), __float_as_uint(oh[j][h][1]),
                              __float_as_uint(oh[j][h][2]), __float_as_uint(oh[j][h][3])};
        }
        const float nm = fmaxf(mm, r_k);
        const float c1 = mm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mm - nm);
        const float c2 = __builtin_amdgcn_exp2f(r_k - nm);
        ll = ll * c1 + l_k * c2;
#pragma unroll
        for (int h = 0; h < NDH; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[h][i] = acc[h][i] * c1 + __uint_as_float(ob[kk][h][i]) * c2;
        mm = nm;
      }
    }
    write_out(j, acc, ll);
  }
  // the next call on this workspace waits for flags of epoch + 2
  __syncthreads();
  if (tid == 0)
    __builtin_amdgcn_raw_buffer_store_b32(epoch + 1u, frs, static_cast<int>((p.flag_stride - 1) * 4), 0, kXchgW);
}

typedef void (*WideKernel)(const WideParams);

template <typename ET, int D, int AM>
WideKernel pick_wide_qb(int qb) {
  return qb <= 1 ? wide_decode_kernel<ET, D, 1, 0, AM> : wide_decode_kernel<ET, D, 2, 0, AM>;
}

// am: the cache's addressing (0 contiguous, 1 paged, 2 ring)
template <typename ET, int D>
WideKernel pick_wide_am(int qb, int am) {
  if (am == 1) return pick_wide_qb<ET, D, 1>(qb);
  if (am == 2) return pick_wide_qb<ET, D, 2>(qb);
  return pick_wide_qb<ET, D, 0>(qb);
}

template <typename ET, int D, int KQ>
WideKernel pick_wide_qb_q(int qb) {
  return qb <= 1 ? wide_decode_kernel<ET, D, 1, KQ> : wide_decode_kernel<ET, D, 2, KQ>;
}

template <typename ET, int KQ>
WideKernel pick_wide_d_q(int32_t d, int qb) {
  if (d == 128) return pick_wide_qb_q<ET, 128, KQ>(qb);
  if (d == 64) return pick_wide_qb_q<ET, 64, KQ>(qb);
  return nullptr;
}

// The 8-bit mode: codes of this format widened to the queries' type.
WideKernel pick_wide_kernel_q(int32_t format, int32_t q_dtype, int32_t d, int qb) {
  if (format != KVC_QFMT_FP8_E4M3 && format != KVC_QFMT_INT8) return nullptr;
  const bool fp8 = format == KVC_QFMT_FP8_E4M3;
  if (q_dtype == KVC_BF16) return fp8 ? pick_wide_d_q<Bf16P, kWQFp8>(d, qb) : pick_wide_d_q<Bf16P, kWQInt8>(d, qb);
  if (q_dtype == KVC_F16) return fp8 ? pick_wide_d_q<F16P, kWQFp8>(d, qb) : pick_wide_d_q<F16P, kWQInt8>(d, qb);
  return nullptr;
}

WideKernel pick_wide_kernel(int32_t dtype, int32_t d, int qb, int am) {
  if (dtype == KVC_BF16 && d == 128) return pick_wide_am<Bf16P, 128>(qb, am);
  if (dtype == KVC_BF16 && d == 64) return pick_wide_am<Bf16P, 64>(qb, am);
  if (dtype == KVC_F16 && d == 128) return pick_wide_am<F16P, 128>(qb, am);
  if (dtype == KVC_F16 && d == 64) return pick_wide_am<F16P, 64>(qb, am);
  return nullptr;
}

}  // namespace

bool kvc::wide_supported(int32_t dtype, int32_t head_dim, int32_t pairs) {
  return (dtype == KVC_BF16 || dtype == KVC_F16) && (head_dim == 64 || head_dim == 128) &&
         pairs >= KVC_WIDE_MIN_PAIRS && pairs <= kvc::kWideMaxPairs;
}

kvc_status_t kvc::launch_wide(const kvc_cache_t* cache, const int32_t* seq_lens, int32_t n_pending,
                              const void* k_new, const void* v_new, int64_t new_stride_b, int64_t new_stride_h,
                              int64_t new_stride_t, const void* q, int32_t n_q_heads, int32_t t_q,
                              float scale_log2, void* out, int32_t out_dtype, const kvc::WsRegions& ws,
                              int32_t splits, int32_t* lens_next, uint32_t* dev_status, hipStream_t stream,
                              bool check_only, const kvc::WideQuant* quant, const kvc::PageInfo* pg, bool ring) {
  // (arguments validated by the caller)
  const int s = quant != nullptr ? 1 : kvc::elem_bytes(cache->dtype);   // 8-bit mode: strides in bytes
  const int32_t tq = t_q > 0 ? t_q : 1;
  const int32_t group = n_q_heads / cache->n_kv_heads;
  const int32_t pairs = group * tq;
  const int qb = (std::min(pairs, kvc::kWidePairBlock) + 63) / 64;   // column blocks of 64 pairs per workgroup
  const int am = pg != nullptr ? 1 : (ring ? 2 : 0);
  if (am != 0 && (t_q > 0 || quant != nullptr)) return KVC_ERR_UNSUPPORTED;   // paged and ring: decode, 16-bit
  WideKernel kern = quant != nullptr ? pick_wide_kernel_q(quant->format, quant->q_dtype, cache->head_dim, qb)
                                     : pick_wide_kernel(cache->dtype, cache->head_dim, qb, am);
  if (kern == nullptr || qb > 2 || pairs > kvc::kWideMaxPairs) return KVC_ERR_UNSUPPORTED;
  if (quant != nullptr && (t_q > 0 || k_new != nullptr || lens_next != nullptr)) return KVC_ERR_UNSUPPORTED;
  WideParams p;
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
  p.nst = new_stride_t * s;
  // a block's rows are folded in as one tile, each thread loading one chunk
  // of the rows a fused fill appends
  static_assert(kvc::kWideMaxBlock <= kWTile, "a block is one tile");
  if (t_q > 0 && (t_q > kvc::kWideMaxBlock || (k_new != nullptr && t_q * (cache->head_dim / 8) > 512)))
    return KVC_ERR_UNSUPPORTED;
  p.ws_flag = ws.flags;
  p.flag_stride = ws.flag_stride;
  p.ws_sync = ws.sync;
  p.ws_o = ws.o;
  p.ws_ml = ws.ml;
  p.lens_next = lens_next;
  p.table = pg != nullptr ? pg->table : nullptr;
  p.table_stride = pg != nullptr ? pg->table_stride : 0;
  p.page_shift = pg != nullptr ? pg->page_shift : 0;
  p.n_pages = pg != nullptr ? pg->n_pages : 0;
  p.k_scale = quant != nullptr ? reinterpret_cast<const char*>(quant->k_scale) : nullptr;
  p.v_scale = quant != nullptr ? reinterpret_cast<const char*>(quant->v_scale) : nullptr;
  p.ssb = quant != nullptr ? quant->scale_stride_b * 4 : 0;
  p.ssh = quant != nullptr ? quant->scale_stride_h * 4 : 0;
  p.out = out;
  p.status = dev_status;
  p.batch = cache->batch;
  p.n_q = n_q_heads;
  p.n_kv = cache->n_kv_heads;
  p.group = group;
  p.n_hblk = kvc::head_blocks(pairs);
  p.n_pb = kvc::wide_pair_blocks(pairs);
  if (p.n_pb > p.n_hblk) return KVC_ERR_UNSUPPORTED;    // (a flag row per pair block: never with 8+ pairs)
  p.max_len = cache->max_len;
  p.n_pending = n_pending;
  p.n_splits = splits;
  p.out_f32 = out_dtype == KVC_F32 ? 1 : 0;
  p.t_q = tq;
  p.block = t_q > 0 ? 1 : 0;
  p.out_vec = reinterpret_cast<uintptr_t>(out) % 16 == 0 ? 1 : 0;
  p.scale_log2 = scale_log2;
  p.merge_spins = kvc::merge_spin_limit();
  const int64_t units = static_cast<int64_t>(cache->batch) * cache->n_kv_heads;
  const int64_t wgs = (units + 7) / 8 * 8 * p.n_pb * splits;    // see the placement in the kernel
  if (wgs > 0x7fffffffll) return KVC_ERR_SHAPE;
  if (check_only) return KVC_OK;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(wgs)), dim3(512), 0, stream, p);
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}
