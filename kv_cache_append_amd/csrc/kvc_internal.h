// Host-side helpers shared by the C-ABI entry points (no device code here).
#ifndef KVC_INTERNAL_H_
#define KVC_INTERNAL_H_

#include <stddef.h>
#include <stdint.h>

#include "kvc.h"

// Decode split placement and exchange (device code): with
// KVC_XCD_COLOCATE every workgroup of a (sequence, KV head) unit takes a
// workgroup id with the same residue mod 8, so the dispatcher, which deals
// ids round-robin over the eight XCDs, places the unit's splits on one XCD.
// KVC_XCHG_POLICY is the buffer cache policy of the splits' exchange
// (partials and ready flags): 16, device scope (write-through, miss in the
// per-XCD L2). With KVC_LOCAL_EXCHANGE (splits on one XCD) the exchange
// stays in that XCD's L2 instead: plain stores (the CU's L1 writes through
// to L2), ready flags polled with L2 atomics (KVC_XCHG_L2_POLL), and plain
// loads of partials the merging CU has not read before in the launch.
#ifndef KVC_XCD_COLOCATE
#define KVC_XCD_COLOCATE 1
#endif
#ifndef KVC_LOCAL_EXCHANGE
#define KVC_LOCAL_EXCHANGE 1
#endif
#if KVC_XCD_COLOCATE && KVC_LOCAL_EXCHANGE
#define KVC_XCHG_POLICY 0
#define KVC_XCHG_L2_POLL 1
#else
#define KVC_XCHG_POLICY 16
#define KVC_XCHG_L2_POLL 0
#endif

namespace kvc {

// Bytes per stored element, 0 for an unknown dtype code.
int elem_bytes(int32_t dtype);

// Shape, dtype, pointer and stride checks common to every call on a cache.
// need_vec16: the caller's kernels use 16-byte loads on cache rows.
kvc_status_t check_cache(const kvc_cache_t* c, bool need_vec16);

// Largest power-of-two byte width (16, 8, 4 or 2, at least the element size)
// that divides every given byte offset/stride and pointer; used by the copy
// kernels to pick their vector width.
int copy_vector_bytes(const kvc_cache_t* c, const void* src_k, const void* src_v,
                      const int64_t* src_strides_bytes, int n_src_strides);

// Decode kernels are built for these head dims; head_dim * elem_bytes must be
// a multiple of 16 and at most 1024.
bool decode_head_dim_supported(int32_t head_dim, int32_t dtype);

// Query heads handled by one decode workgroup (1, 2, 4 or 8) and the number
// of such head blocks per KV head.
int heads_per_block(int32_t group);
int head_blocks(int32_t group);

// Sequence splits per (sequence, KV head, head block) when the caller passes
// 0. n_q_heads counts (query, head) pairs for a query block. With wide = true
// (a contiguous 16-bit cache the wide-group kernel serves) the count is that
// kernel's, which runs one workgroup per (sequence, KV head) and split.
int32_t auto_splits(const kvc_cache_t* c, int32_t n_q_heads, bool wide = false);
// Whether a contiguous decode of this cache and pair count runs on the
// wide-group kernel.
bool routes_wide(const kvc_cache_t* c, int32_t n_q_heads);
// Splits chosen from the sequences' lengths (host array of c->batch values)
// by modelling the launch; see kvc_decode_splits_for_lengths.
int32_t splits_for_lengths(const kvc_cache_t* c, int32_t n_q_heads, const int32_t* lens);

// Workspace: uint32 ready flags [B * H_kv * head_blocks, S] (word S - 1 of
// each row is that block's merge epoch), then the wide-group kernel's merge
// words [B * H_kv * pair blocks, kWideSyncWords] (uint32), then fp32 partial outputs [B, H_q, S, D],
// then fp32 (reference, sum) pairs [B, H_q, S, 2]; each region starts on a
// 256-byte boundary.
size_t workspace_bytes(const kvc_cache_t* c, int32_t n_q_heads, int32_t n_splits);

// Where a decode call's split exchange lives: ready flags (one row of
// flag_stride words per (sequence, KV head, head block); the row's last word
// is that block's merge epoch), partial outputs [B, H_kv * pairs, S, D] and
// partial (reference, sum) pairs [B, H_kv * pairs, S, 2]. A caller's
// workspace has rows of S words (workspace_regions); the library's own
// scratch (kvc_decode_step_noalloc) has rows of KVC_MAX_SPLITS words.
struct WsRegions {
  uint32_t* flags;
  int32_t flag_stride;
  uint32_t* sync;   // the wide-group kernel: kWideSyncWords per (sequence, KV head, pair block)
  float* o;
  float* ml;
};
// Per (sequence, KV head, pair block), for the wide-group kernel's spread
// merge (up to kWideSpreadMax splits): an arrival count (word 0), one claim
// word per output slice (words 1 ..) and the merge epoch (the last word), in
// a row of kWideSyncWords uint32.
constexpr int kWideSpreadMax = 32;
constexpr int kWideSyncWords = 64;
constexpr size_t kWideSyncBytes = kWideSyncWords * sizeof(uint32_t);
static_assert(1 + kWideSpreadMax < kWideSyncWords, "spread merge words");
WsRegions workspace_regions(const kvc_cache_t* c, int32_t n_q_heads, int32_t n_splits, void* ws);
// Lays out a decode call's exchange space once its split count is known.
typedef kvc_status_t (*RegionsFn)(const kvc_cache_t* c, int32_t n_q_heads, int32_t n_splits, WsRegions* out);
// kvc_decode_step with the exchange in space that regions_fn lays out
// instead of a caller's workspace (same validation, kernels and results).
kvc_status_t decode_step_in_regions(const kvc_cache_t* cache, const int32_t* seq_lens, const void* k_new,
                                    const void* v_new, int64_t new_stride_b, int64_t new_stride_h, const void* q,
                                    int32_t n_q_heads, float scale, void* out, int32_t out_dtype, int32_t n_splits,
                                    uint32_t* dev_status, hipStream_t stream, RegionsFn regions_fn);
size_t workspace_flag_offset(const kvc_cache_t* c, int32_t n_q_heads, int32_t n_splits);
size_t workspace_sync_offset(const kvc_cache_t* c, int32_t n_q_heads, int32_t n_splits);
size_t workspace_o_offset(const kvc_cache_t* c, int32_t n_q_heads, int32_t n_splits);
size_t workspace_ml_offset(const kvc_cache_t* c, int32_t n_q_heads, int32_t n_splits);

// A paged cache seen as a cache descriptor: the pools as k/v, the page
// stride in place of stride_b, capacity pages_per_seq * page_size as
// max_len; plus what the kernels need to walk the page table.
struct PageInfo {
  const int32_t* table;
  int32_t table_stride;
  int32_t page_shift;   // log2(page_size)
  int32_t n_pages;
};
// Checks the paged descriptor (decode: page_size >= 16) and fills `view` and
// `info`; same status codes as check_cache.
kvc_status_t paged_view(const kvc_paged_cache_t* pc, bool for_decode, kvc_cache_t* view, PageInfo* info);

// Checks a quantised cache descriptor. for_decode: the queries must be fp16
// or bf16 (the append and fill calls also take fp32 rows).
kvc_status_t check_qcache(const kvc_qcache_t* c, bool for_decode);
// The geometry of a quantised cache (batch, heads, max_len, head_dim) as a
// cache descriptor, for the split heuristic and the workspace layout only.
kvc_cache_t qcache_view(const kvc_qcache_t* c);

// The wide-group decode kernel (kvc_wide.hip): fp16/bf16 caches with head
// dim 64 or 128 and KVC_WIDE_MIN_PAIRS..kWideMaxPairs (query, head) pairs per
// KV head (group size times queries per sequence); contiguous caches. One
// workgroup takes up to kWidePairBlock pairs of a (sequence, KV head) unit;
// a unit with more pairs has several such pair blocks, each streaming the
// unit's K/V (on the unit's XCD, so all but the first mostly from its L2).
// Its launch takes arguments already validated by launch_decode.
#ifndef KVC_WIDE_MIN_PAIRS
#define KVC_WIDE_MIN_PAIRS 8
#endif
constexpr int kWidePairBlock = 128;
constexpr int kWideMaxPairs = 512;
inline int wide_pair_blocks(int32_t pairs) {
  return pairs <= kWidePairBlock ? 1 : (pairs + kWidePairBlock - 1) / kWidePairBlock;
}
bool wide_supported(int32_t dtype, int32_t head_dim, int32_t pairs);
// The longest block of queries the wide-group kernel takes: the block's
// rows are folded in as one LDS tile of keys.
constexpr int kWideMaxBlock = 64;
// The kernel's 8-bit mode (kvc_quant_decode_attn): the cache view's k and v
// hold the codes (one byte each, strides in bytes); the scales as here.
struct WideQuant {
  int32_t format;             // KVC_QFMT_*
  int32_t q_dtype;            // KVC_F16 or KVC_BF16: the queries' type, which the codes are widened to
  const float* k_scale;
  const float* v_scale;
  int64_t scale_stride_b, scale_stride_h;   // in floats; the token axis is contiguous
};
// check_only: every host check, nothing enqueued (for a call that enqueues a
// second launch after a first one and must fail before either). quant: the
// 8-bit mode (decode only, no fused append). pg: a paged cache (cache is its
// view, see paged_view); ring: a sliding-window ring cache; both decode only.
kvc_status_t launch_wide(const kvc_cache_t* cache, const int32_t* seq_lens, int32_t n_pending, const void* k_new,
                         const void* v_new, int64_t new_stride_b, int64_t new_stride_h, int64_t new_stride_t,
                         const void* q, int32_t n_q_heads, int32_t t_q, float scale_log2, void* out,
                         int32_t out_dtype, const WsRegions& ws, int32_t splits, int32_t* lens_next,
                         uint32_t* dev_status, hipStream_t stream, bool check_only = false,
                         const WideQuant* quant = nullptr, const PageInfo* pg = nullptr, bool ring = false);
// Whether a decode on this 8-bit cache runs on the wide-group kernel's 8-bit
// mode: fp16/bf16 queries, head dim 64 or 128, KVC_WIDE_QUANT_MIN_GROUP ..
// kWideMaxPairs query heads per KV head.
#ifndef KVC_WIDE_QUANT_MIN_GROUP
#define KVC_WIDE_QUANT_MIN_GROUP 16
#endif
bool quant_routes_wide(const kvc_qcache_t* c, int32_t n_q_heads);

// Bound on the polls of the decode split merge's wait for ready flags (about
// 2^20 by default; kvc_debug_set_merge_spin_limit changes it for tests of the
// time-out path).
int32_t merge_spin_limit();

// The matrix-core prefill kernel (kvc_prefill.hip): whether it is built for
// this dtype and head dim, and its checks and launch (kvc_prefill_attn;
// check_only as for launch_wide).
bool prefill_supported(int32_t dtype, int32_t head_dim);
kvc_status_t launch_prefill(const kvc_cache_t* cache, const int32_t* seq_lens, int32_t t_q, const void* q,
                            int32_t n_q_heads, float scale, void* out, int32_t out_dtype, uint32_t* dev_status,
                            hipStream_t stream, bool check_only = false);

}  // namespace kvc

#endif  // KVC_INTERNAL_H_
