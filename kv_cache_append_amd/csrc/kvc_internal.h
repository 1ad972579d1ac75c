// Host-side helpers shared by the C-ABI entry points (no device code here).
#ifndef KVC_INTERNAL_H_
#define KVC_INTERNAL_H_

#include <stddef.h>
#include <stdint.h>

#include "kvc.h"

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

// Sequence splits per (sequence, KV head, head block) when the caller passes 0.
int32_t auto_splits(const kvc_cache_t* c, int32_t n_q_heads);
// Splits chosen from the sequences' lengths (host array of c->batch values)
// by modelling the launch; see kvc_decode_splits_for_lengths.
int32_t splits_for_lengths(const kvc_cache_t* c, int32_t n_q_heads, const int32_t* lens);

// Workspace: uint32 tickets [B * H_kv * head_blocks], then uint32 ready
// flags [B * H_kv * head_blocks, S] (both zero between calls), then fp32
// partial outputs [B, H_q, S, D], then fp32 (reference, sum) pairs
// [B, H_q, S, 2]; each region starts on a 256-byte boundary.
size_t workspace_bytes(const kvc_cache_t* c, int32_t n_q_heads, int32_t n_splits);
size_t workspace_flag_offset(const kvc_cache_t* c, int32_t n_q_heads, int32_t n_splits);
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

// The matrix-core prefill kernel (kvc_prefill.hip): whether it is built for
// this dtype and head dim, and its launch (arguments as kvc_prefill_attn,
// already validated except for what the kernel itself needs).
bool prefill_supported(int32_t dtype, int32_t head_dim);
kvc_status_t launch_prefill(const kvc_cache_t* cache, const int32_t* seq_lens, int32_t t_q, const void* q,
                            int32_t n_q_heads, float scale, void* out, int32_t out_dtype, uint32_t* dev_status,
                            hipStream_t stream);

}  // namespace kvc

#endif  // KVC_INTERNAL_H_
