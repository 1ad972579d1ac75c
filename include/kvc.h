/*
 * kvc.h -- KV-cache append and single-query decode attention for AMD Instinct
 * MI355X (CDNA4, gfx950). C ABI of libkvc.so.
 *
 * One decode step of one attention layer, as three web pages on the KV cache
 * describe it:
 *   - glossary entry "KV 缓存" (llm-glossary.tokens-kit.com), sections
 *     "placing it back in the inference chain", "two mathematically equivalent
 *     decode paths" (path B) and "capacity formula";
 *   - course notes "第 1 周 · Day 4：KV Cache 与 MQA / GQA" (semidirectx.com),
 *     §1.3 (prefill and decode), §1.4 (memory formula), §2.3 and §3.4 (GQA
 *     grouping), §3.1 (preallocated cache and its update);
 *   - textbook section "11.7 KV Cache：形状、显存与带宽" (yongzhen.wang),
 *     §2.2 (single-step decode) and §2.3 (memory formula).
 *
 * Conventions shared by every call:
 *   - Pointers named h_* are host pointers; every other data pointer is a
 *     device pointer (HBM) on the current HIP device.
 *   - The caller owns every buffer (caches, q, out, workspace, seq_lens,
 *     status word). The library never allocates or frees device memory, never
 *     synchronises the stream, and keeps no mutable global state apart from
 *     one test setting (kvc_debug_set_merge_spin_limit); calls on different
 *     streams are independent.
 *   - Work is enqueued on `stream` (NULL = the null stream) and returns
 *     before it runs. Results are visible after the stream is synchronised.
 *   - Strides are in elements. The head-dimension axis (D) is contiguous.
 *   - Host-detectable errors return a status before anything is enqueued and
 *     with no side effects. Conditions that depend on device data (a full
 *     cache, a negative length) are handled on the device: the sequence is
 *     skipped and a bit is OR-ed into the optional device status word.
 */
#ifndef KVC_H_
#define KVC_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of cache elements (and of q and k_new/v_new). */
typedef enum kvc_dtype {
  KVC_F32 = 0,
  KVC_F16 = 1,   /* IEEE binary16 */
  KVC_BF16 = 2   /* bfloat16 */
} kvc_dtype_t;

typedef enum kvc_status {
  KVC_OK = 0,
  KVC_ERR_NULL = 1,        /* a required pointer is NULL */
  KVC_ERR_SHAPE = 2,       /* a size is negative/zero where it must be positive, or strides overlap rows */
  KVC_ERR_DTYPE = 3,       /* unknown dtype code */
  KVC_ERR_ALIGN = 4,       /* a pointer or stride breaks the alignment the kernels need */
  KVC_ERR_GQA = 5,         /* n_q_heads is not a positive multiple of n_kv_heads */
  KVC_ERR_WORKSPACE = 6,   /* workspace missing or smaller than kvc_decode_workspace_bytes() */
  KVC_ERR_UNSUPPORTED = 7, /* head_dim / dtype / group size the decode kernels are not built for */
  KVC_ERR_HIP = 8          /* the HIP runtime reported an error at launch */
} kvc_status_t;

/* Largest n_splits the decode calls accept (their automatic choice stays below it). */
#define KVC_MAX_SPLITS 256

/* Bits OR-ed into the optional device status word (uint32_t). */
#define KVC_DEVERR_CAPACITY 1u  /* a write or read would pass max_len: that sequence was skipped/clamped */
#define KVC_DEVERR_BADLEN   2u  /* seq_lens[b] < 0: that sequence was skipped / treated as empty */
#define KVC_DEVERR_PAGE     8u  /* a page-table entry is not an index into the page pool: those rows were
                                   not written (append/fill) or read as zeros (decode: outputs invalid) */
#define KVC_DEVERR_SYNC     4u  /* a split merge gave up waiting for another workgroup (never expected;
                                   the outputs of that call are not valid; the workspace stays usable:
                                   see kvc_decode_workspace_bytes) */

/*
 * One layer's preallocated cache: K and V each [batch, n_kv_heads, max_len,
 * head_dim] with the given element strides (course notes §3.1: allocate once
 * to the maximum length; glossary "two equivalent decode paths": the new slot
 * is written in place). K and V share shape, strides and dtype.
 */
typedef struct kvc_cache {
  void* k;
  void* v;
  int32_t batch;
  int32_t n_kv_heads;
  int32_t max_len;
  int32_t head_dim;
  int32_t dtype;       /* kvc_dtype_t */
  int32_t reserved0;   /* must be 0 */
  int64_t stride_b;
  int64_t stride_h;
  int64_t stride_t;
} kvc_cache_t;

/*
 * kvc_append -- write the new token's k_t, v_t into slot seq_lens[b] of every
 * sequence (course notes §3.1 update with one token; glossary path B; textbook
 * §2.2 "append k_t, v_t to the cache").
 *
 *   cache     the layer's cache (device buffers).
 *   seq_lens  int32[batch], device: tokens already cached per sequence. READ
 *             ONLY: one array serves all layers of a step; advance it once per
 *             step with kvc_seq_lens_advance.
 *   k_new,
 *   v_new     [batch, n_kv_heads, head_dim] in the cache dtype, element
 *             strides new_stride_b, new_stride_h (D contiguous).
 *   dev_status optional uint32 device word; KVC_DEVERR_* bits are OR-ed in.
 *
 * The copy is bit-exact. If seq_lens[b] >= max_len (or < 0) nothing is written
 * for sequence b and the status bit is set. Every other slot is untouched.
 * batch == 0 is a no-op.
 */
kvc_status_t kvc_append(const kvc_cache_t* cache, const int32_t* seq_lens,
                        const void* k_new, const void* v_new,
                        int64_t new_stride_b, int64_t new_stride_h,
                        uint32_t* dev_status, hipStream_t stream);

/*
 * kvc_prefill_fill -- write t_new tokens per sequence at slots
 * [seq_lens[b], seq_lens[b] + t_new) (course notes §3.1 update with T tokens;
 * §1.3 prefill writes every position's K/V; §3.5 chunked prefill when
 * seq_lens[b] > 0).
 *
 *   k, v      [batch, n_kv_heads, t_new, head_dim] in the cache dtype with
 *             element strides src_stride_b, src_stride_h, src_stride_t.
 *   t_new     tokens per sequence (0 is a no-op).
 *
 * seq_lens is read only. A sequence whose range does not fit in [0, max_len)
 * is not written and KVC_DEVERR_CAPACITY is set. The copy is bit-exact.
 */
kvc_status_t kvc_prefill_fill(const kvc_cache_t* cache, const int32_t* seq_lens,
                              const void* k, const void* v,
                              int64_t src_stride_b, int64_t src_stride_h, int64_t src_stride_t,
                              int32_t t_new, uint32_t* dev_status, hipStream_t stream);

/*
 * kvc_decode_workspace_bytes -- bytes of device workspace kvc_decode_attn /
 * kvc_decode_step need for this cache, query-head count and split count
 * (n_splits = 0 means the library's choice, the same one the decode calls
 * make). The bound holds for any seq_lens <= max_len. Returns 0 for invalid
 * arguments.
 *
 * Layout and lifetime: uint32 ready flags (one per sequence, KV head, block
 * of query heads and split; the last split's word of each block holds that
 * block's epoch, a count of its merges), then 64 uint32 words per
 * (sequence, KV head) for the wide-group kernel's shared merge (an arrival
 * count that each call returns to zero, per-split claim words that hold the
 * epoch of the call that last claimed them, and that merge's own epoch in
 * the last word), then fp32 per-split partial results. The caller zero-fills the workspace once after
 * allocating it. A call's publishing splits raise their flags (or claims) to
 * epoch + 1 and its merging split waits for exactly that value, then
 * advances the epoch, so the workspace serves any number of later calls with
 * the same batch,
 * n_kv_heads, n_q_heads and split count (any lengths, any layer) without
 * clearing, including calls after one that reported KVC_DEVERR_SYNC: a flag
 * raised late in that call holds an old epoch's value and is never taken
 * for a later call's. Where the geometry changes, the region layout moves:
 * zero-fill the workspace again first (or keep one workspace per geometry).
 * Calls that share a workspace must not run concurrently.
 */
size_t kvc_decode_workspace_bytes(const kvc_cache_t* cache, int32_t n_q_heads, int32_t n_splits);

/*
 * kvc_decode_splits -- the number of sequence splits kvc_decode_attn uses for
 * this cache when n_splits == 0 (0 for invalid arguments).
 */
int32_t kvc_decode_splits(const kvc_cache_t* cache, int32_t n_q_heads);

/*
 * kvc_decode_splits_for_lengths -- a split count for a decode call on this
 * cache when the caller knows the lengths it will attend (h_lens: host array
 * of cache->batch token counts, e.g. seq_lens + n_pending). It models the
 * launch -- workgroups dispatched in launch order to the CUs' slots, the
 * running ones sharing the chip's streaming rate up to what one workgroup
 * reaches alone, a fixed start-up cost per workgroup and a merge cost per
 * extra split -- for split counts from 1 up to min(32, max_len / 256). It
 * returns kvc_decode_splits's count unless the model expects another count
 * to be more than a sixth faster, as when a few sequences are far longer
 * than the rest; those get more, shorter splits, so that no CU is left with
 * a long tail. The model is calibrated on the (bandwidth-bound) 16-bit
 * decode kernels. Host only, a few milliseconds for a few thousand
 * (sequence, KV head) pairs; 0 for invalid arguments. Pass the result as
 * n_splits (and size the workspace for it).
 */
int32_t kvc_decode_splits_for_lengths(const kvc_cache_t* cache, int32_t n_q_heads, const int32_t* h_lens);

/*
 * kvc_decode_attn -- the single new query of every head attends all cached
 * tokens: out[b,h,:] = softmax(scale * q[b,h,:] . K[b,g,t,:]) V[b,g,t,:] over
 * t < N_b = seq_lens[b] + n_pending, with g = h / (n_q_heads / n_kv_heads)
 * (textbook §2.2 single-step decode; glossary decode path; course notes §3.4
 * grouping floor(j/(h/G))). No mask: every cached token precedes the query
 * (course notes §3.3). After kvc_append of the step's token, n_pending = 1
 * attends the t+1 keys of course notes §1.3.
 *
 *   q         [batch, n_q_heads, head_dim], contiguous, cache dtype.
 *   scale     softmax scale, normally 1/sqrt(head_dim); must be finite and
 *             > 0, else KVC_ERR_UNSUPPORTED.
 *   out       [batch, n_q_heads, head_dim], contiguous, dtype out_dtype
 *             (KVC_F32, or the cache dtype rounded to nearest even).
 *   workspace device buffer of at least kvc_decode_workspace_bytes(cache,
 *             n_q_heads, n_splits) bytes, 16-byte aligned, zero-filled once
 *             after allocation (see kvc_decode_workspace_bytes).
 *   n_splits  sequence splits per (sequence, KV head), 0..KVC_MAX_SPLITS;
 *             0 = library choice; larger values return KVC_ERR_SHAPE.
 *             The result does not depend on it beyond fp32 rounding order.
 *
 * Limit: (max_len + 2048) * stride_t * elem_bytes must stay below 2^31 (one
 * sequence's slice of one KV head is addressed with 32-bit offsets), else
 * KVC_ERR_SHAPE. Sequences with N_b == 0 produce a zero row. N_b is clamped to max_len (with
 * KVC_DEVERR_CAPACITY set) so the kernels never read past the cache.
 * Accumulation is fp32; results are run-to-run deterministic.
 * Supported: head_dim in {64, 128, 256} for every dtype, plus head_dim 4..32
 * (powers of two with head_dim * elem_bytes >= 16); any group size.
 * Groups of 8..512 query heads per KV head on fp16/bf16 caches with head_dim
 * 64 or 128 run on a kernel that streams each KV head's K/V once per 128
 * heads of the group, both products on the matrix cores (course notes §2.2,
 * §2.5: the group shares its K/V, saving bytes, not FLOPs); the other shapes
 * read K/V once per block of up to 8 query heads.
 */
kvc_status_t kvc_decode_attn(const kvc_cache_t* cache, const int32_t* seq_lens, int32_t n_pending,
                             const void* q, int32_t n_q_heads, float scale,
                             void* out, int32_t out_dtype,
                             void* workspace, size_t workspace_bytes, int32_t n_splits,
                             uint32_t* dev_status, hipStream_t stream);

/*
 * kvc_decode_step -- kvc_append followed by kvc_decode_attn with n_pending = 1,
 * in one launch: the new token's k_t, v_t are written into slot seq_lens[b]
 * and every query head attends the seq_lens[b] + 1 tokens [0, seq_lens[b]]
 * (course notes §1.3: k, v appended, then q attends all t+1 keys; textbook
 * §2.2). The cache bytes written and the output are identical to the two
 * separate calls. k_new / v_new are [batch, n_kv_heads, head_dim] with
 * element strides new_stride_b, new_stride_h; here they must be 16-byte
 * aligned (pointers and strides in bytes), else KVC_ERR_ALIGN and nothing is
 * enqueued. seq_lens stays read only. A full cache (seq_lens[b] >= max_len) is
 * not written, the flag is set and the sequence attends its max_len stored
 * tokens, as with the separate calls. Other arguments as kvc_decode_attn.
 */
kvc_status_t kvc_decode_step(const kvc_cache_t* cache, const int32_t* seq_lens,
                             const void* k_new, const void* v_new,
                             int64_t new_stride_b, int64_t new_stride_h,
                             const void* q, int32_t n_q_heads, float scale,
                             void* out, int32_t out_dtype,
                             void* workspace, size_t workspace_bytes, int32_t n_splits,
                             uint32_t* dev_status, hipStream_t stream);

/*
 * kvc_decode_step_advance -- kvc_decode_step for the last layer of a decode
 * step: the same launch also writes seq_lens_next[b] = seq_lens[b] + 1 for
 * every sequence (what kvc_seq_lens_advance does in a launch of its own;
 * course notes §3.1: each update advances the write position). The
 * lengths are read from seq_lens and written to seq_lens_next, int32[batch]
 * device arrays that must not overlap (KVC_ERR_SHAPE), so no workgroup of the
 * launch sees a changed length; the next step reads seq_lens_next (a
 * caller alternates two arrays). Cache bytes and outputs are those of
 * kvc_decode_step; seq_lens_next is written whatever the device status (a
 * negative or full length plus one, as kvc_seq_lens_advance would).
 * NULL seq_lens_next (with batch > 0): KVC_ERR_NULL. Other arguments as
 * kvc_decode_step.
 */
kvc_status_t kvc_decode_step_advance(const kvc_cache_t* cache, const int32_t* seq_lens, int32_t* seq_lens_next,
                                     const void* k_new, const void* v_new,
                                     int64_t new_stride_b, int64_t new_stride_h,
                                     const void* q, int32_t n_q_heads, float scale,
                                     void* out, int32_t out_dtype,
                                     void* workspace, size_t workspace_bytes, int32_t n_splits,
                                     uint32_t* dev_status, hipStream_t stream);

/*
 * kvc_decode_step_noalloc -- kvc_decode_step for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops or harnesses
 * that forbid hipMalloc): no workspace argument, and the call allocates
 * nothing. The split exchange (ready flags with their epochs, partial
 * results) lives in a device array of the library, 16 MiB on each GPU it
 * runs on, allocated when the library is loaded there and held until the
 * process ends. Calls of any geometry may follow one another on it. A call
 * whose exchange does not fit -- more than 2048 (sequence, KV head, block of
 * query heads) rows, or more partial results than the rest of the array holds
 * (batch * n_q_heads * splits * (head_dim + 2) * 4 bytes, about 14 MiB) --
 * returns KVC_ERR_WORKSPACE before anything is enqueued. Every call on one
 * GPU uses the same array: calls that overlap in time on one GPU (on two
 * streams) race and must not be issued. Results are bit-identical to
 * kvc_decode_step with the same n_splits. Other arguments as kvc_decode_step.
 */
kvc_status_t kvc_decode_step_noalloc(const kvc_cache_t* cache, const int32_t* seq_lens,
                                     const void* k_new, const void* v_new,
                                     int64_t new_stride_b, int64_t new_stride_h,
                                     const void* q, int32_t n_q_heads, float scale,
                                     void* out, int32_t out_dtype, int32_t n_splits,
                                     uint32_t* dev_status, hipStream_t stream);

/*
 * kvc_block_attn -- a block of t_q new tokens per sequence (a prefill chunk
 * or a speculative verify step) attends the cache with the causal mask
 * aligned to the lower right (course notes "第 1 周 · Day 4" §3.3, masks with
 * a cache): query i of sequence b sees slots 0 .. seq_lens[b] + i. The
 * block's own K/V rows must already be in the cache at slots
 * [seq_lens[b], seq_lens[b] + t_q) (kvc_prefill_fill with the same seq_lens
 * writes them); seq_lens is only read. Scale and GQA grouping as in
 * kvc_decode_attn; with t_q = 1 the result is the same as kvc_decode_attn
 * with n_pending = 1.
 *
 *   t_q       queries per sequence, >= 1 (t_q * n_q_heads <= 2^24).
 *   q         [batch, t_q, n_q_heads, head_dim], contiguous, cache dtype
 *             (token-major, as a block's projections come out).
 *   out       [batch, t_q, n_q_heads, head_dim], contiguous, out_dtype.
 *   workspace at least kvc_block_workspace_bytes(cache, n_q_heads, t_q,
 *             n_splits) bytes, with the lifetime rules of
 *             kvc_decode_workspace_bytes (geometry includes t_q).
 *   n_splits  as for kvc_decode_attn (0 = library choice).
 *
 * The (query, head) pairs of a KV head are processed like the query heads of
 * a larger group, so K/V rows are streamed once per block of up to 8 pairs,
 * or, on fp16/bf16 caches with head_dim 64 or 128, 8..512 pairs per KV head
 * and t_q <= 64, once per 128 of them (the wide-group kernel, as for decode
 * with 8+ query heads per KV head); this suits verify steps and chunks of up
 * to 64 tokens. Other blocks of t_q >= 8 with t_q * (n_q_heads / n_kv_heads)
 * >= 32 on fp16/bf16 caches with head_dim 64 or 128 run on the kernel of
 * kvc_prefill_attn (the same result bits as that call; n_splits is then
 * unused, the workspace rules stand). A sequence whose
 * block does not fit (seq_lens[b] < 0, or seq_lens[b] + t_q > max_len) gets
 * zero rows and KVC_DEVERR_BADLEN / KVC_DEVERR_CAPACITY. Host-side errors as
 * for kvc_decode_attn, and KVC_ERR_SHAPE for t_q < 1.
 */
kvc_status_t kvc_block_attn(const kvc_cache_t* cache, const int32_t* seq_lens, int32_t t_q,
                            const void* q, int32_t n_q_heads, float scale,
                            void* out, int32_t out_dtype,
                            void* workspace, size_t workspace_bytes, int32_t n_splits,
                            uint32_t* dev_status, hipStream_t stream);

/*
 * kvc_block_workspace_bytes -- workspace kvc_block_attn needs (0 for invalid
 * arguments); n_splits = 0 means the library's choice.
 */
size_t kvc_block_workspace_bytes(const kvc_cache_t* cache, int32_t n_q_heads, int32_t t_q, int32_t n_splits);

/*
 * kvc_block_step -- kvc_prefill_fill of a block's t_q new rows per sequence
 * followed by kvc_block_attn over them, the block form of kvc_decode_step
 * (course notes "第 1 周 · Day 4" §3.1, the cache update of T new tokens, and
 * §3.3, the lower-right causal mask with a cache): k_new/v_new rows t of
 * sequence b are written into slots seq_lens[b] + t, and query i of the block
 * attends slots 0 .. seq_lens[b] + i. Cache bytes and output bits are those
 * of the two separate calls with the same arguments.
 *
 *   k_new, v_new  [batch, n_kv_heads, t_q, head_dim] rows in the cache dtype
 *             with element strides new_stride_b, new_stride_h, new_stride_t
 *             (head_dim contiguous; new_stride_t >= head_dim when t_q > 1).
 *   Other arguments as kvc_block_attn (workspace sized by
 *             kvc_block_workspace_bytes); seq_lens is only read.
 *
 * Where the block runs on the wide-group kernel (fp16/bf16, head_dim 64 or
 * 128, 8..512 (query, head) pairs per KV head), t_q * head_dim <= 4096 and
 * k_new/v_new rows are 16-byte aligned, this is one launch: the kernel
 * folds the block's rows in from k_new/v_new and writes them into the cache
 * (no workgroup reads those slots from the cache). Otherwise it enqueues the
 * fill, then the attention. A block that does not fit (seq_lens[b] < 0 or
 * seq_lens[b] + t_q > max_len) is not written, gets zero rows and sets
 * KVC_DEVERR_BADLEN / KVC_DEVERR_CAPACITY, as with the separate calls.
 * Host-side errors as for kvc_prefill_fill and kvc_block_attn, returned
 * before anything is enqueued.
 */
kvc_status_t kvc_block_step(const kvc_cache_t* cache, const int32_t* seq_lens, int32_t t_q,
                            const void* k_new, const void* v_new,
                            int64_t new_stride_b, int64_t new_stride_h, int64_t new_stride_t,
                            const void* q, int32_t n_q_heads, float scale,
                            void* out, int32_t out_dtype,
                            void* workspace, size_t workspace_bytes, int32_t n_splits,
                            uint32_t* dev_status, hipStream_t stream);

/*
 * kvc_prefill_attn -- the same operation as kvc_block_attn (query i of
 * sequence b attends slots 0 .. seq_lens[b] + i; course notes "第 1 周 ·
 * Day 4" §3.3, masks with a cache), tiled for long blocks: a whole prompt
 * (seq_lens[b] = 0 gives the causal prefill of §1.3) or a long prefill chunk.
 * The block's K/V rows must already be in the cache at slots
 * [seq_lens[b], seq_lens[b] + t_q); seq_lens is only read.
 *
 *   cache     fp16 or bf16, head_dim 64 or 128 (else KVC_ERR_UNSUPPORTED;
 *             fp32 caches and other head dims use kvc_block_attn).
 *   t_q       queries per sequence, >= 1.
 *   q         [batch, t_q, n_q_heads, head_dim], contiguous, cache dtype,
 *             16-byte aligned.
 *   out       [batch, t_q, n_q_heads, head_dim], contiguous, out_dtype
 *             (KVC_F32 or the cache dtype).
 *   scale     softmax scale, finite and > 0.
 *
 * Scores and accumulation are fp32 on the matrix cores; the softmax weights
 * enter the weighted sum of V as two 16-bit parts (about 16 significant
 * bits). No workspace: every output row is produced by one workgroup. A
 * sequence whose block does not fit (seq_lens[b] < 0, or seq_lens[b] + t_q >
 * max_len) gets zero rows and KVC_DEVERR_BADLEN / KVC_DEVERR_CAPACITY.
 * Host-side errors: KVC_ERR_NULL, KVC_ERR_GQA, KVC_ERR_DTYPE, KVC_ERR_ALIGN,
 * KVC_ERR_SHAPE (t_q < 1, or a slice too large for 32-bit offsets).
 */
kvc_status_t kvc_prefill_attn(const kvc_cache_t* cache, const int32_t* seq_lens, int32_t t_q,
                              const void* q, int32_t n_q_heads, float scale,
                              void* out, int32_t out_dtype, uint32_t* dev_status, hipStream_t stream);

/*
 * Ring cache for sliding-window layers (course notes "第 1 周 · Day 4" §2.7:
 * a layer that only attends its most recent W tokens needs a cache of W
 * slots; §1.6: with rotary positions baked into the cached K, the window can
 * roll over a fixed buffer). A kvc_cache_t whose max_len is the window W;
 * seq_lens[b] counts every token sequence b has seen (not capped at W), and
 * token number t lives in slot t % W, overwriting token t - W.
 *
 * kvc_ring_append / kvc_ring_prefill_fill -- write token numbers
 * seq_lens[b] .. seq_lens[b] + t_new - 1 into their slots (of a block longer
 * than W only the last W rows are written, the others would be overwritten
 * within the block). Never a capacity error; seq_lens[b] < 0 skips the
 * sequence (KVC_DEVERR_BADLEN). Any dtype and head dim.
 *
 * kvc_ring_decode_attn / kvc_ring_decode_step -- each sequence attends its
 * most recent min(seq_lens[b] + n_pending, W) tokens (n_pending = 1 for the
 * step, which also writes the new token into slot seq_lens[b] % W). With no
 * mask the order of the slots does not matter. Arguments, workspace
 * (kvc_decode_workspace_bytes) and errors as for the contiguous calls; the
 * step equals kvc_ring_append + kvc_ring_decode_attn bit for bit. Groups of
 * 8..512 query heads on fp16/bf16 caches with head_dim 64 or 128 stream each
 * KV head once per 128 heads, as in kvc_decode_attn.
 */
kvc_status_t kvc_ring_append(const kvc_cache_t* cache, const int32_t* seq_lens,
                             const void* k_new, const void* v_new,
                             int64_t new_stride_b, int64_t new_stride_h,
                             uint32_t* dev_status, hipStream_t stream);
kvc_status_t kvc_ring_prefill_fill(const kvc_cache_t* cache, const int32_t* seq_lens,
                                   const void* k, const void* v,
                                   int64_t src_stride_b, int64_t src_stride_h, int64_t src_stride_t,
                                   int32_t t_new, uint32_t* dev_status, hipStream_t stream);
kvc_status_t kvc_ring_decode_attn(const kvc_cache_t* cache, const int32_t* seq_lens, int32_t n_pending,
                                  const void* q, int32_t n_q_heads, float scale,
                                  void* out, int32_t out_dtype,
                                  void* workspace, size_t workspace_bytes, int32_t n_splits,
                                  uint32_t* dev_status, hipStream_t stream);
kvc_status_t kvc_ring_decode_step(const kvc_cache_t* cache, const int32_t* seq_lens,
                                  const void* k_new, const void* v_new,
                                  int64_t new_stride_b, int64_t new_stride_h,
                                  const void* q, int32_t n_q_heads, float scale,
                                  void* out, int32_t out_dtype,
                                  void* workspace, size_t workspace_bytes, int32_t n_splits,
                                  uint32_t* dev_status, hipStream_t stream);

/*
 * Paged cache (NEXT to the contiguous one): the same logical K/V sequence per
 * (sequence, KV head), stored in fixed-size pages of a shared pool and
 * addressed through a per-sequence page table (glossary "KV 缓存", relation
 * to PagedAttention: paging changes where rows live, not the sequence or the
 * attention result; course notes §1.6 and textbook §8: it removes the
 * fragmentation of per-sequence maximum-length allocations). Logical slot t
 * of sequence b is row t % page_size of page block_table[b * table_stride +
 * t / page_size]. The capacity of a sequence is pages_per_seq * page_size.
 */
typedef struct kvc_paged_cache {
  void* k_pages;                /* K pool: n_pages pages of [n_kv_heads, page_size, head_dim] (strides below) */
  void* v_pages;                /* V pool, same geometry and strides */
  const int32_t* block_table;   /* device, row b holds the physical pages of sequence b's logical pages */
  int32_t batch;
  int32_t n_kv_heads;
  int32_t page_size;            /* tokens per page: a power of two; >= 16 for the decode calls */
  int32_t head_dim;
  int32_t dtype;                /* kvc_dtype_t */
  int32_t n_pages;              /* pages in each pool */
  int32_t pages_per_seq;        /* table entries per sequence */
  int32_t table_stride;         /* elements between table rows, >= pages_per_seq */
  int64_t stride_page;          /* element strides in the pools; head_dim is contiguous */
  int64_t stride_h;
  int64_t stride_t;
} kvc_paged_cache_t;

/*
 * kvc_paged_append / kvc_paged_prefill_fill -- as kvc_append and
 * kvc_prefill_fill, through the page table. A sequence whose block passes
 * its capacity is skipped (KVC_DEVERR_CAPACITY); a row whose table entry is
 * not in [0, n_pages) is not written (KVC_DEVERR_PAGE). Any dtype and head
 * dim; page_size a power of two.
 */
kvc_status_t kvc_paged_append(const kvc_paged_cache_t* cache, const int32_t* seq_lens,
                              const void* k_new, const void* v_new,
                              int64_t new_stride_b, int64_t new_stride_h,
                              uint32_t* dev_status, hipStream_t stream);
kvc_status_t kvc_paged_prefill_fill(const kvc_paged_cache_t* cache, const int32_t* seq_lens,
                                    const void* k, const void* v,
                                    int64_t src_stride_b, int64_t src_stride_h, int64_t src_stride_t,
                                    int32_t t_new, uint32_t* dev_status, hipStream_t stream);

/*
 * kvc_paged_decode_workspace_bytes / kvc_paged_decode_attn /
 * kvc_paged_decode_step -- as their contiguous counterparts, reading K/V
 * through the page table (and, for the step, writing the new row into its
 * page). fp16/bf16 caches with head_dim a multiple of 32 and page_size a
 * power of two >= 16 (else KVC_ERR_UNSUPPORTED). The result equals the
 * contiguous call on the same logical cache bit for bit (groups of 8..512
 * heads at head_dim 64 or 128 on the same wide-group kernel). A table entry
 * outside the pool sets KVC_DEVERR_PAGE; that page reads as zeros and the
 * sequence's output is not valid.
 */
size_t kvc_paged_decode_workspace_bytes(const kvc_paged_cache_t* cache, int32_t n_q_heads, int32_t n_splits);
kvc_status_t kvc_paged_decode_attn(const kvc_paged_cache_t* cache, const int32_t* seq_lens, int32_t n_pending,
                                   const void* q, int32_t n_q_heads, float scale,
                                   void* out, int32_t out_dtype,
                                   void* workspace, size_t workspace_bytes, int32_t n_splits,
                                   uint32_t* dev_status, hipStream_t stream);
kvc_status_t kvc_paged_decode_step(const kvc_paged_cache_t* cache, const int32_t* seq_lens,
                                   const void* k_new, const void* v_new,
                                   int64_t new_stride_b, int64_t new_stride_h,
                                   const void* q, int32_t n_q_heads, float scale,
                                   void* out, int32_t out_dtype,
                                   void* workspace, size_t workspace_bytes, int32_t n_splits,
                                   uint32_t* dev_status, hipStream_t stream);

/*
 * Quantised cache (NEXT to the 16-bit one): K and V stored as 8-bit codes
 * with one fp32 scale per (sequence, KV head, token) for K and another for V
 * (textbook "11.7 KV Cache" §3.1: weights in fp16, cache in fp8/int8, softmax
 * accumulated in fp32; §8: quantising the cache cuts the bytes read; glossary
 * "KV 缓存", how quantisation changes capacity: the scale granularity,
 * packing and the kernel's handling decide the real saving, which is lost if
 * the cache is widened back to 16 bits in memory first). The pages fix no
 * format; this library's is:
 *   scale = amax / QMAX, an fp32 division, amax = max |x| over the row's
 *           head_dim values, QMAX = 448 (KVC_QFMT_FP8_E4M3) or 127
 *           (KVC_QFMT_INT8); a row of zeros gets scale 0 and zero codes;
 *   code  = encode(x / scale), the quotient an fp32 division: OCP 8-bit E4M3
 *           (bias 7, no infinities, 0x7F/0xFF NaN) rounded to nearest even
 *           and saturating at +-448, or int8 (two's complement) rounded half
 *           to even and clamped to [-127, 127];
 *   a code stands for code * scale, and decode attends those values.
 * Rows holding NaN or infinity give unspecified codes and scales. Decode
 * widens the codes in registers, never in memory: per token and head it reads
 * head_dim + 4 bytes of K and as many of V.
 */
#define KVC_QFMT_FP8_E4M3 0
#define KVC_QFMT_INT8 1

typedef struct kvc_qcache {
  void* k;                  /* K codes [batch, n_kv_heads, max_len, head_dim], one byte each */
  void* v;                  /* V codes, same geometry and strides */
  float* k_scale;           /* K scales [batch, n_kv_heads, max_len], fp32, token axis contiguous */
  float* v_scale;           /* V scales, same geometry and strides */
  int32_t batch;
  int32_t n_kv_heads;
  int32_t max_len;
  int32_t head_dim;         /* 64, 128 or 256 */
  int32_t format;           /* KVC_QFMT_* */
  int32_t in_dtype;         /* kvc_dtype_t of the rows appended and of the queries: KVC_F16 or KVC_BF16
                               (KVC_F32 is accepted by the append and fill calls only) */
  int64_t stride_b;         /* code strides in bytes (= elements); head_dim contiguous; */
  int64_t stride_h;         /*   all three multiples of 16 and the code pointers 16-byte aligned */
  int64_t stride_t;
  int64_t scale_stride_b;   /* scale strides in floats (the token stride is 1) */
  int64_t scale_stride_h;
} kvc_qcache_t;

/*
 * kvc_quant_append / kvc_quant_prefill_fill -- as kvc_append and
 * kvc_prefill_fill (same slots, same capacity and negative-length rules), but
 * each new row (in_dtype, [B, H_kv, D] or [B, H_kv, T_new, D], element
 * strides) is quantised on the device into its codes and scale.
 */
kvc_status_t kvc_quant_append(const kvc_qcache_t* cache, const int32_t* seq_lens,
                              const void* k_new, const void* v_new,
                              int64_t new_stride_b, int64_t new_stride_h,
                              uint32_t* dev_status, hipStream_t stream);
kvc_status_t kvc_quant_prefill_fill(const kvc_qcache_t* cache, const int32_t* seq_lens,
                                    const void* k, const void* v,
                                    int64_t src_stride_b, int64_t src_stride_h, int64_t src_stride_t,
                                    int32_t t_new, uint32_t* dev_status, hipStream_t stream);

/*
 * kvc_quant_decode_workspace_bytes / kvc_quant_decode_attn -- as
 * kvc_decode_workspace_bytes and kvc_decode_attn over the values the codes
 * stand for. q is [B, H_q, D] in in_dtype (KVC_F16 or KVC_BF16, else
 * KVC_ERR_UNSUPPORTED); out is fp32 or in_dtype. The workspace rules are the
 * contiguous decode's. Groups of 16..512 query heads per KV head (head_dim
 * 64 or 128) read each KV head's codes once per 128 heads (the wide-group
 * kernel, its codes widened exactly to in_dtype); other groups once per
 * block of up to 8 heads.
 *
 * kvc_quant_decode_step -- kvc_quant_append then kvc_quant_decode_attn with
 * n_pending = 1, in one launch: the workgroup that attends slot seq_lens[b]
 * quantises the new row itself, folds it in and writes its codes and scale
 * (for the groups the wide-group kernel takes: the two launches, enqueued
 * after every host check of both). Codes, scales and output equal those of
 * the two calls bit for bit.
 */
size_t kvc_quant_decode_workspace_bytes(const kvc_qcache_t* cache, int32_t n_q_heads, int32_t n_splits);
kvc_status_t kvc_quant_decode_attn(const kvc_qcache_t* cache, const int32_t* seq_lens, int32_t n_pending,
                                   const void* q, int32_t n_q_heads, float scale,
                                   void* out, int32_t out_dtype,
                                   void* workspace, size_t workspace_bytes, int32_t n_splits,
                                   uint32_t* dev_status, hipStream_t stream);
kvc_status_t kvc_quant_decode_step(const kvc_qcache_t* cache, const int32_t* seq_lens,
                                   const void* k_new, const void* v_new,
                                   int64_t new_stride_b, int64_t new_stride_h,
                                   const void* q, int32_t n_q_heads, float scale,
                                   void* out, int32_t out_dtype,
                                   void* workspace, size_t workspace_bytes, int32_t n_splits,
                                   uint32_t* dev_status, hipStream_t stream);

/*
 * kvc_seq_lens_advance -- seq_lens[b] += n for every b, on the device, once per
 * step after all layers appended (course notes §3.1: pos += T).
 */
kvc_status_t kvc_seq_lens_advance(int32_t* seq_lens, int32_t batch, int32_t n, hipStream_t stream);

/*
 * kvc_cache_bytes -- logical K+V payload 2 * n_layers * n_kv_heads * head_dim *
 * elem_bytes * sum_b h_lens[b] (glossary "capacity formula", ragged form;
 * course notes §1.4; textbook §2.3). Host only. Returns 0 on invalid input.
 */
uint64_t kvc_cache_bytes(int32_t n_layers, int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                         const int32_t* h_lens, int32_t batch);

/*
 * kvc_stream_read -- a measurement aid, not part of the decode path: reads
 * every byte of buf (device, 16-byte aligned, bytes a multiple of 16) once
 * with the 16-byte buffer loads the decode kernel uses, from n_workgroups
 * workgroups of 256 threads, and stores one XOR fold per thread into sink
 * (device, kvc_stream_read_sink_bytes(n_workgroups) bytes) so no load is
 * dropped. Timed over a buffer far larger than the caches on the chip, it
 * gives the streaming-read rate that bounds any kernel streaming the same
 * bytes (textbook "11.7 KV Cache" §4.4: decode sits on the bandwidth roof).
 */
size_t kvc_stream_read_sink_bytes(int32_t n_workgroups);
kvc_status_t kvc_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t n_workgroups,
                             hipStream_t stream);

/*
 * kvc_split_read -- a measurement aid, not part of the decode path: the data
 * movement of a decode launch on this cache without its arithmetic. It runs
 * the workgroups of a decode call with n_splits splits (one per (sequence,
 * KV head) unit and split, a unit's splits on one XCD), reads the K and V
 * rows [0, seq_lens[b] + 1) of every unit once with the decode kernel's
 * 16-byte non-temporal loads of 16-row tiles, merges its four waves through
 * LDS, and exchanges the splits' partial results as decode does (the other
 * splits publish 2 KB and raise an epoch flag; the last split waits, folds
 * and writes). Every loaded 16-byte word is XOR-folded into the unit's 2 KB
 * of out ([units][128] 16-byte words, device), so no load is dropped and the
 * XOR of a unit's words is the XOR of every word of its rows. Timed beside
 * the decode launch, it separates the cost of the stream and the split
 * exchange, which any split decode pays, from that of the attention's
 * arithmetic (textbook "11.7 KV Cache" §4.4, course notes §1.5).
 *
 *   cache     fp32/fp16/bf16, head_dim * elem_bytes of 64, 128, 256 or 512
 *             bytes (else KVC_ERR_UNSUPPORTED); 16-byte aligned rows.
 *   workspace kvc_split_read_workspace_bytes(cache, n_splits) bytes, 256-byte
 *             aligned, zero-filled once after allocation (epoch flags, as
 *             for kvc_decode_workspace_bytes; one workspace per geometry).
 *   n_splits  1..KVC_MAX_SPLITS.
 */
size_t kvc_split_read_workspace_bytes(const kvc_cache_t* cache, int32_t n_splits);
kvc_status_t kvc_split_read(const kvc_cache_t* cache, const int32_t* seq_lens, int32_t n_splits, void* out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* kvc_status_str -- static, human-readable name of a status code. */
const char* kvc_status_str(kvc_status_t status);

/*
 * kvc_debug_set_merge_spin_limit -- a test hook, not for production use: the
 * number of polls after which the decode split merge stops waiting for
 * another split's ready flag and reports KVC_DEVERR_SYNC (default about
 * 2^20, tens of milliseconds; values below 0 are taken as 0). Process-wide,
 * read by each later decode launch; returns the previous value. This
 * setting is the only state the library keeps between calls. Tests use it
 * to force the time-out path from the host and check that the workspace
 * stays usable afterwards.
 */
int32_t kvc_debug_set_merge_spin_limit(int32_t spins);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H_ */
