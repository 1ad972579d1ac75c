// Host-side validation, split heuristic, workspace sizing and the pure-host
// C-ABI calls (kvc_cache_bytes, kvc_status_str). No device code.
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <functional>
#include <queue>
#include <utility>
#include <vector>

#include "kvc_internal.h"

namespace kvc {

int elem_bytes(int32_t dtype) {
  switch (dtype) {
    case KVC_F32: return 4;
    case KVC_F16: return 2;
    case KVC_BF16: return 2;
    default: return 0;
  }
}

static bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

kvc_status_t check_cache(const kvc_cache_t* c, bool need_vec16) {
  if (c == nullptr) return KVC_ERR_NULL;
  const int s = elem_bytes(c->dtype);
  if (s == 0) return KVC_ERR_DTYPE;
  if (c->batch < 0 || c->n_kv_heads <= 0 || c->max_len < 0 || c->head_dim <= 0 || c->reserved0 != 0)
    return KVC_ERR_SHAPE;
  if (c->batch == 0) return KVC_OK;  // nothing will be touched
  if (c->k == nullptr || c->v == nullptr) return KVC_ERR_NULL;
  // Rows of one (b, h) must not overlap, and the D axis is contiguous.
  if (c->stride_t < c->head_dim) return KVC_ERR_SHAPE;
  if (c->n_kv_heads > 1 && c->stride_h < c->head_dim) return KVC_ERR_SHAPE;
  if (c->batch > 1 && c->stride_b < c->head_dim) return KVC_ERR_SHAPE;
  if (c->stride_b < 0 || c->stride_h < 0) return KVC_ERR_SHAPE;
  if (!aligned(c->k, s) || !aligned(c->v, s)) return KVC_ERR_ALIGN;
  if (need_vec16) {
    if (!aligned(c->k, 16) || !aligned(c->v, 16)) return KVC_ERR_ALIGN;
    if ((c->stride_t * s) % 16 || (c->stride_h * s) % 16 || (c->stride_b * s) % 16) return KVC_ERR_ALIGN;
    if ((static_cast<int64_t>(c->head_dim) * s) % 16) return KVC_ERR_ALIGN;
  }
  return KVC_OK;
}

kvc_status_t paged_view(const kvc_paged_cache_t* pc, bool for_decode, kvc_cache_t* view, PageInfo* info) {
  if (pc == nullptr) return KVC_ERR_NULL;
  const int32_t ps = pc->page_size;
  if (ps <= 0 || (ps & (ps - 1)) != 0 || pc->n_pages <= 0 || pc->pages_per_seq <= 0 ||
      pc->table_stride < pc->pages_per_seq)
    return KVC_ERR_SHAPE;
  if (for_decode && ps < 16) return KVC_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(pc->pages_per_seq) * ps > 0x7fffffffll) return KVC_ERR_SHAPE;
  view->k = pc->k_pages;
  view->v = pc->v_pages;
  view->batch = pc->batch;
  view->n_kv_heads = pc->n_kv_heads;
  view->max_len = pc->pages_per_seq * ps;
  view->head_dim = pc->head_dim;
  view->dtype = pc->dtype;
  view->reserved0 = 0;
  view->stride_b = pc->stride_page;
  view->stride_h = pc->stride_h;
  view->stride_t = pc->stride_t;
  // A page's (head, row) grid must not overlap: head-major or row-major.
  if (pc->n_kv_heads > 1 && pc->stride_h < static_cast<int64_t>(ps) * pc->stride_t &&
      pc->stride_t < static_cast<int64_t>(pc->n_kv_heads) * pc->stride_h)
    return KVC_ERR_SHAPE;
  if (pc->batch > 0 && pc->block_table == nullptr) return KVC_ERR_NULL;
  info->table = pc->block_table;
  info->table_stride = pc->table_stride;
  int shift = 0;
  while ((1 << shift) < ps) ++shift;
  info->page_shift = shift;
  info->n_pages = pc->n_pages;
  return KVC_OK;
}

kvc_status_t check_qcache(const kvc_qcache_t* c, bool for_decode) {
  if (c == nullptr) return KVC_ERR_NULL;
  if (c->format != KVC_QFMT_FP8_E4M3 && c->format != KVC_QFMT_INT8) return KVC_ERR_DTYPE;
  if (elem_bytes(c->in_dtype) == 0) return KVC_ERR_DTYPE;
  if (for_decode && c->in_dtype == KVC_F32) return KVC_ERR_UNSUPPORTED;
  if (c->batch < 0 || c->n_kv_heads <= 0 || c->max_len < 0 || c->head_dim <= 0) return KVC_ERR_SHAPE;
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256) return KVC_ERR_UNSUPPORTED;
  if (c->batch == 0) return KVC_OK;  // nothing will be touched
  if (c->k == nullptr || c->v == nullptr || c->k_scale == nullptr || c->v_scale == nullptr) return KVC_ERR_NULL;
  if (c->stride_b < 0 || c->stride_h < 0 || c->stride_t < c->head_dim) return KVC_ERR_SHAPE;
  if (c->n_kv_heads > 1 && c->stride_h < c->head_dim) return KVC_ERR_SHAPE;
  if (c->batch > 1 && c->stride_b < c->head_dim) return KVC_ERR_SHAPE;
  if (c->scale_stride_b < 0 || c->scale_stride_h < 0) return KVC_ERR_SHAPE;
  if (c->n_kv_heads > 1 && c->scale_stride_h < c->max_len) return KVC_ERR_SHAPE;
  if (c->batch > 1 && c->scale_stride_b < c->max_len) return KVC_ERR_SHAPE;
  if (!aligned(c->k, 16) || !aligned(c->v, 16)) return KVC_ERR_ALIGN;
  if (c->stride_b % 16 || c->stride_h % 16 || c->stride_t % 16) return KVC_ERR_ALIGN;
  if (!aligned(c->k_scale, 4) || !aligned(c->v_scale, 4)) return KVC_ERR_ALIGN;
  return KVC_OK;
}

kvc_cache_t qcache_view(const kvc_qcache_t* c) {
  kvc_cache_t v = {};
  v.k = c->k;
  v.v = c->v;
  v.batch = c->batch;
  v.n_kv_heads = c->n_kv_heads;
  v.max_len = c->max_len;
  v.head_dim = c->head_dim;
  v.dtype = KVC_F16;   // not read by the split heuristic or the workspace layout
  v.stride_b = c->stride_b;
  v.stride_h = c->stride_h;
  v.stride_t = c->stride_t;
  return v;
}

int copy_vector_bytes(const kvc_cache_t* c, const void* src_k, const void* src_v,
                      const int64_t* src_strides_bytes, int n_src_strides) {
  const int s = elem_bytes(c->dtype);
  int vb = 16;
  auto fits = [&](int64_t x) { return (x % vb) == 0; };
  while (vb > s) {
    bool ok = fits(static_cast<int64_t>(c->head_dim) * s) && fits(c->stride_t * s) &&
              fits(c->stride_h * s) && fits(c->stride_b * s) &&
              fits(static_cast<int64_t>(reinterpret_cast<uintptr_t>(c->k))) &&
              fits(static_cast<int64_t>(reinterpret_cast<uintptr_t>(c->v))) &&
              fits(static_cast<int64_t>(reinterpret_cast<uintptr_t>(src_k))) &&
              fits(static_cast<int64_t>(reinterpret_cast<uintptr_t>(src_v)));
    for (int i = 0; ok && i < n_src_strides; ++i) ok = fits(src_strides_bytes[i]);
    if (ok) break;
    vb /= 2;
  }
  return vb;
}

bool decode_head_dim_supported(int32_t head_dim, int32_t dtype) {
  const int s = elem_bytes(dtype);
  if (s == 0) return false;
  switch (head_dim) {
    case 4: case 8: case 16: case 32: case 64: case 128: case 256: break;
    default: return false;
  }
  const int row = head_dim * s;
  return row >= 16 && row <= 1024;
}

int heads_per_block(int32_t group) {
  if (group <= 1) return 1;
  if (group <= 2) return 2;
  if (group <= 4) return 4;
  return 8;
}

int head_blocks(int32_t group) {
  const int hb = heads_per_block(group);
  return (group + hb - 1) / hb;
}

bool quant_routes_wide(const kvc_qcache_t* c, int32_t n_q_heads) {
  if (c == nullptr || c->n_kv_heads <= 0 || n_q_heads <= 0 || n_q_heads % c->n_kv_heads != 0) return false;
  const int32_t group = n_q_heads / c->n_kv_heads;
  return (c->in_dtype == KVC_F16 || c->in_dtype == KVC_BF16) && group >= KVC_WIDE_QUANT_MIN_GROUP &&
         wide_supported(c->in_dtype, c->head_dim, group);
}

bool routes_wide(const kvc_cache_t* c, int32_t n_q_heads) {
  if (c == nullptr || c->n_kv_heads <= 0 || n_q_heads <= 0) return false;
  return wide_supported(c->dtype, c->head_dim, n_q_heads / c->n_kv_heads);
}

int32_t auto_splits(const kvc_cache_t* c, int32_t n_q_heads, bool wide) {
  if (c == nullptr || c->n_kv_heads <= 0 || n_q_heads <= 0 || c->batch <= 0) return 1;
  // workgroups per split: one per (sequence, KV head, pair block) on the
  // wide-group kernel, one per (sequence, KV head, head block) on the other
  const int64_t units = static_cast<int64_t>(c->batch) * c->n_kv_heads *
                        (wide ? wide_pair_blocks(n_q_heads / c->n_kv_heads) : head_blocks(n_q_heads / c->n_kv_heads));
  // Measured on MI355X (256 CUs): the fastest launches hold about one
  // workgroup per CU; more, shorter splits pay the per-workgroup start-up
  // and the merge more often than they gain, and with 256 or more units one
  // split (no merge) is fastest.
  const int64_t target_wgs = 256;
  const int64_t min_chunk = 256;          // tokens per workgroup at least
  int64_t s = (target_wgs + units - 1) / units;
  int64_t cap = static_cast<int64_t>(c->max_len) / min_chunk;
  if (cap < 1) cap = 1;
  if (s > cap) s = cap;
  if (s > KVC_MAX_SPLITS) s = KVC_MAX_SPLITS;
  return static_cast<int32_t>(s);
}

// Workgroups of the decode kernel each CU holds at once: the kernels' launch
// bounds (decode_min_wgs in the kernel source) in host form.
static int resident_wgs(int32_t dtype, int32_t head_dim, int gb) {
  const int s = elem_bytes(dtype);
  if (s == 2 && head_dim % 32 == 0) return (gb > 4 || head_dim > 128) ? 1 : 2;   // matrix-core path
  return (s == 2 && gb <= 4) ? 4 : 1;
}

// Modelled duration (microseconds) of one decode launch with S splits over
// sequences of lens[b] tokens. The launch's workgroups are handed out in
// launch order to per_cu slots on each of the chip's CUs; the workgroups
// running at a time share the chip's streaming rate equally, each at most
// the rate one workgroup reaches alone; a workgroup costs a fixed start-up
// time on top of its bytes; a launch with S > 1 splits ends with the split
// merge. (The rates are measured on MI355X with the 16-bit kernels: about
// 6.4 TB/s for a full chip, about 36 GB/s for a workgroup on its own.)
static double model_launch_us(const int32_t* lens, int32_t batch, int32_t n_kv, int hblk, double row_bytes,
                              int per_cu, int32_t S) {
  constexpr int kCus = 256;                    // MI355X compute units
  constexpr double kChipBytesPerUs = 6.4e6;    // all workgroups together
  constexpr double kWgBytesPerUs = 36.0e3;     // one workgroup alone
  constexpr double kStartUs = 1.0;             // per workgroup: arguments, lengths, first loads
  const double merge_us = S == 1 ? 0.0 : 2.5 + 0.5 * (S - 2);
  std::vector<double> work;
  work.reserve(static_cast<size_t>(batch) * n_kv * S * hblk);
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n = lens[b] < 0 ? 0 : lens[b];
    // the decode kernel's split of [0, n): n - 1 rows in equal 16-row-tile
    // chunks, the last active split also taking row n - 1
    const int64_t chunk = std::max<int64_t>(16, ((n - 1 + S - 1) / S + 15) / 16 * 16);
    const int64_t ns = n > 1 ? std::min<int64_t>(S, (n - 1 + chunk - 1) / chunk) : (n == 1 ? 1 : 0);
    for (int32_t g = 0; g < n_kv; ++g)
      for (int64_t sp = 0; sp < S; ++sp) {   // (an inactive split's workgroup only starts)
        const int64_t t0 = sp * chunk;
        const int64_t rows = sp >= ns ? 0 : (sp == ns - 1 ? n : t0 + chunk) - t0;
        for (int h = 0; h < hblk; ++h) work.push_back(kStartUs * kWgBytesPerUs + rows * row_bytes);
      }
  }
  // Every running workgroup moves at the same rate, so they finish in order
  // of the progress mark (bytes per workgroup since the launch) at which
  // their bytes run out; wall time is accumulated between marks at the rate
  // the number of running workgroups allows.
  const size_t slots = static_cast<size_t>(kCus) * per_cu;
  std::priority_queue<double, std::vector<double>, std::greater<double>> finish;
  size_t next = 0;
  while (finish.size() < slots && next < work.size()) finish.push(work[next++]);
  double mark = 0.0, t = 0.0;
  while (!finish.empty()) {
    const double f = finish.top();
    const double rate = std::min(kWgBytesPerUs, kChipBytesPerUs / static_cast<double>(finish.size()));
    t += (f - mark) / rate;
    mark = f;
    finish.pop();
    if (next < work.size()) finish.push(mark + work[next++]);
  }
  return t + merge_us;
}

int32_t splits_for_lengths(const kvc_cache_t* c, int32_t n_q_heads, const int32_t* lens) {
  const int32_t group = n_q_heads / c->n_kv_heads;
  const int gb = heads_per_block(group);
  const bool wide = routes_wide(c, n_q_heads);
  // the wide-group kernel: one workgroup per (sequence, KV head) and split,
  // one per CU
  const int per_cu = wide ? 1 : std::min(resident_wgs(c->dtype, c->head_dim, gb), 4);
  const int hblk = wide ? wide_pair_blocks(group) : head_blocks(group);
  const double row_bytes = 2.0 * c->head_dim * elem_bytes(c->dtype);   // K and V of one token
  int32_t cap = c->max_len / 256;            // chunks of 256 tokens at least, as the default rule
  if (cap < 1) cap = 1;
  if (cap > 32) cap = 32;
  int32_t best = 1;
  double best_us = 0.0;
  static const int32_t kCandidates[] = {1, 2, 3, 4, 5, 6, 8, 10, 12, 16, 20, 24, 32};
  for (int32_t S : kCandidates) {
    if (S > cap) break;
    const double t = model_launch_us(lens, c->batch, c->n_kv_heads, hblk, row_bytes, per_cu, S);
    if (S == 1 || t < best_us) {
      best = S;
      best_us = t;
    }
  }
  // The model is coarse (it does not see, for one, that whole units stream
  // faster than short chunks), so the length-blind count stands unless the
  // model expects another count to cut the launch by more than a sixth, as
  // for a batch with a few sequences far longer than the rest.
  const int32_t blind = std::min<int32_t>(auto_splits(c, n_q_heads, wide), cap);
  const double blind_us = model_launch_us(lens, c->batch, c->n_kv_heads, hblk, row_bytes, per_cu, blind);
  return best_us < blind_us * (1.0 - 1.0 / 6.0) ? best : blind;
}

// The one setting the library keeps between calls (a test hook; see
// kvc_debug_set_merge_spin_limit).
static std::atomic<int32_t> g_merge_spins{1 << 20};

int32_t merge_spin_limit() { return g_merge_spins.load(std::memory_order_relaxed); }

static size_t round256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

static size_t sync_units(const kvc_cache_t* c, int32_t n_q_heads) {
  return static_cast<size_t>(c->batch) * c->n_kv_heads * head_blocks(n_q_heads / c->n_kv_heads);
}

size_t workspace_flag_offset(const kvc_cache_t*, int32_t, int32_t) { return 0; }

size_t workspace_sync_offset(const kvc_cache_t* c, int32_t n_q_heads, int32_t n_splits) {
  return workspace_flag_offset(c, n_q_heads, n_splits) +
         round256(sync_units(c, n_q_heads) * static_cast<size_t>(n_splits) * sizeof(uint32_t));
}

size_t workspace_o_offset(const kvc_cache_t* c, int32_t n_q_heads, int32_t n_splits) {
  return workspace_sync_offset(c, n_q_heads, n_splits) +
         round256(static_cast<size_t>(c->batch) * c->n_kv_heads * wide_pair_blocks(n_q_heads / c->n_kv_heads) *
                  kWideSyncBytes);
}

size_t workspace_ml_offset(const kvc_cache_t* c, int32_t n_q_heads, int32_t n_splits) {
  const size_t rows = static_cast<size_t>(c->batch) * n_q_heads * n_splits;
  return workspace_o_offset(c, n_q_heads, n_splits) + round256(rows * c->head_dim * sizeof(float));
}

WsRegions workspace_regions(const kvc_cache_t* c, int32_t n_q_heads, int32_t n_splits, void* ws) {
  char* base = static_cast<char*>(ws);
  WsRegions r;
  r.flags = reinterpret_cast<uint32_t*>(base + workspace_flag_offset(c, n_q_heads, n_splits));
  r.flag_stride = n_splits;
  r.sync = reinterpret_cast<uint32_t*>(base + workspace_sync_offset(c, n_q_heads, n_splits));
  r.o = reinterpret_cast<float*>(base + workspace_o_offset(c, n_q_heads, n_splits));
  r.ml = reinterpret_cast<float*>(base + workspace_ml_offset(c, n_q_heads, n_splits));
  return r;
}

size_t workspace_bytes(const kvc_cache_t* c, int32_t n_q_heads, int32_t n_splits) {
  const size_t rows = static_cast<size_t>(c->batch) * n_q_heads * n_splits;
  return workspace_ml_offset(c, n_q_heads, n_splits) + round256(rows * 2 * sizeof(float));
}

}  // namespace kvc

extern "C" uint64_t kvc_cache_bytes(int32_t n_layers, int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                                    const int32_t* h_lens, int32_t batch) {
  const int s = kvc::elem_bytes(dtype);
  if (s == 0 || n_layers < 0 || n_kv_heads < 0 || head_dim < 0 || batch < 0) return 0;
  if (batch > 0 && h_lens == nullptr) return 0;
  uint64_t tokens = 0;
  for (int32_t b = 0; b < batch; ++b) {
    if (h_lens[b] < 0) return 0;
    tokens += static_cast<uint64_t>(h_lens[b]);
  }
  return 2ull * static_cast<uint64_t>(n_layers) * static_cast<uint64_t>(n_kv_heads) *
         static_cast<uint64_t>(head_dim) * static_cast<uint64_t>(s) * tokens;
}

extern "C" const char* kvc_status_str(kvc_status_t status) {
  switch (status) {
    case KVC_OK: return "KVC_OK";
    case KVC_ERR_NULL: return "KVC_ERR_NULL: a required pointer is NULL";
    case KVC_ERR_SHAPE: return "KVC_ERR_SHAPE: invalid size or overlapping strides";
    case KVC_ERR_DTYPE: return "KVC_ERR_DTYPE: unknown dtype";
    case KVC_ERR_ALIGN: return "KVC_ERR_ALIGN: pointer or stride misaligned for the kernels";
    case KVC_ERR_GQA: return "KVC_ERR_GQA: n_q_heads is not a positive multiple of n_kv_heads";
    case KVC_ERR_WORKSPACE: return "KVC_ERR_WORKSPACE: workspace missing or too small";
    case KVC_ERR_UNSUPPORTED: return "KVC_ERR_UNSUPPORTED: head_dim/dtype not built into the decode kernels";
    case KVC_ERR_HIP: return "KVC_ERR_HIP: HIP launch error";
    default: return "KVC_ERR_UNKNOWN";
  }
}

extern "C" int32_t kvc_debug_set_merge_spin_limit(int32_t spins) {
  if (spins < 0) spins = 0;
  return kvc::g_merge_spins.exchange(spins, std::memory_order_relaxed);
}

extern "C" size_t kvc_decode_workspace_bytes(const kvc_cache_t* cache, int32_t n_q_heads, int32_t n_splits) {
  if (kvc::check_cache(cache, false) != KVC_OK) return 0;
  if (n_q_heads <= 0 || n_q_heads % cache->n_kv_heads != 0 || n_splits < 0 || n_splits > KVC_MAX_SPLITS) return 0;
  // (the wide-group kernel's count is never below the other kernel's, so a
  // workspace sized for it also serves paged and ring calls of this geometry)
  const int32_t s = n_splits > 0 ? n_splits : kvc::auto_splits(cache, n_q_heads, kvc::routes_wide(cache, n_q_heads));
  return kvc::workspace_bytes(cache, n_q_heads, s);
}

extern "C" size_t kvc_quant_decode_workspace_bytes(const kvc_qcache_t* cache, int32_t n_q_heads, int32_t n_splits) {
  if (kvc::check_qcache(cache, true) != KVC_OK) return 0;
  if (n_q_heads <= 0 || n_q_heads % cache->n_kv_heads != 0 || n_splits < 0 || n_splits > KVC_MAX_SPLITS) return 0;
  const kvc_cache_t view = kvc::qcache_view(cache);
  const int32_t s =
      n_splits > 0 ? n_splits : kvc::auto_splits(&view, n_q_heads, kvc::quant_routes_wide(cache, n_q_heads));
  return kvc::workspace_bytes(&view, n_q_heads, s);
}

extern "C" size_t kvc_paged_decode_workspace_bytes(const kvc_paged_cache_t* cache, int32_t n_q_heads,
                                                   int32_t n_splits) {
  kvc_cache_t view;
  kvc::PageInfo info;
  if (kvc::paged_view(cache, true, &view, &info) != KVC_OK) return 0;
  return kvc_decode_workspace_bytes(&view, n_q_heads, n_splits);
}

extern "C" size_t kvc_block_workspace_bytes(const kvc_cache_t* cache, int32_t n_q_heads, int32_t t_q,
                                            int32_t n_splits) {
  if (kvc::check_cache(cache, false) != KVC_OK) return 0;
  if (n_q_heads <= 0 || n_q_heads % cache->n_kv_heads != 0) return 0;
  if (t_q <= 0 || static_cast<int64_t>(n_q_heads) * t_q > (1 << 24)) return 0;
  return kvc_decode_workspace_bytes(cache, n_q_heads * t_q, n_splits);
}

extern "C" int32_t kvc_decode_splits_for_lengths(const kvc_cache_t* cache, int32_t n_q_heads,
                                                 const int32_t* h_lens) {
  if (kvc::check_cache(cache, false) != KVC_OK || cache->batch <= 0 || h_lens == nullptr) return 0;
  if (n_q_heads <= 0 || n_q_heads % cache->n_kv_heads != 0) return 0;
  return kvc::splits_for_lengths(cache, n_q_heads, h_lens);
}

extern "C" int32_t kvc_decode_splits(const kvc_cache_t* cache, int32_t n_q_heads) {
  if (kvc::check_cache(cache, false) != KVC_OK) return 0;
  if (n_q_heads <= 0 || n_q_heads % cache->n_kv_heads != 0) return 0;
  return kvc::auto_splits(cache, n_q_heads, kvc::routes_wide(cache, n_q_heads));
}
