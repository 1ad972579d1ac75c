// Causal attention of a long block of new queries over the cache (a whole
// prompt, or a long prefill chunk) on the CDNA4 matrix cores.
//
// The operation is the one kvc_block_attn computes (course notes
// "第 1 周 · Day 4" §3.3, masks with a cache; with nothing cached before the
// block it is the causal prefill of §1.3): query i of sequence b sees cache
// slots 0 .. seq_lens[b] + i. For a block of hundreds or thousands of queries
// the work is a pair of dense products per head, so it is tiled as flash
// attention is:
//   * one 256-thread workgroup per (sequence, query head, 128 queries); each
//     of its four waves owns 32 queries (two 16-query column blocks);
//   * the unit's K/V rows go through LDS in tiles of 64 keys: K as it is
//     stored (padded rows), V transposed (one row per head-dim element), so
//     both products read their matrix-core operands as 16-byte LDS loads;
//   * scores are computed transposed, S^T = K Q^T, on
//     v_mfma_f32_16x16x32_{bf16,f16}: a lane then holds the scores of one
//     query, so the running maximum, the rescale and the weights stay in its
//     registers (a max over the four lanes that share a query is the only
//     exchange);
//   * the output is accumulated transposed too, O^T += V^T P^T, with the
//     fp32 weights P split into two 16-bit parts (P = hi + lo, both exact
//     sums of bits), so the product keeps about 16 significant bits of each
//     weight while running on the 16-bit matrix cores; accumulation is fp32;
//   * a 128-query tile of a sequence whose block starts at slot c needs keys
//     [0, c + last query + 1) only; the mask is applied in the tiles that
//     cross the diagonal, and a wave skips tiles it cannot see.
// Workgroups of one (sequence, KV head) share its K/V: when the unit count
// is a multiple of eight they are placed on one XCD (the dispatcher deals
// workgroup ids round-robin over the eight XCDs), heaviest query tiles first.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "kvc.h"
#include "kvc_internal.h"

namespace {

#include "kvc_tile.h"

constexpr int kQTile = 128;      // queries per workgroup
constexpr int kKTile = 64;       // keys per LDS tile

struct PrefillParams {
  const char* k;
  const char* v;
  int64_t sb, sh, st;            // cache strides in bytes
  const int32_t* seq_lens;
  const char* q;                 // [B, t_q, H_q, D]
  void* out;                     // [B, t_q, H_q, D]
  uint32_t* status;
  int32_t batch, n_q, n_kv, group, t_q, max_len, n_qt, out_f32, xcd_major;
  float scale_log2;              // softmax scale times log2(e)
};


template <typename ET, int D>
__global__ __launch_bounds__(256, 2) void prefill_kernel(const PrefillParams p) {
  constexpr int NC = D / 32;            // 32-element slices of a row (score product depth)
  constexpr int ND = D / 16;            // 16-element output blocks
  constexpr int RB = 2 * D;             // bytes per K or V row in LDS
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int kTileBytes = kKTile * RB;   // one K or one V tile
  constexpr int NLD = kKTile * CPR / 256;   // 16-byte loads per thread per tile, K and V each
  // two buffers of a K tile and a V tile: one computed while the next lands
  __shared__ __attribute__((aligned(16))) char smem[4 * kTileBytes];

  const int units = p.batch * p.n_kv;
  const int per_unit = p.group * p.n_qt;
  int unit, qt, hg;
  if (p.xcd_major) {                    // one unit's workgroups on one XCD
    const int xcd = blockIdx.x & 7;
    const int j = blockIdx.x >> 3;
    unit = (j / per_unit) * 8 + xcd;
    const int r = j % per_unit;
    qt = p.n_qt - 1 - r / p.group;
    hg = r % p.group;
  } else {
    const int j = blockIdx.x;
    const int per_qt = units * p.group;
    qt = p.n_qt - 1 - j / per_qt;
    const int r = j % per_qt;
    unit = r / p.group;
    hg = r % p.group;
  }
  if (unit >= units) return;             // grid padding
  const int b = unit / p.n_kv;
  const int g = unit - b * p.n_kv;
  const int h = g * p.group + hg;
  const int c0 = p.seq_lens[b];
  const int i0 = qt * kQTile;
  const int nq = min(kQTile, p.t_q - i0);  // queries of this tile
  if (c0 < 0 || c0 > p.max_len - p.t_q) {   // the block does not fit (no overflow): zero rows, flagged once
    if (threadIdx.x == 0 && qt == 0 && hg == 0 && g == 0 && p.status != nullptr)
      atomicOr(p.status, c0 < 0 ? KVC_DEVERR_BADLEN : KVC_DEVERR_CAPACITY);
    for (int t = threadIdx.x; t < nq * D; t += blockDim.x) {
      const int64_t idx = ((static_cast<int64_t>(b) * p.t_q + i0 + t / D) * p.n_q + h) * D + t % D;
      if (p.out_f32) static_cast<float*>(p.out)[idx] = 0.f;
      else ET::store(p.out, idx, 0.f);
    }
    return;
  }
  const int n = c0 + p.t_q;                            // rows in the cache for this block
  const int n_tiles = (c0 + i0 + nq + kKTile - 1) / kKTile;   // keys [0, c0 + i0 + nq) are seen

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15;
  const int grp = lane >> 4;
  const int wq0 = i0 + 32 * wave;                      // first query of this wave
  const bool wactive = wq0 < p.t_q;
  const int wlim = c0 + min(wq0 + 32, p.t_q);          // this wave's queries see keys [0, wlim)
  const int wmin = c0 + wq0 + 1;                       // ... and all of them keys [0, wmin)

  // The query rows as B operands of the score product (column = query
  // r16 of block qb, 8 elements 32c + 8grp .. of the row), and their limits.
  u32x4 qf[2][NC];
  int lim[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int iq = wq0 + 16 * qb + r16;
    lim[qb] = c0 + iq + 1;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qf[qb][c] = u32x4{0u, 0u, 0u, 0u};
      if (iq < p.t_q)
        qf[qb][c] = *reinterpret_cast<const u32x4*>(
            p.q + ((((static_cast<int64_t>(b) * p.t_q + iq) * p.n_q + h) * D) + 32 * c + 8 * grp) * 2);
    }
  }

  const int64_t uoff = b * p.sb + g * p.sh;
  const uint32_t st = static_cast<uint32_t>(p.st);
  const u32x4 kw = rsrc_words(p.k + uoff, static_cast<uint32_t>(n) * st);
  const u32x4 vw = rsrc_words(p.v + uoff, static_cast<uint32_t>(n) * st);

  // Tiles go from memory straight to LDS (buffer loads to LDS: lane l of a
  // load writes the 16 bytes at the load's LDS base + 16 l), with no
  // registers or stores in between: load i of wave w fills chunk positions
  // 64 (NLD w + i) + lane of the tile, i.e. row / chunk position (q / CPR,
  // q % CPR), from the row's chunk q % CPR ^ tile_swz(row). Rows past the
  // block's end read as zeros.
  const uint32_t smem_lds = KVC_LDS_ADDR(smem);
  auto load_tile = [&](int t, int buf) {
    const uint32_t base = static_cast<uint32_t>(t * kKTile) * st;
    const uint32_t kb = smem_lds + buf * 2 * kTileBytes;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int m = wave * NLD + i;
      const int q = m * 64 + lane;
      const int row = q / CPR;
      const uint32_t off = base + static_cast<uint32_t>(row) * st + static_cast<uint32_t>((q % CPR) ^ tile_swz(row)) * 16u;
      lds_load16<false>(kw, off, kb + m * 1024);
      lds_load16<false>(vw, off, kb + kTileBytes + m * 1024);
    }
  };

  // Per query: the reference r (log2 domain) the weights are taken against,
  // exp2(score - r). It moves only when a score passes r + 8, so weights stay
  // below 2^8 and the accumulators are rescaled only in those (rare) tiles.
  constexpr float kLazy = 8.f;
  float mrun[2] = {-INFINITY, -INFINITY};
  float lrun[2] = {0.f, 0.f};               // this lane's part of the running sum
  f32x4 o[2][ND];                           // O^T: lane holds elements 16db + 4grp + i of query r16
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < ND; ++db) o[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Per-lane parts of the LDS addresses: K row r16's chunk 4c + grp sits at
  // (4c + grp) ^ swz (swz of the row: 16 kb + r16 has r16's low bits); a V
  // read of keys 4 grp + r16 / 4 (+ 32 kc, + 16) takes elements
  // 16 db + 4 (r16 % 4) .., chunk 2 db + (r16 % 4) / 2 ^ vsw, byte vsub.
  const int kswz = tile_swz(r16);
  const int vrow = 4 * grp + (r16 >> 2);
  const int vx = ((r16 & 3) >> 1) ^ tile_swz(vrow);
  const int voff = vrow * RB + 8 * (r16 & 1);
  auto compute = [&](int t, int buf, auto mask_tag) {
    constexpr bool kMask = decltype(mask_tag)::value;   // the tile crosses the diagonal
    const char* const sk = smem + buf * 2 * kTileBytes;
    const char* const sv = sk + kTileBytes;
    f32x4 s[2][4];                          // S^T: lane holds keys 16kb + 4grp + i of query r16
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) s[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Raised wave priority for the score products, back to normal for the
    // softmax: measured 1-2.5 % faster (the other wave's arithmetic then
    // fills the matrix cores' gaps rather than the reverse).
    __builtin_amdgcn_s_setprio(2);
    // K slices of block kb + 1 are requested while block kb's products run
    u32x4 ka[2][NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
      ka[0][c] = *reinterpret_cast<const u32x4*>(sk + r16 * RB + ((4 * c + grp) ^ kswz) * 16);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      if (kb + 1 < 4) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
          ka[(kb + 1) & 1][c] =
              *reinterpret_cast<const u32x4*>(sk + (16 * (kb + 1) + r16) * RB + ((4 * c + grp) ^ kswz) * 16);
      }
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) s[qb][kb] = ET::mfma(ka[kb & 1][c], qf[qb][c], s[qb][kb]);
    }
    // issue order: NC slice reads, then (NC reads, 2 NC products) per block
    // (masks: 0x100 LDS reads, 0x008 matrix-core products)
    __builtin_amdgcn_sched_group_barrier(0x100, NC, 0);
#pragma unroll
    for (int kb = 0; kb < 3; ++kb) {
      __builtin_amdgcn_sched_group_barrier(0x100, NC, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * NC, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * NC, 0);
    const float c = p.scale_log2;
    __builtin_amdgcn_s_setprio(0);
    u32x4 phi[2][2], plo[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;                  // raw scores: the scale is positive
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (kMask)
            s[qb][kb][i] = (t * kKTile + 16 * kb + 4 * grp + i < lim[qb]) ? s[qb][kb][i] : -INFINITY;
          mx = fmaxf(mx, s[qb][kb][i]);
        }
      if (__any(mx * c > mrun[qb] + kLazy)) {   // wave-uniform; every tile at first
        mx = fmaxf(mx, __shfl_xor(mx, 16));    // the query's maximum over its four lanes
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float ms = mx * c;
        const bool up = ms > mrun[qb] + kLazy;   // the four lanes of a query agree
        const float alpha = !up ? 1.f : (mrun[qb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun[qb] - ms));
        mrun[qb] = up ? ms : mrun[qb];
        lrun[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[qb][db][i] *= alpha;
      }
      const float nr = -mrun[qb];
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        float e[8];                          // slots 8grp .. 8grp+7 of this 32-key chunk
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          e[j] = __builtin_amdgcn_exp2f(fmaf(s[qb][2 * kc + (j >> 2)][j & 3], c, nr));   // masked: 0
          lrun[qb] += e[j];
        }
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) ET::split(e[2 * w], e[2 * w + 1], hi[w], lo[w]);
        phi[qb][kc] = u32x4{hi[0], hi[1], hi[2], hi[3]};
        plo[qb][kc] = u32x4{lo[0], lo[1], lo[2], lo[3]};
      }
    }
    // V^T operands k = 2 db + kc: rows 16 db + r16, keys 32 kc + 4 grp .. + 3
    // and 32 kc + 16 + 4 grp .. + 3 (the slots of the weights' lane layout),
    // two transposing reads each, requested kVAhead operands ahead of their
    // products. Each operand's four products take the high parts of both
    // query blocks, then the low parts (no product waits on the one before).
    constexpr int NV = 2 * ND;
    constexpr int kVAhead = 2;
    auto read_v = [&](int k) -> u32x4 {
      const char* const vp = sv + 32 * (k & 1) * RB + voff + ((2 * (k >> 1)) ^ vx) * 16;
      const u32x2 lo4 = lds_read_tr(vp), hi4 = lds_read_tr(vp + 16 * RB);
      return u32x4{lo4[0], lo4[1], hi4[0], hi4[1]};
    };
    u32x4 va[kVAhead + 1];
#pragma unroll
    for (int k = 0; k < kVAhead; ++k) va[k] = read_v(k);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if (k + kVAhead < NV) va[(k + kVAhead) % (kVAhead + 1)] = read_v(k + kVAhead);
      const u32x4 a = va[k % (kVAhead + 1)];
      const int db = k >> 1, kc = k & 1;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) o[qb][db] = ET::mfma(a, phi[qb][kc], o[qb][db]);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) o[qb][db] = ET::mfma(a, plo[qb][kc], o[qb][db]);
    }
    // issue order: the first kVAhead operands' reads, then (the reads of
    // operand k + kVAhead, the four products of operand k); with the
    // compiler's own order the products of each operand waited for its reads
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kVAhead, 0);
#pragma unroll
    for (int k = 0; k < NV - kVAhead; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * kVAhead, 0);
  };

  // Tiles below t_split hold no key past any query's limit; the others are
  // computed with the mask. (Two loops, one kind of tile each, so that each
  // is compiled on its own.)
  const int t_split = (c0 + i0 + 1) / kKTile;
  // A step waits for this wave's loads of tile t, then the barrier: every
  // wave's loads of tile t have landed, and every wave is done with tile
  // t - 1, whose buffer then takes tile t + 1's loads (issued for every
  // step, past the last tile too: loads under a branch would make the
  // compiler wait for all loads in flight) while tile t is computed.
  auto step = [&](int t, auto mask_tag) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    load_tile(t + 1, (t + 1) & 1);
    if (wactive && t * kKTile < wlim) compute(t, t & 1, mask_tag);
  };
  load_tile(0, 0);
  // The query registers, used here so that the compiler waits for their
  // loads once, ahead of the loop: a wait it placed in the loop would count
  // only the loads it knows of, not the tile loads, and so wait for those.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int c = 0; c < NC; ++c) asm volatile("" ::"v"(qf[qb][c]));
  int t = 0;
  for (; t < t_split; ++t) step(t, std::false_type{});
  for (; t < n_tiles; ++t) step(t, std::true_type{});
  if (!wactive) return;

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float l = lrun[qb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const float inv = 1.f / l;
    const int iq = wq0 + 16 * qb + r16;
    if (iq < p.t_q) {
      const int64_t row = ((static_cast<int64_t>(b) * p.t_q + iq) * p.n_q + h) * D;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = o[qb][db][i] * inv;
          const int64_t idx = row + 16 * db + 4 * grp + i;
          if (p.out_f32) static_cast<float*>(p.out)[idx] = x;
          else ET::store(p.out, idx, x);
        }
    }
  }
}

typedef void (*PrefillKernel)(const PrefillParams);

PrefillKernel pick_prefill_kernel(int32_t dtype, int32_t d) {
  if (dtype == KVC_BF16 && d == 128) return prefill_kernel<Bf16P, 128>;
  if (dtype == KVC_BF16 && d == 64) return prefill_kernel<Bf16P, 64>;
  if (dtype == KVC_F16 && d == 128) return prefill_kernel<F16P, 128>;
  if (dtype == KVC_F16 && d == 64) return prefill_kernel<F16P, 64>;
  return nullptr;
}

}  // namespace

bool kvc::prefill_supported(int32_t dtype, int32_t head_dim) { return pick_prefill_kernel(dtype, head_dim) != nullptr; }

kvc_status_t kvc::launch_prefill(const kvc_cache_t* cache, const int32_t* seq_lens, int32_t t_q, const void* q,
                                 int32_t n_q_heads, float scale, void* out, int32_t out_dtype, uint32_t* dev_status,
                                 hipStream_t stream, bool check_only) {
  kvc_status_t st = kvc::check_cache(cache, true);
  if (st != KVC_OK) return st;
  if (n_q_heads <= 0 || n_q_heads % cache->n_kv_heads != 0) return KVC_ERR_GQA;
  if (t_q <= 0) return KVC_ERR_SHAPE;
  if (out_dtype != KVC_F32 && out_dtype != cache->dtype) return KVC_ERR_DTYPE;
  PrefillKernel kern = pick_prefill_kernel(cache->dtype, cache->head_dim);
  if (kern == nullptr) return KVC_ERR_UNSUPPORTED;
  const float scale_log2 = scale * 1.44269504088896340736f;  // log2(e)
  if (!(scale > 0.f) || !(scale_log2 < INFINITY)) return KVC_ERR_UNSUPPORTED;
  if (cache->batch == 0) return KVC_OK;
  if (seq_lens == nullptr || q == nullptr || out == nullptr) return KVC_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(q) % 16) return KVC_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(out) % kvc::elem_bytes(out_dtype)) return KVC_ERR_ALIGN;
  const int s = kvc::elem_bytes(cache->dtype);
  // one (sequence, KV head) slice is addressed with 32-bit byte offsets,
  // plus up to one tile past its end (read back as zeros)
  if ((static_cast<int64_t>(cache->max_len) + kKTile) * cache->stride_t * s > 0x7fffffffll) return KVC_ERR_SHAPE;
  const int64_t n_qt = (static_cast<int64_t>(t_q) + kQTile - 1) / kQTile;
  const int64_t units = static_cast<int64_t>(cache->batch) * cache->n_kv_heads;
  const int64_t group = n_q_heads / cache->n_kv_heads;
  const bool xcd_major = units % 8 == 0;                // ids map to units XCD by XCD (see the kernel)
  const int64_t wgs = units * group * n_qt;
  if (wgs > 0x7fffffffll || static_cast<int64_t>(t_q) * n_q_heads > (1ll << 30)) return KVC_ERR_SHAPE;
  if (check_only) return KVC_OK;                      // every check done, nothing enqueued

  PrefillParams p;
  p.k = static_cast<const char*>(cache->k);
  p.v = static_cast<const char*>(cache->v);
  p.sb = cache->stride_b * s;
  p.sh = cache->stride_h * s;
  p.st = cache->stride_t * s;
  p.seq_lens = seq_lens;
  p.q = static_cast<const char*>(q);
  p.out = out;
  p.status = dev_status;
  p.batch = cache->batch;
  p.n_q = n_q_heads;
  p.n_kv = cache->n_kv_heads;
  p.group = static_cast<int32_t>(group);
  p.t_q = t_q;
  p.max_len = cache->max_len;
  p.n_qt = static_cast<int32_t>(n_qt);
  p.out_f32 = out_dtype == KVC_F32 ? 1 : 0;
  p.xcd_major = xcd_major ? 1 : 0;
  p.scale_log2 = scale_log2;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(wgs)), dim3(256), 0, stream, p);
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

extern "C" kvc_status_t kvc_prefill_attn(const kvc_cache_t* cache, const int32_t* seq_lens, int32_t t_q,
                                         const void* q, int32_t n_q_heads, float scale, void* out, int32_t out_dtype,
                                         uint32_t* dev_status, hipStream_t stream) {
  return kvc::launch_prefill(cache, seq_lens, t_q, q, n_q_heads, scale, out, out_dtype, dev_status, stream, false);
}
