"""fp64 reference for KV append, prefill fill and single-query decode attention.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py. Written as plain numpy loops so it can be checked
against the pages by eye; no blocking, no online softmax, no splitting.

Page tags ([KVG], [W1D4], [LA11]) are defined in this package's ``__init__``.
"""

from __future__ import annotations

import math

import numpy as np


def widen(x) -> np.ndarray:
    """Exact widening of stored values to fp64.

    Accepts a numpy array or a torch tensor of fp32/fp16/bf16; every such value
    is exactly representable in fp64, so nothing is rounded here.
    """
    if hasattr(x, "detach"):  # torch tensor, possibly bf16 (numpy has no bf16)
        import torch
        return x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def kv_head_of(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    """KV head that query head ``h`` reads.

    [W1D4 §2.3, §3.4]: with h query heads in G groups, query head j uses K/V head
    floor(j / (h/G)); this is the grouping repeat_interleave produces
    ([KVG] runnable experiment, expand_kv). MHA is n_kv == n_q, MQA is n_kv == 1.
    """
    if n_kv_heads <= 0 or n_q_heads % n_kv_heads != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    return h // (n_q_heads // n_kv_heads)


def append(k_cache, v_cache, seq_lens, k_new, v_new):
    """Write one new token per sequence into a preallocated cache.

    [W1D4 §3.1] KVCache.update: the cache is allocated once to max_len and the
    T new tokens go to slots [pos, pos+T); here T = 1 and each sequence b has its
    own pos = seq_lens[b] (the ragged form of the capacity formula in [KVG]
    "capacity formula"). [KVG] "two equivalent decode paths": the append is an
    in-place slot write; every other slot stays as it was.

    Arrays may be of any dtype (use integer views for a bitwise model of bf16).
    k_cache, v_cache: [B, H_kv, T_max, D]; k_new, v_new: [B, H_kv, D].
    Returns (k_out, v_out, overflow) where overflow[b] is True when slot
    seq_lens[b] lies outside [0, T_max): that sequence is then left untouched.
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    batch, _, t_max, _ = k_out.shape
    overflow = np.zeros(batch, dtype=bool)
    for b in range(batch):
        pos = int(seq_lens[b])
        if pos < 0 or pos >= t_max:
            overflow[b] = True
            continue
        k_out[b, :, pos, :] = k_new[b]
        v_out[b, :, pos, :] = v_new[b]
    return k_out, v_out, overflow


def prefill_fill(k_cache, v_cache, seq_lens, k, v):
    """Write T_new tokens per sequence at slots [seq_lens[b], seq_lens[b]+T_new).

    [W1D4 §3.1] KVCache.update with T = T_new (prefill, or a prompt fed in chunks
    when seq_lens[b] > 0, [W1D4 §3.5] test 1). k, v: [B, H_kv, T_new, D].
    A sequence whose range does not fit in [0, T_max) is left untouched and
    flagged.
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    batch, _, t_max, _ = k_out.shape
    t_new = k.shape[2]
    overflow = np.zeros(batch, dtype=bool)
    for b in range(batch):
        pos = int(seq_lens[b])
        if pos < 0 or pos + t_new > t_max:
            overflow[b] = True
            continue
        for i in range(t_new):
            k_out[b, :, pos + i, :] = k[b, :, i, :]
            v_out[b, :, pos + i, :] = v[b, :, i, :]
    return k_out, v_out, overflow


def decode_attention(q, k_cache, v_cache, seq_lens, n_pending: int = 1, scale=None):
    """Single new query per head attending every cached token, in fp64.

    [LA11 §2.2] single-step decode: after k_t, v_t are appended,
    s_t = q_t K^T * scale and o_t = softmax(s_t) V over all cached tokens.
    [KVG] decode_one / [W1D4 §1.3]: one query per head, no mask (every cached
    token precedes the query). The page's garbled formula lost the square root
    of the divisor; the glossary's code divides by sqrt(head_dim), which is the
    default here. [W1D4 §3.4] query head h reads KV head floor(h / (H_q/H_kv)).

    q: [B, H_q, D]; caches [B, H_kv, T_max, D]; each sequence b attends its
    first N_b = seq_lens[b] + n_pending slots. Softmax is the two-pass textbook
    form: max, exponentials, sum, weighted sum of V, divide. A sequence with
    N_b == 0 gives a zero row (softmax over an empty set has no value).
    Returns fp64 [B, H_q, D].
    """
    q = widen(q)
    k = widen(k_cache)
    v = widen(v_cache)
    batch, n_q, d = q.shape
    n_kv, t_max = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((batch, n_q, d), dtype=np.float64)
    for b in range(batch):
        n = int(seq_lens[b]) + int(n_pending)
        if n > t_max:
            raise ValueError(f"sequence {b} attends {n} tokens but the cache holds {t_max}")
        if n <= 0:
            continue
        for h in range(n_q):
            g = kv_head_of(h, n_q, n_kv)
            keys = k[b, g, :n, :]
            vals = v[b, g, :n, :]
            scores = (keys @ q[b, h]) * scale          # [N]
            m = scores.max()
            e = np.exp(scores - m)
            out[b, h] = (e @ vals) / e.sum()
    return out


def chunk_attention(q, k_cache, v_cache, seq_lens, scale=None):
    """Several new queries per sequence attending the cache, in fp64.

    A prefill chunk or a speculative verify step: T new tokens have been
    appended after seq_lens[b] cached ones, and each of their queries attends
    with the causal mask aligned to the lower right. [W1D4 §3.3] masks: a
    block of T queries against S keys sees keys 0..S - T + i for query i
    (a top-left alignment, as SDPA's is_causal uses, would hide cached keys
    from the block). With T = 1 this is the single-query decode of
    [LA11 §2.2]; with nothing cached before the block it is the full causal
    prefill of [KVG] path A. Scale and GQA grouping as in decode_attention.

    q: [B, T, H_q, D] (token-major, as a chunk's projections come out);
    caches [B, H_kv, T_max, D] already holding the block's rows at slots
    [seq_lens[b], seq_lens[b] + T). Query i of sequence b attends slots
    0..seq_lens[b] + i with the two-pass softmax. Returns fp64 [B, T, H_q, D].
    """
    q = widen(q)
    k = widen(k_cache)
    v = widen(v_cache)
    batch, t_q, n_q, d = q.shape
    n_kv, t_max = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((batch, t_q, n_q, d), dtype=np.float64)
    for b in range(batch):
        base = int(seq_lens[b])
        if base < 0 or base + t_q > t_max:
            raise ValueError(f"sequence {b}: block [{base}, {base + t_q}) does not fit a cache of {t_max}")
        for i in range(t_q):
            n = base + i + 1                          # keys 0 .. seq_lens[b] + i
            for h in range(n_q):
                g = kv_head_of(h, n_q, n_kv)
                scores = (k[b, g, :n, :] @ q[b, i, h]) * scale
                m = scores.max()
                e = np.exp(scores - m)
                out[b, i, h] = (e @ v[b, g, :n, :]) / e.sum()
    return out


def causal_attention(q, k, v, n_q_heads: int, n_kv_heads: int, scale=None):
    """Full causal self-attention over a prefix ("path A" of [KVG]).

    [KVG] prefill: scores = q K^T / sqrt(D) plus an upper-triangular -inf mask
    (row i sees keys 0..i), softmax along the keys, times V. GQA heads map as
    in ``kv_head_of``. q: [H_q, T, D]; k, v: [H_kv, T, D]. Returns [H_q, T, D].
    """
    q = widen(q)
    k = widen(k)
    v = widen(v)
    _, t, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros_like(q)
    mask = np.triu(np.full((t, t), -np.inf), 1)
    for h in range(n_q_heads):
        g = kv_head_of(h, n_q_heads, n_kv_heads)
        s = (q[h] @ k[g].T) * scale + mask              # [T, T]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        p = e / e.sum(axis=1, keepdims=True)
        out[h] = p @ v[g]
    return out


def project(x, w, n_heads: int, head_dim: int):
    """Per-token projection x @ W split into heads, in fp64.

    [KVG] runnable experiment, project: (x @ W) viewed as (tokens, heads, D) and
    transposed so that head h owns columns [h*D, (h+1)*D). x: [T, hidden];
    returns [n_heads, T, D]. Rows are independent, so a longer prefix leaves
    the earlier rows unchanged ([W1D4 §1.2]).
    """
    x = widen(x)
    w = widen(w)
    # one row at a time, so a row's bits never depend on how many rows a BLAS
    # call was given (the invariant above is then exact, not up to rounding)
    y = np.stack([row @ w for row in x])
    return y.reshape(x.shape[0], n_heads, head_dim).transpose(1, 0, 2)


def _merge_heads(ctx_last):
    """[H_q, D] context of one position -> [H_q * D] (head-major), as the page's
    transpose(1, 2).reshape does before the output projection."""
    return ctx_last.reshape(-1)


def toy_path_a(x, wq, wk, wv, wo, n_q: int, n_kv: int, head_dim: int, n_prompt: int):
    """Path A of [KVG] "two equivalent decode paths": at every decode step the
    whole prefix is projected again and run through causal attention; only the
    last position's output is kept, then multiplied by W_o.

    x: [T_total, hidden] (one sequence). Returns (outputs [n_dec, hidden],
    contexts [n_dec, H_q, D]).
    """
    x = widen(x)
    wo = widen(wo)
    outputs, contexts = [], []
    for t in range(n_prompt, x.shape[0]):
        prefix = x[: t + 1]
        q = project(prefix, wq, n_q, head_dim)
        k = project(prefix, wk, n_kv, head_dim)
        v = project(prefix, wv, n_kv, head_dim)
        ctx = causal_attention(q, k, v, n_q, n_kv)[:, -1, :]
        contexts.append(ctx)
        outputs.append(_merge_heads(ctx) @ wo)
    return np.stack(outputs), np.stack(contexts)


def toy_path_b(x, wq, wk, wv, wo, n_q: int, n_kv: int, head_dim: int, n_prompt: int):
    """Path B of [KVG]: prefill the prompt's K/V once into a preallocated cache
    ([W1D4 §3.1]), then per token project only the new position, append its
    k, v, and let its q attend the whole cache ([W1D4 §1.3]).

    Returns (outputs [n_dec, hidden], contexts [n_dec, H_q, D], k_cache, v_cache)
    with caches [1, H_kv, T_total, D] in fp64.
    """
    x = widen(x)
    wo = widen(wo)
    t_total = x.shape[0]
    k_cache = np.zeros((1, n_kv, t_total, head_dim))
    v_cache = np.zeros((1, n_kv, t_total, head_dim))
    seq_lens = np.array([0])
    kp = project(x[:n_prompt], wk, n_kv, head_dim)[None]
    vp = project(x[:n_prompt], wv, n_kv, head_dim)[None]
    k_cache, v_cache, ovf = prefill_fill(k_cache, v_cache, seq_lens, kp, vp)
    assert not ovf.any()
    seq_lens = seq_lens + n_prompt
    outputs, contexts = [], []
    for t in range(n_prompt, t_total):
        row = x[t: t + 1]
        q = project(row, wq, n_q, head_dim)[:, 0, :][None]      # [1, H_q, D]
        k_new = project(row, wk, n_kv, head_dim)[:, 0, :][None]  # [1, H_kv, D]
        v_new = project(row, wv, n_kv, head_dim)[:, 0, :][None]
        k_cache, v_cache, ovf = append(k_cache, v_cache, seq_lens, k_new, v_new)
        assert not ovf.any()
        ctx = decode_attention(q, k_cache, v_cache, seq_lens, n_pending=1)[0]
        contexts.append(ctx)
        outputs.append(_merge_heads(ctx) @ wo)
        seq_lens = seq_lens + 1
    return np.stack(outputs), np.stack(contexts), k_cache, v_cache


# ------------------------------------------------------- sliding window --
#
# [W1D4 §2.7] sliding-window attention (Mistral): every layer attends only the
# most recent W tokens, so its cache is capped at W; [W1D4 §1.6]: with RoPE
# the positions stay baked into the cached K, so the window can roll over a
# fixed buffer without rebuilding it; [KVG] "与上下游术语的关系": this caps the
# read length only because the layer itself limits what it sees (it is not a
# lossless truncation of full attention). Here the cache of a window-W layer
# has W slots; token number t of a sequence (t counted from 0 over its whole
# history) lives in slot t % W, overwriting token t - W.


def ring_slot(t: int, window: int) -> int:
    """Slot of token number t in a ring of `window` slots."""
    return t % window


def ring_append(k_cache, v_cache, seq_lens, k_new, v_new):
    """Write token number seq_lens[b] of each sequence into slot
    seq_lens[b] % W of its ring (W = the cache's T_max), overwriting the token
    W positions older. Arrays [B, H_kv, W, D]; k_new, v_new [B, H_kv, D]. A
    negative count leaves the sequence untouched. Returns (k', v')."""
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    window = k_out.shape[2]
    for b in range(k_out.shape[0]):
        t = int(seq_lens[b])
        if t < 0:
            continue
        s = ring_slot(t, window)
        k_out[b, :, s, :] = np.asarray(k_new)[b]
        v_out[b, :, s, :] = np.asarray(v_new)[b]
    return k_out, v_out


def ring_decode_attention(q, k_cache, v_cache, seq_lens, n_pending: int = 1, scale=None):
    """Decode with a sliding window of W = the cache's T_max slots: each
    sequence attends its most recent min(seq_lens[b] + n_pending, W) tokens,
    which occupy slots [0, min(seq_lens[b] + n_pending, W)) of the ring in
    rotated order. With no mask the result does not depend on the order of
    the (key, value) rows (pinned by the permutation test), so this is the
    single-query decode over those slots."""
    window = np.asarray(widen(k_cache)).shape[2]
    n = [min(max(int(x), 0) + n_pending, window) for x in seq_lens]
    return decode_attention(q, k_cache, v_cache, np.array(n) - n_pending, n_pending=n_pending, scale=scale)


# ------------------------------------------------------------ paged cache --
#
# [KVG] "与上下游术语的关系" and the note under the slot figure, [W1D4] §1.6
# (fragmentation) and [LA11] §8 (optimisation table): a paged cache stores
# the same logical K/V sequence in fixed-size physical pages addressed
# through a per-sequence page table, so that storage need not be contiguous;
# it does not change the logical sequence or the attention result. Here the
# pool is [n_pages, H_kv, P, D] and logical slot t of sequence b lives in
# page block_table[b][t // P] at row t % P. The pages leave the page size
# open; the library takes any multiple of 16 tokens.


def paged_slot(block_table, b: int, t: int, page_size: int):
    """(physical page, row in page) of logical slot t of sequence b."""
    return int(block_table[b][t // page_size]), t % page_size


def paged_view(pages, block_table, n_tokens: int, lengths=None):
    """Logical cache [B, H_kv, n_tokens, D] gathered from a page pool
    [n_pages, H_kv, P, D] through block_table [B, pages per sequence]; with
    `lengths`, sequence b gathers only its first lengths[b] slots (the rest
    stay zero, and their table entries are not read)."""
    pages = np.asarray(pages)
    batch = len(block_table)
    n_pages, n_kv, page_size, d = pages.shape
    out = np.zeros((batch, n_kv, n_tokens, d), dtype=pages.dtype)
    for b in range(batch):
        n_b = n_tokens if lengths is None else min(n_tokens, max(int(lengths[b]), 0))
        for t in range(n_b):
            pg, r = paged_slot(block_table, b, t, page_size)
            if not 0 <= pg < n_pages:
                raise IndexError(f"sequence {b} slot {t}: page {pg} is not in the pool")
            out[b, :, t, :] = pages[pg, :, r, :]
    return out


def paged_prefill_fill(k_pages, v_pages, block_table, seq_lens, k, v):
    """Write T_new tokens per sequence at logical slots [seq_lens[b],
    seq_lens[b] + T_new) through the page table ([W1D4 §3.1] update, paged).
    A sequence whose block passes the table's capacity is left untouched;
    a row whose table entry is not a valid pool index is not written. Both
    are reported in `flagged`. k, v: [B, H_kv, T_new, D].
    Returns (k_pages', v_pages', flagged)."""
    k_out = np.array(k_pages, copy=True)
    v_out = np.array(v_pages, copy=True)
    n_pages, _, page_size, _ = k_out.shape
    batch, _, t_new, _ = np.asarray(k).shape
    cap = len(block_table[0]) * page_size if batch else 0
    flagged = np.zeros(batch, dtype=bool)
    for b in range(batch):
        pos = int(seq_lens[b])
        if pos < 0 or pos + t_new > cap:
            flagged[b] = True
            continue
        for i in range(t_new):
            pg, r = paged_slot(block_table, b, pos + i, page_size)
            if not 0 <= pg < n_pages:
                flagged[b] = True
                continue
            k_out[pg, :, r, :] = np.asarray(k)[b, :, i, :]
            v_out[pg, :, r, :] = np.asarray(v)[b, :, i, :]
    return k_out, v_out, flagged


def paged_append(k_pages, v_pages, block_table, seq_lens, k_new, v_new):
    """One new token per sequence into the paged cache (k_new, v_new:
    [B, H_kv, D]); see paged_prefill_fill."""
    return paged_prefill_fill(k_pages, v_pages, block_table, seq_lens,
                              np.asarray(k_new)[:, :, None, :], np.asarray(v_new)[:, :, None, :])


def paged_decode_attention(q, k_pages, v_pages, block_table, seq_lens, n_pending: int = 1, scale=None):
    """decode_attention over the logical cache the page table describes."""
    lengths = [max(int(x), 0) + n_pending for x in seq_lens]
    n = max(lengths) if lengths else 0
    k = paged_view(widen(k_pages), block_table, n, lengths)
    v = paged_view(widen(v_pages), block_table, n, lengths)
    return decode_attention(q, k, v, seq_lens, n_pending=n_pending, scale=scale)


def cache_bytes(n_layers: int, n_kv_heads: int, head_dim: int, elem_bytes: int, lengths) -> int:
    """Logical K+V payload in bytes.

    [KVG] capacity formula (ragged form 2*L*H_kv*D*s*sum_i T_i); [W1D4 §1.4];
    [LA11 §2.3] (elements 2*B*H_kv*T*d_k, times bytes per element, times L).
    The leading 2 counts K and V.
    """
    total_tokens = sum(int(t) for t in lengths)
    return 2 * n_layers * n_kv_heads * head_dim * elem_bytes * total_tokens


def concat_append_positions(n_tokens: int) -> int:
    """Token positions moved when a cache grows by concatenation, one token per
    step: step t copies the t-1 old positions plus the new one ([W1D4 §3.1],
    the pages' anti-pattern)."""
    moved = 0
    length = 0
    for _ in range(n_tokens):
        length += 1
        moved += length
    return moved


def prealloc_append_positions(n_tokens: int) -> int:
    """Token positions written when the cache is preallocated: one per step."""
    written = 0
    for _ in range(n_tokens):
        written += 1
    return written


# ------------------------------------------------------------ quantized KV --
#
# [LA11] §3.1 (the second counterfactual) and §8 (the table of optimisations):
# the usual compromise keeps weights in fp16, stores the cache as fp8 or int8
# and accumulates the softmax in fp32; quantising the cache cuts the bytes each
# decode step reads, at some loss of precision. [KVG] "MHA、GQA、MLA 与量化如何
# 改变容量": the real saving also depends on the scale granularity (per token,
# head or group), zero points and packing, and it shrinks if the kernel widens
# the cache back to 16 bits in memory before using it. The pages fix no format;
# this oracle takes the following one (the library implements the same):
#   * one fp32 scale per (sequence, KV head, token) for K and another for V:
#     scale = amax / QMAX, an fp32 division, where amax is the largest |x| over
#     that token's D values of that head and QMAX is 127 (int8) or 448 (the
#     largest finite fp8 e4m3 value);
#   * code = encode(x / scale), the quotient an fp32 division; int8 rounds
#     half to even and clamps to [-127, 127]; fp8 is the OCP 8-bit format
#     E4M3 (bias 7, no infinities, S.1111.111 is NaN), rounded to nearest even
#     and saturating at +-448;
#   * a row of zeros has scale 0 and all codes 0;
#   * the value a code stands for is code * scale, and attention runs on those
#     values exactly as decode_attention does.
# Symmetric codes, no zero point: projected keys and values are centred on
# zero, and one scale per row then suffices. Codes are held as bytes (int8 as
# two's complement), scales as float32.

QFMT_FP8_E4M3 = 0
QFMT_INT8 = 1
QMAX = {QFMT_FP8_E4M3: 448.0, QFMT_INT8: 127.0}


def _round_half_even(x: float) -> int:
    """Nearest integer, ties to even (Python's round() on a float)."""
    return int(round(x))


def e4m3_encode_one(x: float) -> int:
    """One value to its OCP E4M3 byte: round to nearest even, saturate at 448.

    The representable magnitudes are m * 2^-9 for m = 0..7 (subnormals, biased
    exponent 0) and (1 + m/8) * 2^(e-7) for biased exponents e = 1..15, except
    e = 15 with m = 7, which is NaN. Anything at or above 448 in magnitude
    (infinities included) becomes 448; NaN becomes 0x7F.
    """
    if math.isnan(x):
        return 0x7F
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0x00
    a = abs(x)
    if a >= 448.0:
        return sign | 0x7E
    if a < 2.0 ** -6:                         # subnormal spacing 2^-9
        m = _round_half_even(a * 2.0 ** 9)    # exact: a power-of-two scaling
        return sign | (0x08 if m == 8 else m)  # 8 * 2^-9 is the smallest normal
    frac, ex = math.frexp(a)                  # a = frac * 2^ex, frac in [0.5, 1)
    e = ex - 1                                # a = (2 frac) * 2^e
    m = _round_half_even(a * 2.0 ** (3 - e))  # in [8, 16]: 1.mmm scaled by 8
    if m == 16:
        e, m = e + 1, 8
    code = ((e + 7) << 3) | (m - 8)
    return sign | min(code, 0x7E)             # [448, 464) already saturated above


def e4m3_decode_one(code: int) -> float:
    """Value of an OCP E4M3 byte."""
    code = int(code) & 0xFF
    s = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def int8_encode_one(y: float) -> int:
    """Quotient to an int8 code: round half to even, clamp to [-127, 127]."""
    return max(-127, min(127, _round_half_even(y)))


def code_value(code: int, fmt: int) -> float:
    """The number a code byte stands for before scaling."""
    if fmt == QFMT_FP8_E4M3:
        return e4m3_decode_one(code)
    c = int(code) & 0xFF
    return float(c - 256 if c >= 128 else c)


def quantize_rows(x, fmt: int):
    """Quantise rows x[..., D] (values exact in fp32) to (codes uint8 [..., D],
    scales float32 [...]) with one scale per row, as defined above."""
    x32 = np.asarray(widen(x), dtype=np.float32)
    lead = x32.shape[:-1]
    codes = np.zeros(x32.shape, dtype=np.uint8)
    scales = np.zeros(lead, dtype=np.float32)
    qmax = np.float32(QMAX[fmt])
    for idx in np.ndindex(*lead):
        row = x32[idx]
        amax = np.max(np.abs(row)) if row.size else np.float32(0)
        if amax == 0:
            continue
        scale = np.float32(amax) / qmax                      # fp32 division
        scales[idx] = scale
        for i, xi in enumerate(row):
            y = float(np.float32(xi) / scale)                 # fp32 division
            if fmt == QFMT_FP8_E4M3:
                codes[idx + (i,)] = e4m3_encode_one(y)
            else:
                codes[idx + (i,)] = int8_encode_one(y) & 0xFF
    return codes, scales


def dequantize(codes, scales, fmt: int) -> np.ndarray:
    """fp64 values code * scale; codes [..., D], scales [...]."""
    c = np.asarray(codes, dtype=np.uint8)
    lut = np.array([code_value(i, fmt) for i in range(256)], dtype=np.float64)
    return lut[c] * np.asarray(scales, dtype=np.float64)[..., None]


def quant_prefill_fill(k_codes, v_codes, k_scales, v_scales, seq_lens, k, v, fmt: int):
    """Quantise T_new rows per sequence (k, v [B, H_kv, T_new, D]) into slots
    [seq_lens[b], seq_lens[b] + T_new) of a quantised cache (codes
    [B, H_kv, T_max, D] uint8, scales [B, H_kv, T_max] float32), with
    prefill_fill's rules: a sequence whose range does not fit in [0, T_max) is
    left untouched and flagged. Returns (k_codes, v_codes, k_scales, v_scales,
    overflow)."""
    kc, vc = np.array(k_codes, copy=True), np.array(v_codes, copy=True)
    ks, vs = np.array(k_scales, copy=True), np.array(v_scales, copy=True)
    batch, _, t_max, _ = kc.shape
    kq, ksq = quantize_rows(k, fmt)
    vq, vsq = quantize_rows(v, fmt)
    t_new = kq.shape[2]
    overflow = np.zeros(batch, dtype=bool)
    for b in range(batch):
        pos = int(seq_lens[b])
        if pos < 0 or pos + t_new > t_max:
            overflow[b] = True
            continue
        kc[b, :, pos:pos + t_new] = kq[b]
        vc[b, :, pos:pos + t_new] = vq[b]
        ks[b, :, pos:pos + t_new] = ksq[b]
        vs[b, :, pos:pos + t_new] = vsq[b]
    return kc, vc, ks, vs, overflow


def quant_append(k_codes, v_codes, k_scales, v_scales, seq_lens, k_new, v_new, fmt: int):
    """One new token per sequence (k_new, v_new [B, H_kv, D]) quantised into
    slot seq_lens[b]; the one-row case of quant_prefill_fill."""
    return quant_prefill_fill(k_codes, v_codes, k_scales, v_scales, seq_lens,
                              np.asarray(widen(k_new))[:, :, None, :], np.asarray(widen(v_new))[:, :, None, :], fmt)


def quant_decode_attention(q, k_codes, k_scales, v_codes, v_scales, seq_lens, fmt: int, n_pending: int = 1,
                           scale=None):
    """decode_attention over the values the quantised cache stands for."""
    return decode_attention(q, dequantize(k_codes, k_scales, fmt), dequantize(v_codes, v_scales, fmt), seq_lens,
                            n_pending=n_pending, scale=scale)
