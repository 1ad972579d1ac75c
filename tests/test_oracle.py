"""Pins for the CPU oracle: each check ties it to something other than itself.

Sources (page title and section):
  KVG  = glossary "KV 缓存" (llm-glossary.tokens-kit.com/terms/kv-cache/)
  W1D4 = "第 1 周 · Day 4：KV Cache 与 MQA / GQA" (semidirectx.com course notes)
  LA11 = "11.7 KV Cache：形状、显存与带宽" (yongzhen.wang textbook)
"""

import csv
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
UNITS = {"B": 1, "KiB": 2**10, "MiB": 2**20, "GiB": 2**30}


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        lines = [ln for ln in f if not ln.startswith("#")]
    return list(csv.DictReader(lines))


# ---------------------------------------------------------------- capacity --

@pytest.mark.parametrize("row", _rows("capacity_values.csv"), ids=lambda r: r["citation"][:48])
def test_cache_bytes_matches_printed_values(row):
    """Every cache size the pages print (tests/golden/capacity_values.csv)."""
    got = oracle.cache_bytes(int(row["n_layers"]), int(row["n_kv_heads"]), int(row["head_dim"]),
                             int(row["elem_bytes"]), [int(row["seq_len"])] * int(row["batch"]))
    want = float(row["value"]) * UNITS[row["unit"]]
    tol = float(row["rel_tol"])
    if tol == 0:
        assert got == want, row["citation"]
    else:
        assert abs(got - want) <= tol * want, (got, want, row["citation"])


def test_cache_bytes_ragged_form():
    """KVG capacity formula: a ragged batch counts sum_i T_i, not B * max T."""
    lens = [3000, 4500, 6000]
    assert oracle.cache_bytes(32, 32, 128, 2, lens) == 524288 * sum(lens)
    assert oracle.cache_bytes(32, 32, 128, 2, lens) < oracle.cache_bytes(32, 32, 128, 2, [6000] * 3)


def test_concat_versus_prealloc_positions():
    """W1D4 §3.1 (check group 8): generating 4096 tokens, concatenation moves
    about 8.39 million positions, preallocation writes 4096, about 2048x."""
    moved = oracle.concat_append_positions(4096)
    written = oracle.prealloc_append_positions(4096)
    assert written == 4096
    assert round(moved / 1e6, 2) == 8.39
    assert moved == 4096 * 4097 // 2
    assert round(moved / written) == 2048


# ------------------------------------------------------------- GQA mapping --

def test_kv_head_of_grouping():
    """W1D4 §2.3 diagram: 8 query heads, 2 KV heads -> q0..q3 read k0, q4..q7 read k1;
    MQA maps all to k0; MHA is the identity."""
    assert [oracle.kv_head_of(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [oracle.kv_head_of(h, 8, 1) for h in range(8)] == [0] * 8
    assert [oracle.kv_head_of(h, 8, 8) for h in range(8)] == list(range(8))
    with pytest.raises(ValueError):
        oracle.kv_head_of(0, 6, 4)


def _rand(shape, seed, *names, dtype="fp32"):
    return synth.normal(shape, dtype, seed, *names)


def test_gqa_equals_mha_on_repeat_interleaved_cache():
    """W1D4 §3.4 / KVG expand_kv: GQA sharing must equal MHA over K/V expanded
    with repeat_interleave (torch's op), exactly; j mod G grouping (torch.repeat)
    must differ (W1D4 §3.4 warns it raises no error)."""
    b, hq, hkv, t, d = 2, 8, 2, 11, 16
    q = _rand((b, hq, d), 1, "q")
    k = _rand((b, hkv, t, d), 1, "k")
    v = _rand((b, hkv, t, d), 1, "v")
    lens = np.array([6, 10])
    gqa = oracle.decode_attention(q, k, v, lens, n_pending=1)
    k_exp = torch.repeat_interleave(k, hq // hkv, dim=1)
    v_exp = torch.repeat_interleave(v, hq // hkv, dim=1)
    mha = oracle.decode_attention(q, k_exp, v_exp, lens, n_pending=1)
    assert np.array_equal(gqa, mha)
    wrong = oracle.decode_attention(q, k.repeat(1, hq // hkv, 1, 1), v.repeat(1, hq // hkv, 1, 1),
                                    lens, n_pending=1)
    assert np.abs(wrong - gqa).max() > 1e-3


def test_gqa_with_groups_equal_heads_is_mha():
    """W1D4 §2.3 (check group 6): G = h gives the MHA result, difference exactly 0."""
    b, h, t, d = 1, 4, 9, 8
    q = _rand((b, h, d), 2, "q")
    k = _rand((b, h, t, d), 2, "k")
    v = _rand((b, h, t, d), 2, "v")
    lens = np.array([8])
    out = oracle.decode_attention(q, k, v, lens)
    for hh in range(h):  # each head alone, as a one-head MHA problem
        one = oracle.decode_attention(q[:, hh:hh + 1], k[:, hh:hh + 1], v[:, hh:hh + 1], lens)
        assert np.array_equal(out[:, hh], one[:, 0])


# ------------------------------------------------- library routine (SDPA) --

@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (8, 1), (6, 3)])
def test_decode_attention_matches_torch_sdpa(hq, hkv):
    """Library pin: single-query attention equals torch's
    scaled_dot_product_attention (fp64, enable_gqa, which groups heads like
    repeat_interleave per W1D4 §A.3), per sequence over its N_b tokens."""
    b, t_max, d = 3, 40, 32
    q = _rand((b, hq, d), 3, "q", hq, hkv).double()
    k = _rand((b, hkv, t_max, d), 3, "k", hq, hkv).double()
    v = _rand((b, hkv, t_max, d), 3, "v", hq, hkv).double()
    lens = np.array([0, 17, 39])
    got = oracle.decode_attention(q, k, v, lens, n_pending=1)
    for i in range(b):
        n = lens[i] + 1
        ref = F.scaled_dot_product_attention(q[i:i + 1, :, None, :], k[i:i + 1, :, :n], v[i:i + 1, :, :n],
                                             enable_gqa=True)[0, :, 0, :].numpy()
        assert np.abs(got[i] - ref).max() < 1e-13


def test_decode_attention_n_pending_zero_and_scale_argument():
    """n_pending counts tokens past seq_lens; an explicit scale replaces 1/sqrt(D)."""
    b, h, t, d = 1, 2, 12, 8
    q = _rand((b, h, d), 4, "q").double()
    k = _rand((b, h, t, d), 4, "k").double()
    v = _rand((b, h, t, d), 4, "v").double()
    got = oracle.decode_attention(q, k, v, np.array([7]), n_pending=0, scale=0.3)
    ref = F.scaled_dot_product_attention(q[:, :, None], k[:, :, :7], v[:, :, :7], scale=0.3)[:, :, 0].numpy()
    assert np.abs(got - ref).max() < 1e-13


def test_causal_attention_matches_torch_sdpa():
    """Path A's causal prefill (KVG prefill with triu(-inf, 1)) equals torch's
    SDPA with is_causal=True for square T x T (both masks agree when T_q == T_k)."""
    hq, hkv, t, d = 4, 2, 13, 4
    q = _rand((hq, t, d), 5, "q").double()
    k = _rand((hkv, t, d), 5, "k").double()
    v = _rand((hkv, t, d), 5, "v").double()
    got = oracle.causal_attention(q, k, v, hq, hkv)
    ref = F.scaled_dot_product_attention(q[None], k[None], v[None], is_causal=True, enable_gqa=True)[0]
    assert np.abs(got - ref.numpy()).max() < 1e-13


def test_top_left_causal_mask_is_wrong_for_decode():
    """W1D4 §3.3: SDPA is_causal=True aligns the triangle top-left, so a single
    query sees only key 0. Decode needs no mask; the two must differ."""
    hq, t, d = 2, 9, 8
    q = _rand((1, hq, d), 6, "q").double()
    k = _rand((1, hq, t, d), 6, "k").double()
    v = _rand((1, hq, t, d), 6, "v").double()
    good = oracle.decode_attention(q, k, v, np.array([t - 1]))
    top_left = F.scaled_dot_product_attention(q[:, :, None], k, v, is_causal=True)[:, :, 0].numpy()
    assert np.abs(top_left - v[:, :, 0].numpy()).max() < 1e-15   # sees only key 0
    assert np.abs(good - top_left).max() > 1e-2


# -------------------------------------------------------------- closed forms --

def test_single_token_returns_its_value_exactly():
    """N = 1: softmax of one score is 1, so o = V_0 bit for bit."""
    q = _rand((2, 4, 8), 7, "q")
    k = _rand((2, 2, 5, 8), 7, "k")
    v = _rand((2, 2, 5, 8), 7, "v")
    out = oracle.decode_attention(q, k, v, np.array([0, 0]), n_pending=1)
    for h in range(4):
        assert np.array_equal(out[:, h], oracle.widen(v)[:, h // 2, 0])


def test_zero_query_gives_mean_of_values():
    """q = 0: every score is 0, weights are uniform, o = mean_t V_t."""
    v = _rand((1, 1, 10, 8), 8, "v").double()
    k = _rand((1, 1, 10, 8), 8, "k").double()
    out = oracle.decode_attention(torch.zeros(1, 1, 8, dtype=torch.float64), k, v, np.array([9]))
    assert np.abs(out[0, 0] - v[0, 0].numpy().mean(axis=0)).max() < 1e-15


def test_identical_keys_give_uniform_weights():
    q = _rand((1, 3, 8), 9, "q").double()
    k = _rand((1, 1, 1, 8), 9, "k").double().expand(1, 1, 6, 8).contiguous()
    v = _rand((1, 1, 6, 8), 9, "v").double()
    out = oracle.decode_attention(q, k, v, np.array([5]))
    for h in range(3):
        assert np.abs(out[0, h] - v[0, 0].numpy().mean(axis=0)).max() < 1e-15


def test_scale_pins_weights_three_to_one():
    """Closed form that fixes the 1/sqrt(D) scale and the softmax direction:
    with D = 4 (scale 1/2) and q.k0 - q.k1 = 2 ln 3, the scores differ by ln 3,
    so the weights are 3:1 and o = 0.75 v0 + 0.25 v1. Dropping the square root
    would give 9:1; dividing by D, 1.73:1; softmax of -s, 1:3."""
    d = 4
    q = np.array([[[1.0, 0.0, 0.0, 0.0]]])
    k = np.zeros((1, 1, 2, d))
    k[0, 0, 0, 0] = 2.0 * math.log(3.0)
    v = np.array([[[[1.0, 2.0, 3.0, 4.0], [5.0, -6.0, 7.0, -8.0]]]])
    out = oracle.decode_attention(q, k, v, np.array([1]))
    want = 0.75 * v[0, 0, 0] + 0.25 * v[0, 0, 1]
    assert np.abs(out[0, 0] - want).max() < 1e-14


def test_dominant_score_selects_its_value():
    d = 8
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = 1.0
    k = np.zeros((1, 1, 5, d))
    k[0, 0, 3, 0] = 200.0 * math.sqrt(d)  # score 200 against 0: weight 1 - 4e-87
    v = oracle.widen(_rand((1, 1, 5, d), 10, "v"))
    out = oracle.decode_attention(q, k, v, np.array([4]))
    assert np.abs(out[0, 0] - v[0, 0, 3]).max() < 1e-15


def test_permuting_cached_tokens_leaves_output_unchanged():
    """No mask, no positions inside the op: a joint permutation of the (K_t, V_t)
    rows changes only the summation order."""
    q = _rand((1, 4, 16), 11, "q")
    k = oracle.widen(_rand((1, 2, 20, 16), 11, "k"))
    v = oracle.widen(_rand((1, 2, 20, 16), 11, "v"))
    perm = np.random.default_rng(0).permutation(20)
    a = oracle.decode_attention(q, k, v, np.array([19]))
    b = oracle.decode_attention(q, k[:, :, perm], v[:, :, perm], np.array([19]))
    assert np.abs(a - b).max() < 1e-15


def test_weights_sum_to_one_via_constant_values():
    """If every V row is the same vector c, o = c * sum(p) = c."""
    q = _rand((1, 2, 8), 12, "q")
    k = _rand((1, 1, 30, 8), 12, "k")
    c = np.linspace(-1, 1, 8)
    v = np.broadcast_to(c, (1, 1, 30, 8)).copy()
    out = oracle.decode_attention(q, k, v, np.array([29]))
    assert np.abs(out[0] - c).max() < 1e-15


def test_empty_sequence_gives_zero_row():
    q = _rand((2, 2, 8), 13, "q")
    k = _rand((2, 2, 4, 8), 13, "k")
    v = _rand((2, 2, 4, 8), 13, "v")
    out = oracle.decode_attention(q, k, v, np.array([0, 3]), n_pending=0)
    assert np.all(out[0] == 0.0) and np.all(np.isfinite(out[1]))


def test_mpmath_brute_force_fifty_digits():
    """Brute force at 50 significant digits on tiny inputs bounds the fp64
    oracle's rounding error."""
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 50
    hq, hkv, t, d = 4, 2, 7, 5
    q = oracle.widen(_rand((1, hq, d), 14, "q"))
    k = oracle.widen(_rand((1, hkv, t, d), 14, "k"))
    v = oracle.widen(_rand((1, hkv, t, d), 14, "v"))
    got = oracle.decode_attention(q, k, v, np.array([t - 1]))
    for h in range(hq):
        g = h // (hq // hkv)
        s = [mpmath.fsum(mpmath.mpf(q[0, h, i]) * mpmath.mpf(k[0, g, j, i]) for i in range(d))
             / mpmath.sqrt(d) for j in range(t)]
        w = [mpmath.exp(x) for x in s]
        z = mpmath.fsum(w)
        for i in range(d):
            o = mpmath.fsum(w[j] * mpmath.mpf(v[0, g, j, i]) for j in range(t)) / z
            assert abs(float(o) - got[0, h, i]) < 1e-14


# ------------------------------------------------------------ append model --

def test_append_writes_one_slot_bitwise_and_nothing_else():
    """W1D4 §3.1 update with T = 1, per-sequence positions; KVG: the append is an
    in-place slot write. bf16 is modelled on its 16-bit patterns."""
    b, h, t_max, d = 3, 2, 6, 8
    kc = synth.normal((b, h, t_max, d), "bf16", 15, "kc").view(torch.int16).numpy()
    vc = synth.normal((b, h, t_max, d), "bf16", 15, "vc").view(torch.int16).numpy()
    kn = synth.normal((b, h, d), "bf16", 15, "kn").view(torch.int16).numpy()
    vn = synth.normal((b, h, d), "bf16", 15, "vn").view(torch.int16).numpy()
    lens = np.array([0, 5, 6])        # last one is full: overflow
    k2, v2, ovf = oracle.append(kc, vc, lens, kn, vn)
    assert list(ovf) == [False, False, True]
    for i, pos in enumerate(lens):
        for s in range(t_max):
            if s == pos and not ovf[i]:
                assert np.array_equal(k2[i, :, s], kn[i]) and np.array_equal(v2[i, :, s], vn[i])
            else:
                assert np.array_equal(k2[i, :, s], kc[i, :, s]) and np.array_equal(v2[i, :, s], vc[i, :, s])


def test_prefill_fill_chunked_equals_one_shot():
    """W1D4 §3.5 test 1 includes prefill in chunks: two fills at offsets 0 and 5
    give the same cache as one fill of 9 tokens; a fill past T_max is refused."""
    b, h, t_max, d = 2, 2, 12, 4
    k = oracle.widen(_rand((b, h, 9, d), 16, "k"))
    v = oracle.widen(_rand((b, h, 9, d), 16, "v"))
    empty = np.full((b, h, t_max, d), -7.0)
    k1, v1, _ = oracle.prefill_fill(empty, empty, np.zeros(b, int), k, v)
    ka, va, _ = oracle.prefill_fill(empty, empty, np.zeros(b, int), k[:, :, :5], v[:, :, :5])
    kb, vb, _ = oracle.prefill_fill(ka, va, np.full(b, 5), k[:, :, 5:], v[:, :, 5:])
    assert np.array_equal(k1, kb) and np.array_equal(v1, vb)
    _, _, ovf = oracle.prefill_fill(empty, empty, np.array([3, 4]), k, v)
    assert list(ovf) == [False, True]


def test_past_kv_rows_do_not_change_when_prefix_grows():
    """W1D4 §1.2 (check group 1): K/V of the first 12 positions are identical,
    difference exactly 0, whether the prefix has 12 or 13 tokens."""
    cfg = synth.CONFIGS["toy_gqa"]
    x = _rand((13, cfg.hidden), 17, "x")
    wk = _rand((cfg.hidden, cfg.n_kv_heads * cfg.head_dim), 17, "wk")
    k12 = oracle.project(x[:12], wk, cfg.n_kv_heads, cfg.head_dim)
    k13 = oracle.project(x[:13], wk, cfg.n_kv_heads, cfg.head_dim)
    assert np.array_equal(k12, k13[:, :12])


def test_project_head_h_owns_its_column_block():
    """KVG project: view(tokens, heads, D).transpose -> head h is columns [hD, (h+1)D)."""
    x = oracle.widen(_rand((5, 16), 18, "x"))
    w = oracle.widen(_rand((16, 12), 18, "w"))
    p = oracle.project(x, w, 3, 4)
    for h in range(3):
        assert np.abs(p[h] - x @ w[:, 4 * h: 4 * h + 4]).max() < 1e-15


# ----------------------------------------------------- path A == path B --

def _toy_inputs(cfg, seed=7, n_q=None, n_kv=None, prompt=None, decode=None):
    n_q = n_q or cfg.n_q_heads
    n_kv = n_kv or cfg.n_kv_heads
    t = (prompt or cfg.prompt) + (decode or cfg.decode)
    std = 1.0 / math.sqrt(cfg.hidden)
    wq = synth.normal((cfg.hidden, n_q * cfg.head_dim), "fp32", seed, "toy", "wq", std=std)
    wk = synth.normal((cfg.hidden, n_kv * cfg.head_dim), "fp32", seed, "toy", "wk", std=std)
    wv = synth.normal((cfg.hidden, n_kv * cfg.head_dim), "fp32", seed, "toy", "wv", std=std)
    wo = synth.normal((n_q * cfg.head_dim, cfg.hidden), "fp32", seed, "toy", "wo", std=std)
    x = synth.normal((t, cfg.hidden), "fp32", seed, "toy", "x")
    return x, wq, wk, wv, wo


def test_toy_full_recompute_equals_incremental_decode():
    """KVG runnable experiment, toy shape: B=1, hidden 16, H_q=4, H_kv=2, D=4,
    prompt 8 + 5 decode steps. Path A (full-prefix recompute) and path B
    (prefill + append + one-query attention) agree per step; the final cache is
    [1, 2, 13, 4] and its rows are the projected K/V rows."""
    cfg = synth.CONFIGS["toy_gqa"]
    x, wq, wk, wv, wo = _toy_inputs(cfg)
    out_a, ctx_a = oracle.toy_path_a(x, wq, wk, wv, wo, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.prompt)
    out_b, ctx_b, kc, vc = oracle.toy_path_b(x, wq, wk, wv, wo, cfg.n_q_heads, cfg.n_kv_heads,
                                             cfg.head_dim, cfg.prompt)
    assert out_a.shape == (cfg.decode, cfg.hidden)
    assert np.abs(out_a - out_b).max() < 1e-13
    assert np.abs(ctx_a - ctx_b).max() < 1e-13
    assert kc.shape == (1, 2, 13, 4) and vc.shape == (1, 2, 13, 4)
    assert np.array_equal(kc[0], oracle.project(x, wk, cfg.n_kv_heads, cfg.head_dim))
    assert np.array_equal(vc[0], oracle.project(x, wv, cfg.n_kv_heads, cfg.head_dim))


@pytest.mark.parametrize("n_kv", [8, 2, 1], ids=["MHA", "GQA", "MQA"])
def test_prefill_plus_decode_equals_full_forward(n_kv):
    """W1D4 §1.3 (check group 2): prefill 8 then decode 12 equals one forward
    over 20 tokens up to fp64 rounding (the page reports 3.6e-15 / 6.2e-15 /
    5.8e-15 for MHA / GQA / MQA)."""
    cfg = synth.CONFIGS["toy_gqa"]
    x, wq, wk, wv, wo = _toy_inputs(cfg, seed=20 + n_kv, n_q=8, n_kv=n_kv, prompt=8, decode=12)
    out_a, _ = oracle.toy_path_a(x, wq, wk, wv, wo, 8, n_kv, cfg.head_dim, 8)
    out_b, _, _, _ = oracle.toy_path_b(x, wq, wk, wv, wo, 8, n_kv, cfg.head_dim, 8)
    assert np.abs(out_a - out_b).max() < 5e-14


# ------------------------------------------- multi-query block (lower right) --

def _block_inputs(seed, b, t_q, hq, hkv, t_max, d):
    q = _rand((b, t_q, hq, d), seed, "cq", t_q).double()
    k = _rand((b, hkv, t_max, d), seed, "ck", t_q).double()
    v = _rand((b, hkv, t_max, d), seed, "cv", t_q).double()
    return q, k, v


@pytest.mark.parametrize("hq,hkv,t_q", [(4, 4, 3), (8, 2, 5), (8, 1, 2), (6, 3, 7)])
def test_chunk_attention_matches_sdpa_with_lower_right_mask(hq, hkv, t_q):
    """Library pin: W1D4 §3.3's mask for a block of T queries against S keys is
    ones(T, S).tril(S - T); torch SDPA (fp64, enable_gqa) with that boolean
    mask, per sequence over its S = seq_lens[b] + T keys."""
    b, t_max, d = 3, 40, 16
    q, k, v = _block_inputs(30, b, t_q, hq, hkv, t_max, d)
    lens = np.array([0, 11, t_max - t_q])
    got = oracle.chunk_attention(q, k, v, lens)
    for i in range(b):
        s = int(lens[i]) + t_q
        mask = torch.ones(t_q, s, dtype=torch.bool).tril(s - t_q)
        ref = F.scaled_dot_product_attention(q[i:i + 1].transpose(1, 2), k[i:i + 1, :, :s], v[i:i + 1, :, :s],
                                             attn_mask=mask, enable_gqa=True)[0].transpose(0, 1).numpy()
        assert np.abs(got[i] - ref).max() < 1e-13


def test_chunk_attention_with_one_query_is_decode():
    """T = 1 reduces to the single-query decode with the new token appended
    (LA11 §2.2), which the SDPA and closed-form pins above fix."""
    b, hq, hkv, t_max, d = 2, 8, 2, 30, 16
    q, k, v = _block_inputs(31, b, 1, hq, hkv, t_max, d)
    lens = np.array([5, 29])
    got = oracle.chunk_attention(q, k, v, lens)[:, 0]
    ref = oracle.decode_attention(q[:, 0], k, v, lens, n_pending=1)
    assert np.abs(got - ref).max() < 1e-15


def test_chunk_attention_with_empty_cache_is_causal_prefill():
    """Nothing cached before the block: the full causal prefill of KVG path A
    (and SDPA is_causal, since T_q == T_k there)."""
    hq, hkv, t, d = 4, 2, 13, 8
    q, k, v = _block_inputs(32, 1, t, hq, hkv, t, d)
    got = oracle.chunk_attention(q, k, v, np.array([0]))[0]          # [T, H_q, D]
    ref = oracle.causal_attention(q[0].transpose(0, 1), k[0], v[0], hq, hkv)
    assert np.abs(got - ref.transpose(1, 0, 2)).max() < 1e-14
    sd = F.scaled_dot_product_attention(q.transpose(1, 2), k, v, is_causal=True, enable_gqa=True)[0]
    assert np.abs(got - sd.transpose(0, 1).numpy()).max() < 1e-13


def test_chunked_prefill_equals_one_shot_prefill():
    """W1D4 §3.5, first must-pass test, chunked variant: a prompt prefilled in
    blocks (each attending the cache plus itself with the lower-right mask)
    gives the same rows as one causal prefill of the whole prompt."""
    hq, hkv, t, d = 8, 2, 23, 16
    q, k, v = _block_inputs(33, 1, t, hq, hkv, t, d)
    whole = oracle.chunk_attention(q, k, v, np.array([0]))
    pieces, start = [], 0
    for size in (5, 1, 9, 8):
        pieces.append(oracle.chunk_attention(q[:, start:start + size], k, v, np.array([start])))
        start += size
    assert np.abs(np.concatenate(pieces, axis=1) - whole).max() < 1e-14


def test_top_left_mask_is_wrong_for_a_cached_block():
    """W1D4 §3.3: with cached keys, SDPA is_causal=True (top-left) hides the
    cache from the block's early queries; the lower-right result differs."""
    hq, t_q, s, d = 2, 3, 10, 8
    q, k, v = _block_inputs(34, 1, t_q, hq, hq, s, d)
    good = oracle.chunk_attention(q, k, v, np.array([s - t_q]))[0]
    top_left = F.scaled_dot_product_attention(q.transpose(1, 2), k, v, is_causal=True)[0].transpose(0, 1).numpy()
    assert np.abs(top_left[0] - v[0, :, 0].numpy()).max() < 1e-15    # query 0 sees only key 0
    assert np.abs(good - top_left).max() > 1e-2


def test_chunk_attention_mpmath_fifty_digits():
    """Brute force at 50 digits on a tiny block: query i of the block sees keys
    0..S-T+i."""
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 50
    hq, hkv, t_q, base, d = 2, 1, 3, 4, 4
    q, k, v = _block_inputs(35, 1, t_q, hq, hkv, base + t_q, d)
    q, k, v = oracle.widen(q), oracle.widen(k), oracle.widen(v)
    got = oracle.chunk_attention(q, k, v, np.array([base]))
    for i in range(t_q):
        n = base + i + 1
        for h in range(hq):
            s = [mpmath.fsum(mpmath.mpf(q[0, i, h, c]) * mpmath.mpf(k[0, 0, j, c]) for c in range(d)) / mpmath.sqrt(d)
                 for j in range(n)]
            w = [mpmath.exp(x) for x in s]
            z = mpmath.fsum(w)
            for c in range(d):
                o = mpmath.fsum(w[j] * mpmath.mpf(v[0, 0, j, c]) for j in range(n)) / z
                assert abs(float(o) - got[0, i, h, c]) < 1e-14


def test_chunk_attention_rejects_blocks_that_do_not_fit():
    q, k, v = _block_inputs(36, 1, 4, 2, 2, 10, 4)
    with pytest.raises(ValueError):
        oracle.chunk_attention(q, k, v, np.array([7]))
    with pytest.raises(ValueError):
        oracle.chunk_attention(q, k, v, np.array([-1]))


# --------------------------------------------------------------- paged cache --

def test_paged_view_worked_example():
    """A page table by hand: page size 2, sequence 0 owns pages [2, 0, 3],
    sequence 1 owns [1]; logical slot t of a sequence is row t % 2 of page
    table[b][t // 2]. Values encode (page, row, d) so every gathered element
    is checked against its address."""
    n_pages, hkv, psz, d = 4, 1, 2, 3
    pages = np.array([[[[100 * p + 10 * r + c for c in range(d)] for r in range(psz)]] for p in range(n_pages)],
                     dtype=np.float64)
    table = [[2, 0, 3], [1, 1, 1]]
    got = oracle.paged_view(pages, table, 6, lengths=[6, 2])
    assert got[0, 0, :, 0].tolist() == [200, 210, 0, 10, 300, 310]
    assert got[1, 0, :, 0].tolist() == [100, 110, 0, 0, 0, 0]            # past its length: not gathered
    assert got[0, 0, 4].tolist() == [300, 301, 302]


def _paged_from_contiguous(k, v, psz, seed):
    """Scatter a contiguous cache [B, H, T, D] into a pool through a random
    permutation of pages, using paged_prefill_fill from slot 0."""
    b, h, t, d = k.shape
    per_seq = -(-t // psz)
    n_pages = b * per_seq + 3
    perm = np.random.default_rng(seed).permutation(n_pages)[:b * per_seq]
    table = perm.reshape(b, per_seq).tolist()
    kp = np.full((n_pages, h, psz, d), np.nan)
    vp = np.full((n_pages, h, psz, d), np.nan)
    kp, vp, ovf = oracle.paged_prefill_fill(kp, vp, table, np.zeros(b, dtype=int), k, v)
    assert not ovf.any()
    return kp, vp, table


def test_paged_fill_then_view_round_trips_bitwise():
    """Paging stores the same logical sequence (KVG, relation to
    PagedAttention): scatter through a page table, gather back, identical."""
    k = oracle.widen(_rand((3, 2, 37, 8), 40, "pk"))
    v = oracle.widen(_rand((3, 2, 37, 8), 40, "pv"))
    kp, vp, table = _paged_from_contiguous(k, v, 4, 41)
    assert np.array_equal(oracle.paged_view(kp, table, 37), k)
    assert np.array_equal(oracle.paged_view(vp, table, 37), v)


def test_paged_decode_equals_contiguous_decode():
    """The attention result does not depend on where pages sit in the pool."""
    b, hq, hkv, t, d = 3, 8, 2, 45, 16
    q = _rand((b, hq, d), 42, "pq")
    k = oracle.widen(_rand((b, hkv, t, d), 42, "pk"))
    v = oracle.widen(_rand((b, hkv, t, d), 42, "pv"))
    kp, vp, table = _paged_from_contiguous(k, v, 8, 43)
    lens = np.array([0, 20, 44])
    want = oracle.decode_attention(q, k, v, lens, n_pending=1)
    got = oracle.paged_decode_attention(q, kp, vp, table, lens, n_pending=1)
    assert np.array_equal(got, want)


def test_paged_append_writes_one_slot_through_the_table():
    """The new token lands in row seq_lens[b] % P of page table[b][seq_lens[b] // P];
    nothing else in the pool changes; a full table, or a page outside the
    pool, leaves the row unwritten and is reported."""
    n_pages, hkv, psz, d = 6, 2, 4, 3
    kp = np.arange(n_pages * hkv * psz * d, dtype=np.float64).reshape(n_pages, hkv, psz, d)
    vp = -kp
    table = [[5, 1], [0, 9], [2, 3]]
    kn = np.full((3, hkv, d), 7.0)
    vn = np.full((3, hkv, d), -7.0)
    k2, v2, ovf = oracle.paged_append(kp, vp, table, np.array([6, 5, 8]), kn, vn)
    assert ovf.tolist() == [False, True, True]        # page 9 is not in the pool; slot 8 is past 2 pages
    assert np.array_equal(k2[1, :, 2], kn[0]) and np.array_equal(v2[1, :, 2], vn[0])
    changed = np.argwhere(k2 != kp)
    assert {(int(p), int(r)) for p, _, r, _ in changed} == {(1, 2)}


def test_paged_fill_skips_only_the_rows_of_a_page_outside_the_pool():
    """Reading R29 (the pages leave invalid page-table entries open): a block
    of 12 rows over pages of 4, whose middle page id is outside the pool,
    still writes the 8 rows of its two valid pages; the 4 rows of the bad
    page are not written anywhere, and the sequence is reported. The other
    sequence is written in full and not reported."""
    n_pages, hkv, psz, d = 5, 1, 4, 2
    kp = np.full((n_pages, hkv, psz, d), -1.0)
    vp = np.full((n_pages, hkv, psz, d), -2.0)
    table = [[3, 7, 0], [1, 2, 4]]                      # page 7 is not in the pool of 5
    k = np.arange(2 * hkv * 12 * d, dtype=np.float64).reshape(2, hkv, 12, d)
    v = k + 1000.0
    k2, v2, flagged = oracle.paged_prefill_fill(kp, vp, table, np.array([0, 0]), k, v)
    assert flagged.tolist() == [True, False]
    assert np.array_equal(k2[3, :, :, :], k[0, :, 0:4]) and np.array_equal(v2[3], v[0, :, 0:4])
    assert np.array_equal(k2[0, :, :, :], k[0, :, 8:12]) and np.array_equal(v2[0], v[0, :, 8:12])
    for p, rows in ((1, slice(0, 4)), (2, slice(4, 8)), (4, slice(8, 12))):
        assert np.array_equal(k2[p], k[1, :, rows]) and np.array_equal(v2[p], v[1, :, rows])
    # every pool row is accounted for: sequence 0's rows 4..7 went nowhere
    written = {3, 0, 1, 2, 4}
    assert written == set(range(n_pages))
    assert not np.isin(k[0, :, 4:8], k2).any()


# ----------------------------------------------------------- sliding window --

def _ring_from_history(k_hist, v_hist, window):
    """Append a whole history token by token into a ring of `window` slots."""
    b, h, t, d = k_hist.shape
    kr = np.full((b, h, window, d), np.nan)
    vr = np.full((b, h, window, d), np.nan)
    for i in range(t):
        kr, vr = oracle.ring_append(kr, vr, np.full(b, i), k_hist[:, :, i], v_hist[:, :, i])
    return kr, vr


@pytest.mark.parametrize("t_hist,window", [(5, 8), (8, 8), (9, 8), (37, 8), (100, 16)])
def test_ring_decode_equals_attention_over_the_last_w_tokens(t_hist, window):
    """W1D4 §2.7: a window-W layer attends the most recent W tokens. After
    appending a history of T tokens one by one into a W-slot ring, the ring
    decode equals the plain decode over rows [max(0, T - W), T) of the full
    history (contiguous, in order), up to fp64 rounding order."""
    b, hq, hkv, d = 2, 8, 2, 16
    k_hist = oracle.widen(_rand((b, hkv, t_hist, d), 50, "rk", t_hist))
    v_hist = oracle.widen(_rand((b, hkv, t_hist, d), 50, "rv", t_hist))
    q = oracle.widen(_rand((b, hq, d), 50, "rq", t_hist))
    kr, vr = _ring_from_history(k_hist, v_hist, window)
    got = oracle.ring_decode_attention(q, kr, vr, np.full(b, t_hist - 1), n_pending=1)
    lo = max(0, t_hist - window)
    want = oracle.decode_attention(q, k_hist[:, :, lo:], v_hist[:, :, lo:], np.full(b, t_hist - lo - 1), n_pending=1)
    assert np.abs(got - want).max() < 1e-14


def test_ring_slots_hold_the_last_w_tokens():
    """Closed form: after T appends, slot t % W holds token t for t in [T - W, T)."""
    b, h, t_hist, d, window = 1, 2, 23, 4, 8
    k_hist = np.arange(b * h * t_hist * d, dtype=np.float64).reshape(b, h, t_hist, d)
    kr, _ = _ring_from_history(k_hist, -k_hist, window)
    for t in range(t_hist - window, t_hist):
        assert np.array_equal(kr[0, :, t % window], k_hist[0, :, t])


def test_ring_append_ignores_negative_counts():
    kr = np.zeros((2, 1, 4, 2))
    k2, _ = oracle.ring_append(kr, kr, np.array([-1, 6]), np.ones((2, 1, 2)), np.ones((2, 1, 2)))
    assert np.array_equal(k2[0], kr[0]) and k2[1, 0, 2].tolist() == [1.0, 1.0]


# ------------------------------------------------------------ quantized KV --
# The pages name fp8/int8 caches with per-token/per-head scales ([LA11] §3.1,
# §8; [KVG] "MHA、GQA、MLA 与量化如何改变容量") but fix no format; the format
# pinned here is the oracle's stated reading (OCP E4M3 or symmetric int8, one
# fp32 scale per token and KV head).

def _e4m3_values():
    """Every finite E4M3 magnitude, ascending (from torch's own decoding)."""
    v = torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    return np.unique(v.astype(np.float64))


def test_e4m3_decode_matches_torch_for_every_code():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = np.array([oracle.e4m3_decode_one(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.isnan(got).sum() == 2                        # S.1111.111 only


def test_e4m3_encode_matches_torch_below_the_saturation_point():
    """torch's fp32 -> float8_e4m3fn conversion (round to nearest even) on
    every finite value, every midpoint between neighbours, points just either
    side of each midpoint, and log-uniform random values of both signs."""
    vals = _e4m3_values()
    mids = (vals[:-1] + vals[1:]) / 2
    eps = np.nextafter(mids.astype(np.float32), np.float32(np.inf)).astype(np.float64)
    below = np.nextafter(mids.astype(np.float32), np.float32(0)).astype(np.float64)
    rng = np.random.default_rng(3)
    rand = np.exp2(rng.uniform(-14, np.log2(447.9), 4000))
    x = np.concatenate([vals, mids, eps, below, rand]).astype(np.float32)
    x = np.concatenate([x, -x])
    x = x[np.abs(x) < 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode_one(float(v)) for v in x], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_closed_forms_and_saturation():
    """Values fixed by the OCP E4M3 definition, and the oracle's reading for
    magnitudes at or above 448 (saturate; torch would give NaN there)."""
    enc = oracle.e4m3_encode_one
    assert enc(1.0) == 0x38 and enc(-2.0) == 0xC0 and enc(448.0) == 0x7E
    assert enc(2.0 ** -6) == 0x08 and enc(2.0 ** -9) == 0x01 and enc(0.875 * 2.0 ** -6) == 0x07
    assert enc(2.0 ** -10) == 0x00 and enc(3 * 2.0 ** -10) == 0x02       # ties to even in the subnormals
    assert enc(1.0625) == 0x38 and enc(1.1875) == 0x3A                   # ties to even, 1 + m/8
    assert enc(7.75 * 2.0 ** -9) == 0x08                                 # rounds up to the first normal
    assert enc(464.0) == 0x7E and enc(1e30) == 0x7E and enc(math.inf) == 0x7E and enc(-math.inf) == 0xFE
    assert enc(math.nan) == 0x7F and enc(-0.0) == 0x80 and enc(0.0) == 0x00


def test_int8_code_rounds_half_to_even_and_clamps():
    enc = oracle.int8_encode_one
    assert [enc(x) for x in (2.5, 3.5, -2.5, -3.5, 0.5, 1.5, 126.5, 127.49)] == [2, 4, -2, -4, 0, 2, 126, 127]
    assert enc(127.6) == 127 and enc(300.0) == 127 and enc(-128.0) == -127
    assert oracle.code_value(0xFF, oracle.QFMT_INT8) == -1.0 and oracle.code_value(0x81, oracle.QFMT_INT8) == -127.0


@pytest.mark.parametrize("fmt", [oracle.QFMT_FP8_E4M3, oracle.QFMT_INT8])
def test_quantize_rows_scale_and_extreme_code(fmt):
    """scale = fp32(amax) / QMAX as an fp32 division, computed here with torch;
    the element of largest magnitude gets the top code; a zero row gets scale
    0 and zero codes."""
    x = synth.normal((3, 4, 32), "bf16", 5, "qscale").float()
    x[1, 2] = 0.0
    codes, scales = oracle.quantize_rows(x, fmt)
    qmax = 448.0 if fmt == oracle.QFMT_FP8_E4M3 else 127.0
    want = x.abs().amax(-1) / torch.tensor(qmax, dtype=torch.float32)
    want[1, 2] = 0.0
    assert np.array_equal(scales, want.numpy())
    assert not codes[1, 2].any() and scales[1, 2] == 0
    top = 0x7E if fmt == oracle.QFMT_FP8_E4M3 else 127
    i = x.abs().argmax(-1)
    for b in range(3):
        for h in range(4):
            if b == 1 and h == 2:
                continue
            c = int(codes[b, h, i[b, h]])
            assert c & 0x7F == top if fmt == oracle.QFMT_FP8_E4M3 else (c if c < 128 else 256 - c) == top


@pytest.mark.parametrize("fmt", [oracle.QFMT_FP8_E4M3, oracle.QFMT_INT8])
def test_quantize_rows_error_bounds(fmt):
    """int8: |x - value| <= scale/2 (plus the fp32 quotient's rounding);
    fp8: half a unit in the last place of a 3-bit mantissa for normals,
    2^-10 * scale in the subnormal range."""
    x = synth.normal((4, 8, 128), "fp32", 6, "qerr").double().numpy()
    x[0, 0] *= 1e-3
    codes, scales = oracle.quantize_rows(x.astype(np.float32), fmt)
    err = np.abs(oracle.dequantize(codes, scales, fmt) - x)
    s = scales.astype(np.float64)[..., None]
    if fmt == oracle.QFMT_INT8:
        assert (err <= s * (0.5 + 2e-5)).all()
    else:
        y = np.abs(x) / s
        bound = np.where(y >= 2.0 ** -6, np.abs(x) * (2.0 ** -4) * (1 + 1e-6), s * 2.0 ** -10 * (1 + 1e-6))
        assert (err <= bound + 1e-30).all()
    assert err.max() > 0


@pytest.mark.parametrize("fmt", [oracle.QFMT_FP8_E4M3, oracle.QFMT_INT8])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4)])
def test_quant_decode_matches_sdpa_on_independently_dequantised_cache(fmt, hq, hkv):
    """The cache's values rebuilt without the oracle's codec (torch's
    float8_e4m3fn decoding, or int8 as signed bytes, times the scales), then
    torch SDPA with GQA: K and V scales, token and head indexing all enter."""
    b, t, d = 3, 40, 32
    k = synth.normal((b, hkv, t, d), "bf16", 7, "qsd", "k").float()
    v = synth.normal((b, hkv, t, d), "bf16", 7, "qsd", "v").float()
    q = synth.normal((b, hq, d), "bf16", 7, "qsd", "q")
    kc, ks = oracle.quantize_rows(k, fmt)
    vc, vs = oracle.quantize_rows(v, fmt)
    lens = np.array([0, 17, 39])

    def deq(c, s):
        ct = torch.from_numpy(c)
        base = ct.view(torch.float8_e4m3fn).double() if fmt == oracle.QFMT_FP8_E4M3 else ct.view(torch.int8).double()
        return base * torch.from_numpy(s).double()[..., None]

    kd, vd = deq(kc, ks), deq(vc, vs)
    got = oracle.quant_decode_attention(q, kc, ks, vc, vs, lens, fmt, n_pending=1)
    for bb in range(b):
        n = int(lens[bb]) + 1
        ref = F.scaled_dot_product_attention(q[bb:bb + 1, :, None].double(), kd[bb:bb + 1, :, :n],
                                             vd[bb:bb + 1, :, :n], enable_gqa=True)[:, :, 0]
        assert np.abs(got[bb] - ref[0].numpy()).max() < 1e-12


def test_quant_scale_folding_invariants():
    """Scaling every K scale by c is the softmax scale times c; scaling every V
    scale by c scales the output by c (c a power of two, so exact)."""
    fmt = oracle.QFMT_INT8
    k = synth.normal((2, 2, 24, 16), "fp32", 8, "qfold", "k")
    v = synth.normal((2, 2, 24, 16), "fp32", 8, "qfold", "v")
    q = synth.normal((2, 4, 16), "fp32", 8, "qfold", "q")
    kc, ks = oracle.quantize_rows(k, fmt)
    vc, vs = oracle.quantize_rows(v, fmt)
    lens = np.array([10, 23])
    base = oracle.quant_decode_attention(q, kc, ks, vc, vs, lens, fmt, n_pending=1)
    k4 = oracle.quant_decode_attention(q, kc, ks * 4, vc, vs, lens, fmt, n_pending=1, scale=0.25 / 4)
    ref4 = oracle.quant_decode_attention(q, kc, ks, vc, vs, lens, fmt, n_pending=1, scale=0.25)
    assert np.allclose(k4, ref4, rtol=0, atol=1e-14)
    v8 = oracle.quant_decode_attention(q, kc, ks, vc, vs * 8, lens, fmt, n_pending=1)
    assert np.array_equal(v8, base * 8)


def test_quant_append_and_fill_slots():
    """The rows land at the slots append/prefill_fill would use, quantised as
    quantize_rows does; other slots and sequences that do not fit stay as
    they were (and are flagged)."""
    fmt = oracle.QFMT_FP8_E4M3
    b, h, t_max, d = 3, 2, 8, 16
    kc = np.full((b, h, t_max, d), 0x7F, dtype=np.uint8)
    vc = kc.copy()
    ks = np.full((b, h, t_max), np.nan, dtype=np.float32)
    vs = ks.copy()
    kn = synth.normal((b, h, 3, d), "bf16", 9, "qapp", "k")
    vn = synth.normal((b, h, 3, d), "bf16", 9, "qapp", "v")
    kc2, vc2, ks2, vs2, over = oracle.quant_prefill_fill(kc, vc, ks, vs, [0, 6, 7], kn, vn, fmt)
    assert over.tolist() == [False, True, True]
    want_c, want_s = oracle.quantize_rows(kn, fmt)
    assert np.array_equal(kc2[0, :, :3], want_c[0]) and np.array_equal(ks2[0, :, :3], want_s[0])
    assert (kc2[0, :, 3:] == 0x7F).all() and (kc2[1:] == 0x7F).all() and np.isnan(vs2[1:]).all()
    kc3, _, ks3, _, over = oracle.quant_append(kc2, vc2, ks2, vs2, [3, -1, 8], kn[:, :, 0], vn[:, :, 0], fmt)
    assert over.tolist() == [False, True, True]
    assert np.array_equal(kc3[0, :, 3], want_c[0, :, 0]) and np.array_equal(kc3[0, :, :3], kc2[0, :, :3])
