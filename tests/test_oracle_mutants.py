"""Plant plausible mistakes in the oracle (on the CPU, never on the GPU path) and
check that the pins in test_oracle.py catch each one."""

import math

import numpy as np
import pytest

import oracle
from oracle import kvc_oracle as ko
import tests.test_oracle as pins


def _mutant_decode(kind):
    def decode(q, k_cache, v_cache, seq_lens, n_pending=1, scale=None):
        q, k, v = ko.widen(q), ko.widen(k_cache), ko.widen(v_cache)
        batch, n_q, d = q.shape
        n_kv = k.shape[1]
        if scale is None:
            scale = 1.0 / d if kind == "scale_by_d" else 1.0 / math.sqrt(d)
        out = np.zeros((batch, n_q, d))
        for b in range(batch):
            n = int(seq_lens[b]) + (0 if kind == "drop_pending" else int(n_pending))
            if n <= 0:
                continue
            for h in range(n_q):
                g = h % n_kv if kind == "mod_grouping" else h // (n_q // n_kv)
                s = (k[b, g, :n] @ q[b, h]) * scale
                if kind == "negated_scores":
                    s = -s
                e = np.exp(s - s.max())
                out[b, h] = (e @ v[b, g, :n]) / e.sum()
        return out
    return decode


DECODE_PINS = [
    pins.test_scale_pins_weights_three_to_one,
    pins.test_gqa_equals_mha_on_repeat_interleaved_cache,
    lambda: pins.test_decode_attention_matches_torch_sdpa(8, 2),
    pins.test_toy_full_recompute_equals_incremental_decode,
]


@pytest.mark.parametrize("kind", ["scale_by_d", "mod_grouping", "drop_pending", "negated_scores"])
def test_decode_mutants_are_caught(kind, monkeypatch):
    monkeypatch.setattr(oracle, "decode_attention", _mutant_decode(kind))
    monkeypatch.setattr(ko, "decode_attention", _mutant_decode(kind))
    caught = 0
    for pin in DECODE_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught >= 1, f"no pin caught mutant {kind}"


def test_causal_mask_off_by_one_is_caught(monkeypatch):
    def causal(q, k, v, n_q_heads, n_kv_heads, scale=None):
        q, k, v = ko.widen(q), ko.widen(k), ko.widen(v)
        _, t, d = q.shape
        scale = 1.0 / math.sqrt(d) if scale is None else scale
        out = np.zeros_like(q)
        mask = np.triu(np.full((t, t), -np.inf), 0)       # hides the diagonal too
        mask[0, 0] = 0.0
        for h in range(n_q_heads):
            g = h // (n_q_heads // n_kv_heads)
            s = (q[h] @ k[g].T) * scale + mask
            e = np.exp(s - s.max(axis=1, keepdims=True))
            out[h] = (e / e.sum(axis=1, keepdims=True)) @ v[g]
        return out
    monkeypatch.setattr(oracle, "causal_attention", causal)
    monkeypatch.setattr(ko, "causal_attention", causal)
    with pytest.raises(AssertionError):
        pins.test_causal_attention_matches_torch_sdpa()


def test_cache_bytes_without_k_and_v_factor_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "cache_bytes",
                        lambda L, h, d, s, lens: L * h * d * s * sum(int(t) for t in lens))
    row = pins._rows("capacity_values.csv")[0]
    with pytest.raises(AssertionError):
        pins.test_cache_bytes_matches_printed_values(row)


def test_append_to_wrong_slot_is_caught(monkeypatch):
    real = ko.append

    def off_by_one(k_cache, v_cache, seq_lens, k_new, v_new):
        return real(k_cache, v_cache, np.asarray(seq_lens) + 1, k_new, v_new)
    monkeypatch.setattr(oracle, "append", off_by_one)
    with pytest.raises(AssertionError):
        pins.test_append_writes_one_slot_bitwise_and_nothing_else()


def _mutant_chunk(kind):
    def chunk(q, k_cache, v_cache, seq_lens, scale=None):
        q, k, v = ko.widen(q), ko.widen(k_cache), ko.widen(v_cache)
        batch, t_q, n_q, d = q.shape
        n_kv = k.shape[1]
        scale = 1.0 / math.sqrt(d) if scale is None else scale
        out = np.zeros((batch, t_q, n_q, d))
        for b in range(batch):
            base = int(seq_lens[b])
            for i in range(t_q):
                if kind == "top_left":
                    n = i + 1
                elif kind == "sees_next":
                    n = min(base + i + 2, base + t_q)
                elif kind == "misses_self":
                    n = base + i
                else:   # "whole_block": no mask inside the block
                    n = base + t_q
                if n <= 0:
                    continue
                for h in range(n_q):
                    g = h // (n_q // n_kv)
                    s = (k[b, g, :n] @ q[b, i, h]) * scale
                    e = np.exp(s - s.max())
                    out[b, i, h] = (e @ v[b, g, :n]) / e.sum()
        return out
    return chunk


CHUNK_PINS = [
    lambda: pins.test_chunk_attention_matches_sdpa_with_lower_right_mask(8, 2, 5),
    pins.test_chunked_prefill_equals_one_shot_prefill,
    pins.test_chunk_attention_with_empty_cache_is_causal_prefill,
]


@pytest.mark.parametrize("kind", ["top_left", "sees_next", "misses_self", "whole_block"])
def test_chunk_mask_mutants_are_caught(kind, monkeypatch):
    monkeypatch.setattr(oracle, "chunk_attention", _mutant_chunk(kind))
    monkeypatch.setattr(ko, "chunk_attention", _mutant_chunk(kind))
    caught = 0
    for pin in CHUNK_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught >= 1, f"no pin caught mutant {kind}"


@pytest.mark.parametrize("kind", ["swapped", "off_by_one_page", "row_from_page_start"])
def test_paged_slot_mutants_are_caught(kind, monkeypatch):
    def slot(block_table, b, t, page_size):
        if kind == "swapped":
            return int(block_table[b][t % page_size]), t // page_size
        if kind == "off_by_one_page":
            return int(block_table[b][min(t // page_size + 1, len(block_table[b]) - 1)]), t % page_size
        return int(block_table[b][t // page_size]), 0
    monkeypatch.setattr(ko, "paged_slot", slot)
    caught = 0
    for pin in (pins.test_paged_view_worked_example, pins.test_paged_fill_then_view_round_trips_bitwise):
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught >= 1, f"no pin caught mutant {kind}"


@pytest.mark.parametrize("kind", ["slot_plus_one", "window_plus_one", "oldest_first_only"])
def test_ring_mutants_are_caught(kind, monkeypatch):
    real_slot, real_dec = ko.ring_slot, ko.ring_decode_attention
    if kind == "slot_plus_one":
        monkeypatch.setattr(ko, "ring_slot", lambda t, w: (t + 1) % w)
    elif kind == "window_plus_one":
        def dec(q, k, v, seq_lens, n_pending=1, scale=None):
            w = np.asarray(ko.widen(k)).shape[2]
            n = [min(max(int(x), 0) + n_pending + 1, w) for x in seq_lens]
            return ko.decode_attention(q, k, v, np.array(n) - n_pending, n_pending=n_pending, scale=scale)
        monkeypatch.setattr(oracle, "ring_decode_attention", dec)
    else:
        def dec(q, k, v, seq_lens, n_pending=1, scale=None):
            w = np.asarray(ko.widen(k)).shape[2]
            n = [min(max(int(x), 0) + n_pending, w) - 1 for x in seq_lens]
            return ko.decode_attention(q, k, v, np.array(n) - n_pending, n_pending=n_pending, scale=scale)
        monkeypatch.setattr(oracle, "ring_decode_attention", dec)
    caught = 0
    for pin in (lambda: pins.test_ring_decode_equals_attention_over_the_last_w_tokens(37, 8),
                lambda: pins.test_ring_decode_equals_attention_over_the_last_w_tokens(5, 8),
                pins.test_ring_slots_hold_the_last_w_tokens):
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught >= 1, f"no pin caught mutant {kind}"


@pytest.mark.parametrize("kind", ["e4m3_truncate", "int8_half_away", "int8_qmax_128", "v_scale_dropped",
                                  "k_scale_next_token"])
def test_quant_mutants_are_caught(kind, monkeypatch):
    """Plausible mistakes in the quantised-cache oracle, each caught by a pin."""
    if kind == "e4m3_truncate":
        real = ko.e4m3_encode_one

        def enc(x):
            c = real(x)
            if math.isnan(x) or c & 0x7F == 0x7E:
                return c
            # toward zero: step back one code when rounding went up in magnitude
            return c - 1 if c & 0x7F and abs(ko.e4m3_decode_one(c)) > abs(x) else c
        monkeypatch.setattr(ko, "e4m3_encode_one", enc)
        monkeypatch.setattr(oracle, "e4m3_encode_one", enc)
        pins_to_run = [pins.test_e4m3_encode_matches_torch_below_the_saturation_point,
                       pins.test_e4m3_closed_forms_and_saturation]
    elif kind == "int8_half_away":
        def enc(y):
            return max(-127, min(127, int(math.copysign(math.floor(abs(y) + 0.5), y))))
        monkeypatch.setattr(ko, "int8_encode_one", enc)
        monkeypatch.setattr(oracle, "int8_encode_one", enc)
        pins_to_run = [pins.test_int8_code_rounds_half_to_even_and_clamps]
    elif kind == "int8_qmax_128":
        monkeypatch.setitem(ko.QMAX, ko.QFMT_INT8, 128.0)
        pins_to_run = [lambda: pins.test_quantize_rows_scale_and_extreme_code(ko.QFMT_INT8)]
    else:
        def dec(q, kc, ks, vc, vs, seq_lens, fmt, n_pending=1, scale=None):
            kd = ko.dequantize(kc, ks, fmt)
            if kind == "k_scale_next_token":
                kd = ko.dequantize(kc, np.roll(ks, -1, axis=-1), fmt)
            vd = ko.dequantize(vc, np.ones_like(vs) if kind == "v_scale_dropped" else vs, fmt)
            return ko.decode_attention(q, kd, vd, seq_lens, n_pending=n_pending, scale=scale)
        monkeypatch.setattr(oracle, "quant_decode_attention", dec)
        pins_to_run = [lambda: pins.test_quant_decode_matches_sdpa_on_independently_dequantised_cache(
            ko.QFMT_INT8, 8, 2)]
    caught = 0
    for pin in pins_to_run:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"no pin caught mutant {kind}"
