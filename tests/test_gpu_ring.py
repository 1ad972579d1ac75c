"""GPU parity of the sliding-window ring cache through the C ABI: ring fill
and append bit-exact against the oracle's token-by-token appends, ring
decode against oracle.ring_decode_attention, and the fused ring step equal
to append + decode bit for bit across wrap-arounds."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import kv_cache_append_amd as kvc
import oracle
import synth
from tests.gpu_cases import TOL, poison_

pytestmark = pytest.mark.gpu


def _history(batch, n_kv, t_hist, d, dtype, tag, device):
    k = synth.normal((batch, n_kv, t_hist, d), dtype, 5, tag, "hk", device=device)
    v = synth.normal((batch, n_kv, t_hist, d), dtype, 5, tag, "hv", device=device)
    return k, v


def _oracle_ring(k_hist, v_hist, lengths, window):
    """Token-by-token oracle appends of each sequence's first lengths[b] tokens."""
    b, h, _, d = k_hist.shape
    kr = np.full((b, h, window, d), np.nan)
    vr = np.full((b, h, window, d), np.nan)
    kh, vh = k_hist.float().cpu().numpy(), v_hist.float().cpu().numpy()
    for i in range(int(max(lengths))):
        cnt = np.array([i if i < lengths[bb] else -1 for bb in range(b)])   # -1: sequence done
        kr, vr = oracle.ring_append(kr, vr, cnt, kh[:, :, min(i, kh.shape[2] - 1)], vh[:, :, min(i, kh.shape[2] - 1)])
    return kr, vr


def _ring_device(k_hist, v_hist, lengths, window, device):
    """Ring filled on the device with one kvc_ring_prefill_fill per sequence
    (a block longer than the window keeps only its last W rows)."""
    b, h, _, d = k_hist.shape
    k = poison_(torch.empty((b, h, window, d), dtype=k_hist.dtype, device=device))
    v = poison_(torch.empty_like(k))
    for bb in range(b):
        n = int(lengths[bb])
        if n == 0:
            continue
        one = torch.full((b,), -1, dtype=torch.int32, device=device)   # other sequences: skipped
        one[bb] = 0
        st = torch.zeros(1, dtype=torch.int32, device=device)
        kvc.ring_prefill_fill(k, v, one, k_hist[:, :, :n].contiguous(), v_hist[:, :, :n].contiguous(), status=st)
    torch.cuda.synchronize()
    return k, v


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp32", 4), ("fp16", 40)])
def test_ring_fill_keeps_the_last_window_bitwise(gpu, dtype, d):
    lengths = [0, 5, 16, 17, 50]
    window = 16
    k_hist, v_hist = _history(5, 2, 50, d, dtype, f"rf{dtype}", gpu)
    k, v = _ring_device(k_hist, v_hist, lengths, window, gpu)
    kr, vr = _oracle_ring(k_hist, v_hist, lengths, window)
    got = k.float().cpu().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(kr))
    assert np.array_equal(np.nan_to_num(got), np.nan_to_num(kr))
    gv = v.float().cpu().numpy()
    assert np.array_equal(np.nan_to_num(gv), np.nan_to_num(vr))


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (32, 8), (4, 4), (16, 2), (64, 1), (128, 1), (512, 2)])
def test_ring_decode_matches_oracle(gpu, dtype, hq, hkv):
    window = 512
    lengths = [1, 300, 511, 512, 513, 2000]
    d = 128
    k_hist, v_hist = _history(len(lengths), hkv, max(lengths), d, dtype, f"rd{dtype}{hq}{hkv}", gpu)
    k, v = _ring_device(k_hist, v_hist, lengths, window, gpu)
    q = synth.normal((len(lengths), hq, d), dtype, 5, "rdq", dtype, hq, device=gpu)
    seq = torch.tensor(lengths, dtype=torch.int32, device=gpu)
    out = torch.empty((len(lengths), hq, d), device=gpu)
    ws = kvc.workspace(k, v, hq)
    kvc.ring_decode_attn(k, v, seq, q, out, ws, n_pending=0)
    torch.cuda.synchronize()
    ref = oracle.ring_decode_attention(q.cpu(), k.cpu(), v.cpu(), np.array(lengths), n_pending=0)
    assert np.abs(out.double().cpu().numpy() - ref).max() <= TOL[dtype]
    # and the same as plain decode over the last W tokens of the full history
    for bb, n in enumerate(lengths):
        lo = max(0, n - window)
        r2 = oracle.decode_attention(q[bb:bb + 1].cpu(), k_hist[bb:bb + 1, :, lo:n].cpu(),
                                     v_hist[bb:bb + 1, :, lo:n].cpu(), np.array([n - lo]), n_pending=0)
        assert np.abs(out[bb:bb + 1].double().cpu().numpy() - r2).max() <= TOL[dtype]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_splits", [0, 2])
def test_ring_wide_groups_odd_window(gpu, d, n_splits):
    """16 query heads per KV head (the wide-group kernel's ring mode) on a
    37-slot ring: the newest slot lands anywhere inside a 64-row tile, and a
    tile holds the whole window; against the oracle and plain decode over
    the last W tokens."""
    window, hq, hkv = 37, 32, 2
    lengths = [1, 36, 37, 38, 100, 1000]
    k_hist, v_hist = _history(len(lengths), hkv, max(lengths), d, "fp16", f"rw{d}{n_splits}", gpu)
    k, v = _ring_device(k_hist, v_hist, lengths, window, gpu)
    q = synth.normal((len(lengths), hq, d), "fp16", 6, "rwq", d, device=gpu)
    seq = torch.tensor(lengths, dtype=torch.int32, device=gpu)
    out = torch.empty((len(lengths), hq, d), device=gpu)
    ws = kvc.workspace(k, v, hq, n_splits)
    kvc.ring_decode_attn(k, v, seq, q, out, ws, n_pending=0, n_splits=n_splits)
    torch.cuda.synchronize()
    ref = oracle.ring_decode_attention(q.cpu(), k.cpu(), v.cpu(), np.array(lengths), n_pending=0)
    assert np.abs(out.double().cpu().numpy() - ref).max() <= TOL["fp16"]
    for bb, n in enumerate(lengths):
        lo = max(0, n - window)
        r2 = oracle.decode_attention(q[bb:bb + 1].cpu(), k_hist[bb:bb + 1, :, lo:n].cpu(),
                                     v_hist[bb:bb + 1, :, lo:n].cpu(), np.array([n - lo]), n_pending=0)
        assert np.abs(out[bb:bb + 1].double().cpu().numpy() - r2).max() <= TOL["fp16"]


@pytest.mark.parametrize("n_splits", [1, 3, 8])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("hq", [8, 32, 512])
def test_ring_step_equals_append_plus_decode_across_wraps(gpu, n_splits, dtype, hq):
    """60 fused steps on a 48-slot ring from lengths around the window: cache
    and output bit-identical to ring append + ring decode, and within
    tolerance of the oracle, while the newest slot walks through the ring.
    16 and 256 query heads per KV head in bf16 run on the wide-group kernel
    (256: two pair blocks)."""
    window, hkv, d = 48, 2, 128 if dtype == "bf16" else 64
    lengths = [0, 20, 47, 48, 100]
    k_hist, v_hist = _history(5, hkv, max(lengths) + 1, d, dtype, f"rs{dtype}{n_splits}{hq}", gpu)
    k1, v1 = _ring_device(k_hist, v_hist, lengths, window, gpu)
    k2, v2 = k1.clone(), v1.clone()
    seq1 = torch.tensor(lengths, dtype=torch.int32, device=gpu)
    seq2 = seq1.clone()
    ws1, ws2 = kvc.workspace(k1, v1, hq, n_splits), kvc.workspace(k1, v1, hq, n_splits)
    for step in range(60):
        kn = synth.normal((5, hkv, d), dtype, step, "rs", "kn", device=gpu)
        vn = synth.normal((5, hkv, d), dtype, step, "rs", "vn", device=gpu)
        q = synth.normal((5, hq, d), dtype, step, "rs", "q", device=gpu)
        o1 = torch.empty((5, hq, d), device=gpu)
        kvc.ring_decode_step(k1, v1, seq1, kn, vn, q, o1, ws1, n_splits=n_splits)
        kvc.seq_lens_advance(seq1)
        kvc.ring_append(k2, v2, seq2, kn, vn)
        o2 = torch.empty((5, hq, d), device=gpu)
        kvc.ring_decode_attn(k2, v2, seq2, q, o2, ws2, n_pending=1, n_splits=n_splits)
        kvc.seq_lens_advance(seq2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
        if step % 17 == 0:
            cnt = (seq2 - 1).cpu().numpy()
            ref = oracle.ring_decode_attention(q.cpu(), k2.cpu(), v2.cpu(), cnt, n_pending=1)
            assert np.abs(o1.double().cpu().numpy() - ref).max() <= TOL[dtype]
    assert torch.equal(torch.nan_to_num(k1), torch.nan_to_num(k2))


def test_ring_negative_length_is_flagged(gpu):
    k = torch.zeros((2, 2, 32, 128), dtype=torch.bfloat16, device=gpu)
    v = torch.zeros_like(k)
    seq = torch.tensor([-2, 40], dtype=torch.int32, device=gpu)
    kn = torch.ones((2, 2, 128), dtype=torch.bfloat16, device=gpu)
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    kvc.ring_append(k, v, seq, kn, kn, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & kvc.DEVERR_BADLEN
    assert torch.count_nonzero(k[0]) == 0
    assert torch.equal(k[1, :, 40 % 32], kn[1])
