"""Parity at the limits the kernels are built for, through the C ABI: the
longest sequence a (sequence, KV head) slice can hold (32-bit offsets), a
very large batch, a very wide GQA group, and the streaming-read calibration
kernel reading every byte once."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import kv_cache_append_amd as kvc
import oracle
import synth
from tests.gpu_cases import TOL, DecodeCase

pytestmark = pytest.mark.gpu


def test_longest_sequence_at_the_offset_bound(gpu):
    """A slice is addressed with 32-bit byte offsets, (T_max + 2048) * D * s
    < 2^31: at D = 128 bf16 that is T_max = 8,386,559 tokens. One sequence
    filled to the last slot by the fused step, GQA 4:1, against the oracle."""
    d, s = 128, 2
    t_max = (2**31 - 1) // (d * s) - 2048
    n = t_max - 1                                   # cached tokens; the step appends slot n, the last
    k = synth.normal((1, 1, t_max, d), "bf16", 3, "lim", "K", device=gpu)
    v = synth.normal((1, 1, t_max, d), "bf16", 3, "lim", "V", device=gpu)
    q = synth.normal((1, 4, d), "bf16", 3, "lim", "q", device=gpu)
    kn = synth.normal((1, 1, d), "bf16", 3, "lim", "kn", device=gpu)
    vn = synth.normal((1, 1, d), "bf16", 3, "lim", "vn", device=gpu)
    seq = torch.tensor([n], dtype=torch.int32, device=gpu)
    ws = kvc.workspace(k, v, 4)
    out = torch.empty((1, 4, d), device=gpu)
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    kvc.decode_step(k, v, seq, kn, vn, q, out, ws, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(k[0, 0, n], kn[0, 0]) and torch.equal(v[0, 0, n], vn[0, 0])
    ref = oracle.decode_attention(q.cpu(), k.cpu(), v.cpu(), np.array([n]), n_pending=1)
    assert np.abs(out.double().cpu().numpy() - ref).max() <= TOL["bf16"]


def test_large_batch_sampled(gpu):
    """2048 ragged sequences x 8 KV heads (16384 units): sampled units against
    the oracle."""
    lengths = synth.ragged_lengths(2048, 1, 200, 5, "limb").tolist()
    sample = [(0, 0), (1, 7), (777, 3), (1500, 5), (2047, 7)]
    case = DecodeCase(batch=2048, n_q=32, n_kv=8, head_dim=128, dtype="bf16", lengths=lengths, tag="limb",
                      device=gpu, host_rows=sample)
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    kvc.append(case.k, case.v, case.seq_lens, case.k_new, case.v_new, status=status)
    ws = kvc.workspace(case.k, case.v, 32)
    out = torch.empty((2048, 32, 128), device=gpu)
    kvc.decode_attn(case.k, case.v, case.seq_lens, case.q, out, ws, n_pending=1, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    got = out.double().cpu().numpy()
    for b, g in sample:
        kh, vh = case.oracle_inputs(b, g)
        ref = oracle.decode_attention(case.q_host[b:b + 1, 4 * g:4 * g + 4], kh[None, None], vh[None, None],
                                      np.array([int(case.lengths[b])]), n_pending=1)[0]
        assert np.abs(got[b, 4 * g:4 * g + 4] - ref).max() <= TOL["bf16"]


def test_wide_gqa_group(gpu):
    """256 query heads on 2 KV heads (groups of 128, 16 head blocks each)."""
    case = DecodeCase(batch=2, n_q=256, n_kv=2, head_dim=128, dtype="bf16", lengths=[100, 3000], tag="limg",
                      device=gpu)
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    kvc.append(case.k, case.v, case.seq_lens, case.k_new, case.v_new, status=status)
    ws = kvc.workspace(case.k, case.v, 256)
    out = torch.empty((2, 256, 128), device=gpu)
    kvc.decode_attn(case.k, case.v, case.seq_lens, case.q, out, ws, n_pending=1, status=status)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    for b in range(2):
        for g in range(2):
            kh, vh = case.oracle_inputs(b, g)
            ref = oracle.decode_attention(case.q_host[b:b + 1, 128 * g:128 * (g + 1)], kh[None, None],
                                          vh[None, None], np.array([int(case.lengths[b])]), n_pending=1)[0]
            assert np.abs(got[b, 128 * g:128 * (g + 1)] - ref).max() <= TOL["bf16"]


def test_stream_read_reads_every_word_once(gpu):
    """kvc_stream_read's per-thread XOR folds equal the host's fold of the words
    each thread is assigned (thread i: words i, i + stride, ...), so every
    16-byte word is read exactly once."""
    n_wg, n_bytes = 64, 64 << 20
    stride = n_wg * 256
    buf = torch.randint(0, 256, (n_bytes,), dtype=torch.uint8, device=gpu)
    sink = torch.zeros(int(kvc.load().kvc_stream_read_sink_bytes(n_wg)) // 4, dtype=torch.int32, device=gpu)
    lib = kvc.load()
    rc = lib.kvc_stream_read(kvc._ptr(buf), n_bytes, kvc._ptr(sink), n_wg, kvc._stream(None))
    assert rc == 0
    torch.cuda.synchronize()
    words = buf.cpu().numpy().view(np.uint32).reshape(-1, stride, 4)     # [rounds, thread, dword]
    want = np.bitwise_xor.reduce(np.bitwise_xor.reduce(words, axis=0), axis=1)
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)


def test_stream_read_launch_rate_is_finite(gpu):
    """The per-launch streaming ceiling the bench reports: launches of a fixed
    size over distinct regions, a positive finite rate."""
    rate = kvc.stream_read_launch_rate(1 << 20, n_bytes=8 << 20, grids=(64,), launches=4)
    assert np.isfinite(rate) and rate > 0
    with pytest.raises(ValueError):
        kvc.stream_read_launch_rate(1000)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp32", 64), ("fp16", 256), ("bf16", 32)])
def test_split_read_reads_every_row_once(gpu, dtype, d):
    """kvc_split_read (the decode launch's loads and split exchange without
    its arithmetic): for every (sequence, KV head) unit, the XOR of its 128
    output words equals the host's XOR of every 16-byte word of its K and V
    rows [0, seq_lens[b] + 1), for 1, 2 and 7 splits and on a second call on
    the same workspace (the flags' epochs), so each row is read once and
    every partial is folded in once."""
    tdt = synth.DTYPES[dtype]
    b_, hkv, t_max = 5, 3, 2100
    lens = [0, 1, 17, 300, 2048]
    raw = torch.randint(-(1 << 15), 1 << 15, (2, b_, hkv, t_max, d * tdt.itemsize // 2), dtype=torch.int16,
                        device=gpu)
    k, v = raw[0].view(tdt), raw[1].view(tdt)
    seq = torch.tensor(lens, dtype=torch.int32, device=gpu)
    kh = k.cpu().view(torch.int16).numpy().view(np.uint32)
    vh = v.cpu().view(torch.int16).numpy().view(np.uint32)
    want = np.zeros((b_ * hkv, 4), dtype=np.uint32)
    for bb in range(b_):
        n = min(lens[bb] + 1, t_max)
        for g in range(hkv):
            words = np.concatenate([kh[bb, g, :n].reshape(-1, 4), vh[bb, g, :n].reshape(-1, 4)])
            want[bb * hkv + g] = np.bitwise_xor.reduce(words, axis=0)
    for splits in (1, 2, 7):
        ws = kvc.split_read_workspace(k, v, splits)
        for rep in range(2):
            out = torch.full((b_ * hkv, 128, 4), -1, dtype=torch.int32, device=gpu)
            kvc.split_read(k, v, seq, splits, out, ws)
            torch.cuda.synchronize()
            got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32), axis=1)
            assert np.array_equal(got, want), (splits, rep)
