"""GPU parity of kvc_block_attn (a block of new queries per sequence with the
lower-right causal mask) against oracle.chunk_attention, through the C ABI.
The block's K/V rows are written with kvc_prefill_fill, as a caller would."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import kv_cache_append_amd as kvc
import oracle
import synth
from tests.gpu_cases import TOL, poison_

pytestmark = pytest.mark.gpu


class BlockCase:
    """Cache [B, H_kv, T_max, D] with seq_lens[b] cached rows, a block of t_q
    new rows per sequence (k/v) and its queries q [B, t_q, H_q, D]; NaN past
    the cached rows. Host copies are taken before any libkvc call."""

    def __init__(self, *, batch, n_q, n_kv, d, dtype, lengths, t_q, t_max=None, seed=11, tag="blk",
                 device="cuda"):
        self.t_q, self.n_q, self.n_kv, self.dtype = t_q, n_q, n_kv, dtype
        self.lengths = torch.as_tensor(lengths, dtype=torch.int32)
        self.t_max = int(t_max if t_max is not None else int(self.lengths.max()) + t_q)
        tdt = synth.DTYPES[dtype]
        self.k = poison_(torch.empty((batch, n_kv, self.t_max, d), dtype=tdt, device=device))
        self.v = poison_(torch.empty_like(self.k))
        rows = max(int(self.lengths.max()), 1)
        for name, dst in (("K", self.k), ("V", self.v)):
            full = synth.normal((batch, n_kv, rows, d), dtype, seed, tag, name, device=device)
            for b in range(batch):
                n = int(self.lengths[b])
                if n > 0:
                    dst[b, :, :n].copy_(full[b, :, :n])
        self.k_blk = synth.normal((batch, n_kv, t_q, d), dtype, seed, tag, "kb", device=device)
        self.v_blk = synth.normal((batch, n_kv, t_q, d), dtype, seed, tag, "vb", device=device)
        self.q = synth.normal((batch, t_q, n_q, d), dtype, seed, tag, "q", device=device)
        self.seq_lens = self.lengths.to(device)
        self.k_host, self.v_host = self.k.cpu(), self.v.cpu()
        self.kb_host, self.vb_host, self.q_host = self.k_blk.cpu(), self.v_blk.cpu(), self.q.cpu()

    def fill(self):
        kvc.prefill_fill(self.k, self.v, self.seq_lens, self.k_blk, self.v_blk)

    def oracle(self):
        """fp64 reference on the host: the block written after the cached rows."""
        k, v = self.k_host.clone(), self.v_host.clone()
        for b in range(k.shape[0]):
            n = int(self.lengths[b])
            k[b, :, n:n + self.t_q] = self.kb_host[b]
            v[b, :, n:n + self.t_q] = self.vb_host[b]
        return oracle.chunk_attention(self.q_host, k, v, self.lengths.numpy())


def _run(case: BlockCase, n_splits=0, out_dtype=torch.float32, status=None):
    out = torch.empty(case.q.shape, dtype=out_dtype, device=case.q.device)
    ws = kvc.block_workspace(case.k, case.v, case.n_q, case.t_q, n_splits)
    kvc.block_attn(case.k, case.v, case.seq_lens, case.q, out, ws, n_splits=n_splits, status=status)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("hq,hkv,t_q", [(8, 2, 4), (8, 8, 3), (32, 8, 5), (4, 1, 7), (6, 2, 2), (16, 1, 16)])
def test_block_matches_oracle(gpu, dtype, hq, hkv, t_q):
    case = BlockCase(batch=4, n_q=hq, n_kv=hkv, d=128, dtype=dtype, lengths=[0, 37, 300, 1025], t_q=t_q,
                     tag=f"blk{dtype}{hq}{hkv}{t_q}")
    case.fill()
    got = _run(case).double().cpu().numpy()
    ref = case.oracle()
    assert not np.isnan(got).any()
    assert np.abs(got - ref).max() <= TOL[dtype]


@pytest.mark.parametrize("dtype,d,hq,hkv,t_q", [
    ("bf16", 128, 8, 8, 64),      # MHA chunk of 64 tokens: 64 pairs
    ("fp16", 128, 32, 8, 32),     # 128 pairs
    ("bf16", 64, 16, 8, 64),      # D = 64, 128 pairs
    ("bf16", 128, 4, 4, 40),      # 40 pairs, a block that is not a multiple of 16
    ("bf16", 128, 64, 1, 8),      # MQA verify of 8 tokens: 512 pairs in four pair blocks
    ("fp16", 128, 32, 8, 64),     # 256 pairs, 64 queries: two pair blocks
])
def test_blocks_up_to_64_queries_on_the_wide_kernel(gpu, dtype, d, hq, hkv, t_q):
    """Blocks of 8..64 queries with 8..512 (query, head) pairs per KV head
    (the wide-group kernel's range): within the bar of the oracle, the
    block's own keys under the causal mask included, and run to run
    deterministic."""
    case = BlockCase(batch=4, n_q=hq, n_kv=hkv, d=d, dtype=dtype, lengths=[0, 37, 300, 1025], t_q=t_q,
                     tag=f"wblk{dtype}{d}{hq}{hkv}{t_q}")
    case.fill()
    got = _run(case)
    again = _run(case)
    assert torch.equal(got, again)
    g = got.double().cpu().numpy()
    assert not np.isnan(g).any()
    assert np.abs(g - case.oracle()).max() <= TOL[dtype]


@pytest.mark.parametrize("d", [64, 256, 32])
def test_block_other_head_dims(gpu, d):
    case = BlockCase(batch=2, n_q=8, n_kv=2, d=d, dtype="bf16", lengths=[90, 513], t_q=3, tag=f"blkd{d}")
    case.fill()
    assert np.abs(_run(case).double().cpu().numpy() - case.oracle()).max() <= TOL["bf16"]


@pytest.mark.parametrize("n_splits", [1, 2, 5, 64])
def test_block_split_counts(gpu, n_splits):
    case = BlockCase(batch=3, n_q=8, n_kv=2, d=128, dtype="fp16", lengths=[5, 700, 2000], t_q=4,
                     tag=f"blks{n_splits}")
    case.fill()
    assert np.abs(_run(case, n_splits).double().cpu().numpy() - case.oracle()).max() <= TOL["fp16"]


@pytest.mark.parametrize("hq,hkv", [(32, 8), (64, 2)])     # the decode kernel; the wide-group kernel
def test_block_of_one_equals_decode_bitwise(gpu, hq, hkv):
    case = BlockCase(batch=3, n_q=hq, n_kv=hkv, d=128, dtype="bf16", lengths=[1, 333, 2047], t_q=1,
                     tag=f"blk1{hq}")
    case.fill()
    got = _run(case)
    out = torch.empty((3, hq, 128), device=gpu)
    ws = kvc.workspace(case.k, case.v, hq)
    kvc.decode_attn(case.k, case.v, case.seq_lens, case.q[:, 0].contiguous(), out, ws, n_pending=1)
    torch.cuda.synchronize()
    assert torch.equal(got[:, 0], out)


def test_block_run_to_run_deterministic(gpu):
    case = BlockCase(batch=4, n_q=32, n_kv=8, d=128, dtype="bf16", lengths=[100, 900, 1500, 2048], t_q=4,
                     tag="blkdet")
    case.fill()
    a = _run(case, n_splits=2)
    b = _run(case, n_splits=2)
    assert torch.equal(a, b)


def test_block_out_in_cache_dtype_is_rounded_fp32(gpu):
    case = BlockCase(batch=2, n_q=8, n_kv=2, d=128, dtype="bf16", lengths=[50, 400], t_q=4, tag="blkod")
    case.fill()
    f32 = _run(case)
    half = _run(case, out_dtype=torch.bfloat16)
    assert torch.equal(half, f32.to(torch.bfloat16))


def test_chunked_prefill_through_the_abi(gpu):
    """A prompt prefilled in chunks (fill, then block attention, then advance)
    gives the rows of one causal prefill of the whole prompt (course notes
    Day 4 §3.5, chunked variant), within the dtype's tolerance."""
    hq, hkv, d, t = 8, 2, 128, 45
    tdt = torch.bfloat16
    k = poison_(torch.empty((1, hkv, t, d), dtype=tdt, device=gpu))
    v = poison_(torch.empty_like(k))
    kp = synth.normal((1, hkv, t, d), "bf16", 3, "cp", "k", device=gpu)
    vp = synth.normal((1, hkv, t, d), "bf16", 3, "cp", "v", device=gpu)
    qp = synth.normal((1, t, hq, d), "bf16", 3, "cp", "q", device=gpu)
    seq = torch.zeros(1, dtype=torch.int32, device=gpu)
    outs, start = [], 0
    for size in (16, 1, 20, 8):
        ws = kvc.block_workspace(k, v, hq, size)
        kvc.prefill_fill(k, v, seq, kp[:, :, start:start + size], vp[:, :, start:start + size])
        out = torch.empty((1, size, hq, d), device=gpu)
        kvc.block_attn(k, v, seq, qp[:, start:start + size].contiguous(), out, ws)
        kvc.seq_lens_advance(seq, size)
        outs.append(out)
        start += size
    torch.cuda.synchronize()
    got = torch.cat(outs, dim=1).double().cpu().numpy()
    ref = oracle.chunk_attention(qp.cpu(), kp.cpu(), vp.cpu(), np.array([0]))
    assert np.abs(got - ref).max() <= TOL["bf16"]


def test_block_that_does_not_fit_gives_zero_rows_and_flags(gpu):
    case = BlockCase(batch=3, n_q=8, n_kv=2, d=128, dtype="fp16", lengths=[10, 60, 20], t_q=5, t_max=64,
                     tag="blkfit")
    case.fill()                                   # sequence 1's block does not fit: not written either
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    got = _run(case, status=status)
    assert int(status.item()) & kvc.DEVERR_CAPACITY
    assert torch.count_nonzero(got[1]) == 0
    k, v = case.k.cpu(), case.v.cpu()
    for b in (0, 2):
        r = oracle.chunk_attention(case.q_host[b:b + 1], k[b:b + 1], v[b:b + 1], np.array([int(case.lengths[b])]))
        assert np.abs(got[b:b + 1].double().cpu().numpy() - r).max() <= TOL["fp16"]


def test_block_negative_length_is_flagged(gpu):
    case = BlockCase(batch=2, n_q=4, n_kv=2, d=128, dtype="fp16", lengths=[10, 30], t_q=2, tag="blkneg")
    case.fill()
    case.seq_lens[1] = -3
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    got = _run(case, status=status)
    assert int(status.item()) & kvc.DEVERR_BADLEN
    assert torch.count_nonzero(got[1]) == 0


@pytest.mark.parametrize("t_q", [4, 8, 16, 32])
def test_verify_step_at_gqa_8b_shape_sampled(gpu, t_q):
    """A block of t_q new tokens at the 8B GQA shape (B=16, 32/8 heads,
    D=128, T=2048, bf16; 16 to 128 (query, head) pairs per KV head, all on
    the wide-group kernel), with the library's split choice, checked on
    sampled sequences."""
    case = BlockCase(batch=16, n_q=32, n_kv=8, d=128, dtype="bf16", lengths=[2048] * 16, t_q=t_q,
                     tag=f"blkv8b{t_q}")
    case.fill()
    got = _run(case)
    k, v = case.k.cpu(), case.v.cpu()
    for b in (0, 7, 15):
        r = oracle.chunk_attention(case.q_host[b:b + 1], k[b:b + 1], v[b:b + 1], np.array([2048]))
        assert np.abs(got[b:b + 1].double().cpu().numpy() - r).max() <= TOL["bf16"]


# kvc_block_step: the fill and the attention of a block in one call (one
# launch where the wide-group kernel serves the block).
@pytest.mark.parametrize("dtype,d,hq,hkv,t_q", [
    ("bf16", 128, 32, 8, 4),      # 16 pairs: one fused launch (the 4-token verify at the 8B GQA shape)
    ("bf16", 128, 32, 8, 2),      # 8 pairs: fused
    ("fp16", 128, 16, 1, 5),      # MQA-like, 80 pairs: fused
    ("bf16", 128, 1, 1, 20),      # 20 pairs, t_q = 20: fused (the block's rows fill most of a tile)
    ("bf16", 64, 16, 2, 3),       # D = 64: fused
    ("fp16", 128, 8, 8, 3),       # 3 pairs: fill, then the decode kernel
    ("fp16", 128, 64, 1, 3),      # 192 pairs: fused, two pair blocks
    ("bf16", 128, 64, 1, 8),      # 512 pairs: fused, four pair blocks
    ("bf16", 128, 32, 8, 8),      # 32 pairs, t_q = 8: fused
    ("bf16", 128, 32, 8, 32),     # 128 pairs, t_q = 32: fused (the rows fill the threads' one pass)
    ("bf16", 128, 8, 8, 48),      # 48 pairs, t_q = 48: fill, then the wide-group kernel
    ("bf16", 64, 16, 8, 64),      # D = 64, 128 pairs, t_q = 64: fused
    ("fp16", 128, 8, 8, 80),      # t_q = 80: fill, then the prefill kernel
    ("fp32", 128, 8, 2, 4),       # fp32 cache: fill, then the decode kernel
])
@pytest.mark.parametrize("n_splits", [0, 3])
def test_block_step_equals_fill_then_attn(gpu, dtype, d, hq, hkv, t_q, n_splits):
    """Cache bytes and output bits of kvc_block_step equal those of
    kvc_prefill_fill + kvc_block_attn on the same inputs, on every route, and
    the output is within the bar of the fp64 oracle."""
    lens = [0, 37, 300, 1025]
    tag = f"bstep{dtype}{d}{hq}{hkv}{t_q}"
    a = BlockCase(batch=4, n_q=hq, n_kv=hkv, d=d, dtype=dtype, lengths=lens, t_q=t_q, tag=tag)
    w = BlockCase(batch=4, n_q=hq, n_kv=hkv, d=d, dtype=dtype, lengths=lens, t_q=t_q, tag=tag)
    out_a = torch.full(a.q.shape, float("nan"), device=gpu)
    st_a = torch.zeros(1, dtype=torch.int32, device=gpu)
    ws = kvc.block_workspace(a.k, a.v, hq, t_q, n_splits)
    kvc.block_step(a.k, a.v, a.seq_lens, a.k_blk, a.v_blk, a.q, out_a, ws, n_splits=n_splits, status=st_a)
    w.fill()
    st_w = torch.zeros(1, dtype=torch.int32, device=gpu)
    out_w = _run(w, n_splits=n_splits, status=st_w)
    torch.cuda.synchronize()
    assert int(st_a.item()) == 0 and int(st_w.item()) == 0
    assert torch.equal(out_a, out_w)
    iv = torch.int32 if dtype == "fp32" else torch.int16
    assert torch.equal(a.k.view(iv), w.k.view(iv)) and torch.equal(a.v.view(iv), w.v.view(iv))
    assert np.abs(out_a.double().cpu().numpy() - a.oracle()).max() <= TOL[dtype]


def test_block_step_repeated_with_a_strided_source(gpu):
    """Three verify blocks in a row through kvc_block_step (the lengths moved
    by the block each time), the block's rows taken from a token-major
    [B, t_q, H_kv, D] buffer through strides, against the oracle over the
    cache the steps built."""
    b_, hq, hkv, d, t_q = 3, 32, 4, 128, 4
    case = BlockCase(batch=b_, n_q=hq, n_kv=hkv, d=d, dtype="bf16", lengths=[5, 190, 700], t_q=t_q,
                     t_max=720, tag="bstep_seq")
    k_ref, v_ref = case.k_host.clone(), case.v_host.clone()
    lens = case.lengths.clone()
    ws = kvc.block_workspace(case.k, case.v, hq, t_q, 0)
    for step in range(3):
        kb = synth.normal((b_, t_q, hkv, d), "bf16", 11, "bstep_seq", step, "k", device=gpu)
        vb = synth.normal((b_, t_q, hkv, d), "bf16", 11, "bstep_seq", step, "v", device=gpu)
        q = synth.normal((b_, t_q, hq, d), "bf16", 11, "bstep_seq", step, "q", device=gpu)
        out = torch.empty((b_, t_q, hq, d), device=gpu)
        status = torch.zeros(1, dtype=torch.int32, device=gpu)
        kvc.block_step(case.k, case.v, case.seq_lens, kb.transpose(1, 2), vb.transpose(1, 2), q, out, ws,
                       status=status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        for bb in range(b_):
            n = int(lens[bb])
            k_ref[bb, :, n:n + t_q] = kb[bb].transpose(0, 1).cpu()
            v_ref[bb, :, n:n + t_q] = vb[bb].transpose(0, 1).cpu()
        ref = oracle.chunk_attention(q.cpu(), k_ref, v_ref, lens.numpy())
        assert np.abs(out.double().cpu().numpy() - ref).max() <= TOL["bf16"]
        lens += t_q
        kvc.seq_lens_advance(case.seq_lens, t_q)
    got_k = case.k.cpu()
    for bb in range(b_):
        n = int(lens[bb])
        assert torch.equal(got_k[bb, :, :n].view(torch.int16), k_ref[bb, :, :n].view(torch.int16))


# one fused launch (80 pairs); fill then attention (5 pairs); one fused launch in three pair blocks (320 pairs)
@pytest.mark.parametrize("hq", [32, 2, 128])
def test_block_step_that_does_not_fit_or_has_a_negative_length(gpu, hq):
    """A block past max_len is not written and gets zero rows (capacity flag);
    a negative length gets zero rows (bad-length flag); the other sequences
    are exact, as with the separate calls."""
    case = BlockCase(batch=3, n_q=hq, n_kv=2, d=128, dtype="bf16", lengths=[10, 60, 20], t_q=5, t_max=64,
                     tag=f"bstepfit{hq}")
    case.seq_lens[2] = -4
    out = torch.empty(case.q.shape, device=gpu)
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    ws = kvc.block_workspace(case.k, case.v, hq, 5, 0)
    kvc.block_step(case.k, case.v, case.seq_lens, case.k_blk, case.v_blk, case.q, out, ws, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & kvc.DEVERR_CAPACITY and int(status.item()) & kvc.DEVERR_BADLEN
    assert torch.count_nonzero(out[1]) == 0 and torch.count_nonzero(out[2]) == 0
    k = case.k.cpu()
    assert torch.isnan(k[1, :, 60:].float()).all()           # not written
    kr, vr = case.k_host.clone(), case.v_host.clone()
    kr[0, :, 10:15], vr[0, :, 10:15] = case.kb_host[0], case.vb_host[0]
    r = oracle.chunk_attention(case.q_host[:1], kr[:1], vr[:1], np.array([10]))
    assert np.abs(out[:1].double().cpu().numpy() - r).max() <= TOL["bf16"]

