"""GPU parity of the wide-group decode kernel (8 to 128 (query, head) pairs
per KV head on a contiguous fp16/bf16 cache with head dim 64 or 128: MQA,
wide GQA and query blocks), through the C ABI, against the fp64 oracle.

The kernel streams each KV head's K/V once for all pairs (course notes
"第 1 周 · Day 4" §2.2, §2.5). Bars as for every decode: max-abs 2e-3 vs the
fp64 oracle for 16-bit caches; the fused step equals append + decode bit for
bit; NaN past the attended rows catches any read out of range."""

import numpy as np
import pytest
import torch

import kv_cache_append_amd as kvc
import oracle
import synth
from tests.gpu_cases import TOL, DecodeCase
from tests.test_gpu_block import BlockCase

pytestmark = pytest.mark.gpu

LENS = [0, 1, 63, 64, 65, 129, 1000, 2111]


def _oracle_all(case: DecodeCase):
    grp = case.n_q // case.n_kv
    ref = np.zeros((case.batch, case.n_q, case.head_dim))
    for (b, g) in case.host:
        k, v = case.oracle_inputs(b, g)
        ref[b, g * grp:(g + 1) * grp] = oracle.decode_attention(
            case.q_host[b:b + 1, g * grp:(g + 1) * grp], k[None, None], v[None, None],
            np.array([int(case.lengths[b])]), n_pending=1)[0]
    return ref


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_q,n_kv", [(8, 1), (24, 2), (16, 1), (32, 1), (64, 1), (128, 1), (64, 2), (256, 1), (320, 2)])
@pytest.mark.parametrize("splits", [0, 1, 2, 3])
def test_wide_decode_step_matches_oracle(gpu, dtype, d, n_q, n_kv, splits):
    """The fused step (append + attend T_b + 1 rows) on the wide kernel, for
    lengths on and around the 64-key tile and empty sequences, with one, two
    (last-split merge), three (spread merge) or the library's number of
    splits; groups of 256 and 160 heads run in two pair blocks of up to 128
    heads; the appended rows are exact."""
    case = DecodeCase(batch=len(LENS), n_q=n_q, n_kv=n_kv, head_dim=d, dtype=dtype, lengths=LENS,
                      tag=f"wide{dtype}{d}{n_q}{n_kv}", device=gpu)
    ws = kvc.workspace(case.k, case.v, n_q, splits)
    out = torch.empty((case.batch, n_q, d), device=gpu)
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    kvc.decode_step(case.k, case.v, case.seq_lens, case.k_new, case.v_new, case.q, out, ws, n_splits=splits,
                    status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    got = out.double().cpu().numpy()
    assert np.isfinite(got).all()
    assert np.abs(got - _oracle_all(case)).max() <= TOL[dtype]
    iv = torch.int16
    for b, n in enumerate(LENS):
        assert torch.equal(case.k[b, :, n].cpu().view(iv), case.k_new[b].cpu().view(iv))
        assert torch.equal(case.v[b, :, n].cpu().view(iv), case.v_new[b].cpu().view(iv))


@pytest.mark.parametrize("splits", [0, 1, 2, 8])
def test_wide_step_equals_append_then_decode(gpu, splits):
    """kvc_decode_step and kvc_append + kvc_decode_attn(n_pending = 1) fold
    the same rows in the same order: identical cache bytes and output bits."""
    lens = [5, 64, 700, 2048]
    a = DecodeCase(batch=4, n_q=64, n_kv=1, head_dim=128, dtype="bf16", lengths=lens, tag="wideq", device=gpu)
    b = DecodeCase(batch=4, n_q=64, n_kv=1, head_dim=128, dtype="bf16", lengths=lens, tag="wideq", device=gpu)
    ws_a, ws_b = kvc.workspace(a.k, a.v, 64, splits), kvc.workspace(b.k, b.v, 64, splits)
    out_a = torch.empty((4, 64, 128), device=gpu)
    out_b = torch.empty_like(out_a)
    kvc.append(a.k, a.v, a.seq_lens, a.k_new, a.v_new)
    kvc.decode_attn(a.k, a.v, a.seq_lens, a.q, out_a, ws_a, n_pending=1, n_splits=splits)
    kvc.decode_step(b.k, b.v, b.seq_lens, b.k_new, b.v_new, b.q, out_b, ws_b, n_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(a.k.view(torch.int16), b.k.view(torch.int16))
    assert torch.equal(a.v.view(torch.int16), b.v.view(torch.int16))
    assert torch.equal(out_a, out_b)
    assert np.abs(out_b.double().cpu().numpy() - _oracle_all(b)).max() <= TOL["bf16"]


def test_wide_many_steps_one_workspace(gpu):
    """Twelve steps of the fused wide step on one workspace with lengths
    growing by one per step (kvc_seq_lens_advance), against the oracle on host
    copies that follow the appends."""
    B, hq, d = 3, 32, 128
    lens0 = [0, 100, 1500]
    case = DecodeCase(batch=B, n_q=hq, n_kv=1, head_dim=d, dtype="fp16", lengths=lens0, t_max=1520,
                      tag="widesteps", device=gpu)
    hk, hv = case.k.cpu().clone(), case.v.cpu().clone()
    ws = kvc.workspace(case.k, case.v, hq)
    lens = list(lens0)
    for step in range(12):
        kn = synth.normal((B, 1, d), "fp16", 5, "ws", step, "k", device=gpu)
        vn = synth.normal((B, 1, d), "fp16", 5, "ws", step, "v", device=gpu)
        q = synth.normal((B, hq, d), "fp16", 5, "ws", step, "q", device=gpu)
        out = torch.empty((B, hq, d), device=gpu)
        kvc.decode_step(case.k, case.v, case.seq_lens, kn, vn, q, out, ws)
        kvc.seq_lens_advance(case.seq_lens, 1)
        torch.cuda.synchronize()
        for b in range(B):
            hk[b, :, lens[b]] = kn[b].cpu()
            hv[b, :, lens[b]] = vn[b].cpu()
        ref = oracle.decode_attention(q.cpu(), hk, hv, np.array(lens), n_pending=1)
        assert np.abs(out.double().cpu().numpy() - ref).max() <= TOL["fp16"], step
        lens = [x + 1 for x in lens]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_wide_out_in_cache_dtype_is_rounded_fp32_out(gpu, dtype):
    """out in the cache dtype is the fp32 output rounded to nearest even."""
    case = DecodeCase(batch=3, n_q=64, n_kv=1, head_dim=128, dtype=dtype, lengths=[10, 300, 999], tag="wideo",
                      device=gpu)
    kvc.append(case.k, case.v, case.seq_lens, case.k_new, case.v_new)
    ws = kvc.workspace(case.k, case.v, 64)
    o32 = torch.empty((3, 64, 128), device=gpu)
    o16 = torch.empty((3, 64, 128), dtype=synth.DTYPES[dtype], device=gpu)
    kvc.decode_attn(case.k, case.v, case.seq_lens, case.q, o32, ws, n_pending=1)
    kvc.decode_attn(case.k, case.v, case.seq_lens, case.q, o16, ws, n_pending=1)
    torch.cuda.synchronize()
    assert torch.equal(o32.to(synth.DTYPES[dtype]).view(torch.int16), o16.view(torch.int16))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("hq,hkv,t_q", [(4, 1, 4), (8, 1, 2), (4, 1, 7), (16, 1, 3), (8, 2, 5), (64, 1, 2),
                                        (64, 1, 4), (64, 1, 8), (32, 8, 40), (16, 2, 20)])
@pytest.mark.parametrize("splits", [0, 2, 3])
def test_wide_query_block_matches_oracle(gpu, dtype, hq, hkv, t_q, splits):
    """A block of t_q new queries per sequence (speculative verify, short
    prefill chunks) with 8..512 (query, head) pairs per KV head runs on the
    wide kernel (more than 128 pairs in pair blocks of up to 128: 256, 512
    and 160 pairs here, the last block partly filled), with one merge of
    each kind; the lower-right causal mask of course notes §3.3."""
    case = BlockCase(batch=4, n_q=hq, n_kv=hkv, d=128, dtype=dtype, lengths=[0, 37, 300, 1025], t_q=t_q,
                     tag=f"wblk{dtype}{hq}{hkv}{t_q}", device=gpu)
    case.fill()
    out = torch.empty(case.q.shape, device=gpu)
    ws = kvc.block_workspace(case.k, case.v, hq, t_q, splits)
    kvc.block_attn(case.k, case.v, case.seq_lens, case.q, out, ws, n_splits=splits)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    assert np.isfinite(got).all()
    assert np.abs(got - case.oracle()).max() <= TOL[dtype]


def test_wide_capacity_and_negative_lengths(gpu):
    """A full cache and a negative length on the wide kernel: both flagged;
    the full sequence writes nothing and attends its max_len stored rows, the
    negative one gives a zero row; the other sequence matches the oracle."""
    lens = [100, 201, 7]
    case = DecodeCase(batch=3, n_q=32, n_kv=1, head_dim=128, dtype="bf16", lengths=lens, t_max=201, tag="widecap",
                      device=gpu)
    ref0 = _oracle_all(case)[0]
    k1, v1, _, _ = case.host[(1, 0)]                  # the 201 stored rows of sequence 1
    ref1 = oracle.decode_attention(case.q_host[1:2], k1[None, None], v1[None, None], np.array([200]),
                                   n_pending=1)[0]
    case.seq_lens.copy_(torch.tensor([100, 201, -3], dtype=torch.int32))
    ws = kvc.workspace(case.k, case.v, 32)
    out = torch.empty((3, 32, 128), device=gpu)
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    k_before = case.k[1].clone()
    kvc.decode_step(case.k, case.v, case.seq_lens, case.k_new, case.v_new, case.q, out, ws, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == kvc.DEVERR_CAPACITY | kvc.DEVERR_BADLEN
    got = out.double().cpu().numpy()
    assert np.abs(got[0] - ref0).max() <= TOL["bf16"]
    assert np.abs(got[1] - ref1).max() <= TOL["bf16"]
    assert (got[2] == 0).all()
    assert torch.equal(case.k[1].view(torch.int16), k_before.view(torch.int16))


def test_wide_spread_merge_rescued_when_splits_give_up(gpu):
    """The spread merge: every split merges one slice of the output once all
    splits have arrived; a split that stops waiting leaves its slice to the
    last one to arrive, which claims and merges every unclaimed slice. With
    the wait bound at zero polls every split but the last gives up at once,
    so the last merges all slices: the outputs must carry no status bit,
    match the oracle and equal, bit for bit, those of the default bound (the
    same fold order), call after call on one workspace."""
    lens = [300, 2047, 4000, 1]
    case = DecodeCase(batch=4, n_q=64, n_kv=1, head_dim=128, dtype="bf16", lengths=lens, tag="widerescue",
                      device=gpu)
    kvc.append(case.k, case.v, case.seq_lens, case.k_new, case.v_new)
    ws = kvc.workspace(case.k, case.v, 64, 8)
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    ref_out = torch.empty((4, 64, 128), device=gpu)
    kvc.decode_attn(case.k, case.v, case.seq_lens, case.q, ref_out, ws, n_pending=1, n_splits=8, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.abs(ref_out.double().cpu().numpy() - _oracle_all(case)).max() <= TOL["bf16"]
    prev = kvc.debug_set_merge_spin_limit(0)
    try:
        for i in range(4):
            out = torch.full((4, 64, 128), float("nan"), device=gpu)
            kvc.decode_attn(case.k, case.v, case.seq_lens, case.q, out, ws, n_pending=1, n_splits=8,
                            status=status)
            torch.cuda.synchronize()
            assert int(status.item()) == 0, i
            assert torch.equal(out, ref_out), i
    finally:
        kvc.debug_set_merge_spin_limit(prev)
    out = torch.empty_like(ref_out)
    kvc.decode_attn(case.k, case.v, case.seq_lens, case.q, out, ws, n_pending=1, n_splits=8, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and torch.equal(out, ref_out)


def test_wide_more_splits_than_the_spread_merge_takes(gpu):
    """More than 32 active splits per (sequence, KV head): the last split
    merges with ready flags instead; outputs against the oracle."""
    lens = [2200, 2400]
    case = DecodeCase(batch=2, n_q=32, n_kv=1, head_dim=64, dtype="fp16", lengths=lens, tag="wide35",
                      device=gpu)
    ws = kvc.workspace(case.k, case.v, 32, 36)
    out = torch.empty((2, 32, 64), device=gpu)
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    for _ in range(2):
        kvc.decode_step(case.k, case.v, case.seq_lens, case.k_new, case.v_new, case.q, out, ws, n_splits=36,
                        status=status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert np.abs(out.double().cpu().numpy() - _oracle_all(case)).max() <= TOL["fp16"]


def test_wide_spread_merge_on_an_oversubscribed_grid(gpu):
    """256 (sequence, KV head) units of 16 pairs at 16 splits each: 4,096
    workgroups, 16 times what the chip holds at once, so splits wait on
    partners dispatched after them. Every slice must still be merged once:
    status stays 0 and sampled units match the oracle."""
    lengths = synth.ragged_lengths(64, 900, 1500, 11, "wideover").tolist()
    sample = [(0, 0), (17, 3), (40, 1), (63, 3)]
    case = DecodeCase(batch=64, n_q=64, n_kv=4, head_dim=128, dtype="bf16", lengths=lengths, tag="wideover",
                      device=gpu, host_rows=sample)
    ws = kvc.workspace(case.k, case.v, 64, 16)
    out = torch.full((64, 64, 128), float("nan"), device=gpu)
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    kvc.decode_step(case.k, case.v, case.seq_lens, case.k_new, case.v_new, case.q, out, ws, n_splits=16,
                    status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    got = out.double().cpu().numpy()
    assert np.isfinite(got).all()
    grp = 16
    for b, g in sample:
        k, v = case.oracle_inputs(b, g)
        ref = oracle.decode_attention(case.q_host[b:b + 1, g * grp:(g + 1) * grp], k[None, None], v[None, None],
                                      np.array([int(case.lengths[b])]), n_pending=1)[0]
        assert np.abs(got[b, g * grp:(g + 1) * grp] - ref).max() <= TOL["bf16"], (b, g)
