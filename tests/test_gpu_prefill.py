"""GPU parity of kvc_prefill_attn (long blocks of new queries, the lower-right
causal mask, matrix-core tiles) against oracle.chunk_attention, through the
C ABI. The block's K/V rows are written with kvc_prefill_fill first."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import kv_cache_append_amd as kvc
import oracle
from tests.gpu_cases import TOL
from tests.test_gpu_block import BlockCase

pytestmark = pytest.mark.gpu


def _run(case: BlockCase, out_dtype=torch.float32, status=None):
    out = torch.full(case.q.shape, float("nan"), dtype=out_dtype, device=case.q.device)
    kvc.prefill_attn(case.k, case.v, case.seq_lens, case.q, out, status=status)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("batch,hq,hkv", [(3, 8, 2), (3, 8, 8), (2, 8, 1), (3, 32, 8), (4, 4, 2)])
def test_prefill_matches_oracle(gpu, dtype, batch, hq, hkv):
    """Two query tiles (128 + a ragged 72), cached prefixes of 0, 37 and 300
    rows (keys not a multiple of the 64-key tile), MHA/GQA/MQA; unit counts of
    6, 24, 2 and 8 take both workgroup orders."""
    lengths = [0, 37, 300, 5][:batch]
    case = BlockCase(batch=batch, n_q=hq, n_kv=hkv, d=128, dtype=dtype, lengths=lengths, t_q=200,
                     tag=f"pf{dtype}{batch}{hq}{hkv}")
    case.fill()
    got = _run(case).double().cpu().numpy()
    ref = case.oracle()
    assert not np.isnan(got).any()
    assert np.abs(got - ref).max() <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_prefill_head_dim_64(gpu, dtype):
    case = BlockCase(batch=2, n_q=8, n_kv=2, d=64, dtype=dtype, lengths=[11, 190], t_q=150, tag=f"pf64{dtype}")
    case.fill()
    assert np.abs(_run(case).double().cpu().numpy() - case.oracle()).max() <= TOL[dtype]


@pytest.mark.parametrize("t_q", [1, 2, 63, 64, 65, 127, 128, 129, 256])
def test_prefill_block_lengths_on_tile_edges(gpu, t_q):
    """Blocks on and around the 64-key and 128-query tile edges, over cached
    prefixes that also sit on and around them."""
    case = BlockCase(batch=4, n_q=8, n_kv=2, d=128, dtype="bf16", lengths=[0, 63, 64, 129], t_q=t_q,
                     tag=f"pfe{t_q}")
    case.fill()
    assert np.abs(_run(case).double().cpu().numpy() - case.oracle()).max() <= TOL["bf16"]


def test_prefill_whole_prompt_is_causal_attention(gpu):
    """Nothing cached before the block: the causal prefill of a 1000-token
    prompt over several query tiles, against the oracle's causal attention."""
    case = BlockCase(batch=1, n_q=4, n_kv=1, d=128, dtype="fp16", lengths=[0], t_q=1000, tag="pfprompt")
    case.fill()
    got = _run(case).double().cpu().numpy()[0]                 # [T, H_q, D]
    ref = oracle.causal_attention(case.q_host[0].permute(1, 0, 2), case.kb_host[0], case.vb_host[0], 4, 1)
    assert np.abs(got - np.transpose(ref, (1, 0, 2))).max() <= TOL["fp16"]


def test_prefill_equals_block_attn_within_tolerance(gpu):
    """kvc_prefill_attn and kvc_block_attn compute the same thing: both sit
    within the bf16 bar of the oracle, so within twice it of each other. A
    block of 7 queries at group 4 (28 (query, head) pairs per KV head) runs
    on the wide-group kernel in kvc_block_attn (only blocks of 8+ queries
    and 32+ pairs that kernel does not take go to the prefill kernel), and
    500 cached tokens span several 64-key tiles of the prefill kernel, so two
    different kernels are compared."""
    t_q = 7
    case = BlockCase(batch=2, n_q=8, n_kv=2, d=128, dtype="bf16", lengths=[17, 500], t_q=t_q, tag="pfblk")
    case.fill()
    ref = case.oracle()
    a = _run(case)
    b = torch.empty_like(a)
    ws = kvc.block_workspace(case.k, case.v, 8, t_q)
    kvc.block_attn(case.k, case.v, case.seq_lens, case.q, b, ws)
    torch.cuda.synchronize()
    assert np.abs(a.double().cpu().numpy() - ref).max() <= TOL["bf16"]
    assert np.abs(b.double().cpu().numpy() - ref).max() <= TOL["bf16"]
    assert (a - b).abs().max().item() <= 2 * TOL["bf16"]


def test_prefill_blocks_that_do_not_fit_are_zero_and_flagged(gpu):
    """A block past max_len and a negative length give zero rows and set
    KVC_DEVERR_CAPACITY and KVC_DEVERR_BADLEN; the other sequences are right."""
    case = BlockCase(batch=3, n_q=8, n_kv=2, d=128, dtype="bf16", lengths=[10, 40, 20], t_q=100, t_max=140,
                     tag="pfbad")
    case.fill()
    ref = case.oracle()[0]
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    case.seq_lens.copy_(torch.tensor([10, 41, -1], dtype=torch.int32))   # 41 + 100 > 140
    got = _run(case, status=status).double().cpu().numpy()
    assert int(status.item()) == kvc.DEVERR_CAPACITY | kvc.DEVERR_BADLEN
    assert np.abs(got[0] - ref).max() <= TOL["bf16"]
    assert (got[1] == 0).all() and (got[2] == 0).all()
    # a length whose sum with t_q passes 2^31 is a capacity error too
    status.zero_()
    case.seq_lens.copy_(torch.tensor([10, 2**31 - 5, 20], dtype=torch.int32))
    got = _run(case, status=status).double().cpu().numpy()
    assert int(status.item()) == kvc.DEVERR_CAPACITY
    assert (got[1] == 0).all() and np.abs(got[0] - ref).max() <= TOL["bf16"]


def test_prefill_out_in_cache_dtype_is_rounded_fp32(gpu):
    case = BlockCase(batch=2, n_q=8, n_kv=2, d=128, dtype="fp16", lengths=[50, 400], t_q=130, tag="pfod")
    case.fill()
    f32 = _run(case)
    half = _run(case, out_dtype=torch.float16)
    assert torch.equal(half, f32.to(torch.float16))


def test_prefill_run_to_run_deterministic(gpu):
    case = BlockCase(batch=2, n_q=32, n_kv=8, d=128, dtype="bf16", lengths=[100, 900], t_q=300, tag="pfdet")
    case.fill()
    assert torch.equal(_run(case), _run(case))


# The timed prefill workload: 16 prompts of 2048 tokens, 32 query heads over
# 8 KV heads, head dim 128, bf16 (an 8B-shaped layer).
PREFILL_SHAPE = dict(batch=16, n_q=32, n_kv=8, d=128, dtype="bf16", t_q=2048)


def test_prefill_full_size_sampled_rows(gpu):
    """The timed prefill workload in the timed launch configuration: sampled
    (sequence, query, head) rows against the oracle, each computed on its own
    as a one-query block over that query's prefix."""
    case = BlockCase(lengths=[0] * PREFILL_SHAPE["batch"], tag="pffull", **PREFILL_SHAPE)
    case.fill()
    got = _run(case)
    assert not torch.isnan(got).any()
    rng = np.random.default_rng(5)
    samples = [(0, 0, 0), (15, 2047, 31), (7, 1023, 5), (3, 127, 8), (3, 128, 9)]
    samples += [tuple(int(x) for x in rng.integers([0, 0, 0], [16, 2048, 32])) for _ in range(11)]
    for b, i, h in samples:
        ref = oracle.chunk_attention(case.q_host[b:b + 1, i:i + 1], case.kb_host[b:b + 1], case.vb_host[b:b + 1],
                                     np.array([i]))[0, 0, h]
        assert np.abs(got[b, i, h].double().cpu().numpy() - ref).max() <= TOL["bf16"], (b, i, h)


def test_prefill_token_major_cache_equals_head_major_bitwise(gpu):
    """A token-major cache ([B, T, H_kv, D] storage seen as [B, H_kv, T, D]
    through strides) gives the same bits as the head-major cache: only the
    addressing differs."""
    case = BlockCase(batch=2, n_q=8, n_kv=2, d=128, dtype="bf16", lengths=[30, 200], t_q=150, tag="pftm")
    case.fill()
    ref = _run(case)
    b, h, t, d = case.k.shape
    k_tm = torch.full((b, t, h, d), float("nan"), dtype=case.k.dtype, device=gpu).permute(0, 2, 1, 3)
    v_tm = torch.full_like(k_tm, float("nan"))
    k_tm.copy_(case.k)
    v_tm.copy_(case.v)
    out = torch.full_like(ref, float("nan"))
    kvc.prefill_attn(k_tm, v_tm, case.seq_lens, case.q, out)
    torch.cuda.synchronize()
    assert k_tm.stride(2) == h * d
    assert torch.equal(out, ref)


@pytest.mark.parametrize("hq,hkv,t_q", [(32, 2, 40), (8, 8, 80), (8, 2, 72), (64, 1, 16)])
def test_long_blocks_of_block_attn_run_on_the_prefill_kernel(gpu, hq, hkv, t_q):
    """kvc_block_attn hands blocks of >= 8 queries with >= 32 (query, head)
    pairs per KV head that the wide-group kernel does not take (more than
    512 pairs, or more than 64 queries) to the prefill kernel: the same bits
    as kvc_prefill_attn, and within the bar of the oracle."""
    case = BlockCase(batch=2, n_q=hq, n_kv=hkv, d=128, dtype="bf16", lengths=[70, 1000], t_q=t_q,
                     tag=f"pfroute{hq}{hkv}{t_q}")
    case.fill()
    direct = _run(case)
    routed = torch.full_like(direct, float("nan"))
    ws = kvc.block_workspace(case.k, case.v, hq, t_q)
    kvc.block_attn(case.k, case.v, case.seq_lens, case.q, routed, ws)
    torch.cuda.synchronize()
    assert torch.equal(routed, direct)
    assert np.abs(routed.double().cpu().numpy() - case.oracle()).max() <= TOL["bf16"]
