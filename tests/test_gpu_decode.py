"""Decode-attention parity: libkvc (HIP, through the C ABI) against the fp64
oracle on identical stored inputs.

Bars: max-abs <= 1e-5 for fp32 caches and <= 2e-3 for fp16/bf16 caches
(fp32 output). Every cache row past T_b + 1 holds NaN, so a read outside the
attended range would show as NaN in the output.
"""

import math

import numpy as np
import pytest
import torch

import kv_cache_append_amd as kvc
import oracle
import synth
from tests.gpu_cases import TOL, DecodeCase

pytestmark = pytest.mark.gpu


def _run(case: DecodeCase, n_splits=0, out_dtype=torch.float32, scale=None):
    dev = case.q.device
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    kvc.append(case.k, case.v, case.seq_lens, case.k_new, case.v_new, status=status)
    ws = kvc.workspace(case.k, case.v, case.n_q, n_splits)
    out = torch.empty((case.batch, case.n_q, case.head_dim), dtype=out_dtype, device=dev)
    kvc.decode_attn(case.k, case.v, case.seq_lens, case.q, out, ws, n_pending=1, n_splits=n_splits,
                    scale=scale, status=status)
    torch.cuda.synchronize()
    return out, int(status.item())


def _oracle_unit(case: DecodeCase, b: int, g: int, scale=None):
    grp = case.n_q // case.n_kv
    k, v = case.oracle_inputs(b, g)
    q = case.q_host[b:b + 1, g * grp:(g + 1) * grp]
    return oracle.decode_attention(q, k[None, None], v[None, None], np.array([int(case.lengths[b])]),
                                   n_pending=1, scale=scale)[0]


def _check_all(case: DecodeCase, out: torch.Tensor, scale=None):
    grp = case.n_q // case.n_kv
    got = out.double().cpu().numpy()
    worst = 0.0
    for (b, g) in case.host:
        ref = _oracle_unit(case, b, g, scale)
        err = np.abs(got[b, g * grp:(g + 1) * grp] - ref).max()
        assert np.isfinite(got[b, g * grp:(g + 1) * grp]).all(), (b, g)
        worst = max(worst, err)
    assert worst <= TOL[case.dtype], worst
    return worst


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("n_q,n_kv", [(8, 8), (8, 2), (8, 1), (6, 2), (16, 1), (64, 2)])
def test_decode_matches_oracle_ragged(gpu, dtype, n_q, n_kv):
    """Ragged lengths spanning many tiles, one sequence empty before the step
    (attends only its new token) and lengths on tile edges."""
    lens = [0, 1, 15, 16, 17, 63, 64, 65, 700, 1023]
    case = DecodeCase(batch=len(lens), n_q=n_q, n_kv=n_kv, head_dim=128, dtype=dtype, lengths=lens,
                      tag=f"ragged{n_q}x{n_kv}")
    out, status = _run(case)
    assert status == 0
    _check_all(case, out)


@pytest.mark.parametrize("head_dim", [4, 8, 16, 32, 64, 256])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_decode_other_head_dims(gpu, head_dim, dtype):
    if head_dim == 4 and dtype != "fp32":
        pytest.skip("a 16-bit row of 4 elements is 8 bytes, below the 16-byte lane slice")
    case = DecodeCase(batch=3, n_q=4, n_kv=2, head_dim=head_dim, dtype=dtype, lengths=[5, 300, 77],
                      tag=f"hd{head_dim}")
    out, status = _run(case)
    assert status == 0
    _check_all(case, out)


@pytest.mark.parametrize("n_splits", [1, 2, 7, 64, 256])
def test_split_count_changes_only_rounding(gpu, n_splits):
    """Any split count gives the oracle's result; more splits than tokens leave
    some workgroups empty."""
    case = DecodeCase(batch=2, n_q=8, n_kv=2, head_dim=128, dtype="bf16", lengths=[1500, 31],
                      tag="splits")
    out, _ = _run(case, n_splits=n_splits)
    _check_all(case, out)


def test_run_to_run_bitwise_deterministic(gpu):
    case = DecodeCase(batch=4, n_q=32, n_kv=8, head_dim=128, dtype="bf16", lengths=[900, 1200, 5, 2047],
                      tag="det")
    a, _ = _run(case)
    b, _ = _run(case)       # append writes the same row again; decode re-runs
    assert torch.equal(a, b)


def test_single_token_returns_its_value_exactly(gpu):
    """N = 1 (empty cache + the appended token): o = v_new exactly in fp32."""
    case = DecodeCase(batch=2, n_q=4, n_kv=2, head_dim=128, dtype="fp32", lengths=[0, 0], tag="n1")
    out, _ = _run(case)
    for h in range(4):
        assert torch.equal(out[:, h].cpu(), case.v_new[:, h // 2].cpu())


def test_empty_sequence_gives_zero_row(gpu):
    dev = torch.device("cuda")
    case = DecodeCase(batch=2, n_q=4, n_kv=2, head_dim=128, dtype="bf16", lengths=[0, 9], tag="empty")
    ws = kvc.workspace(case.k, case.v, 4)
    out = torch.full((2, 4, 128), 5.0, device=dev)
    kvc.decode_attn(case.k, case.v, case.seq_lens, case.q, out, ws, n_pending=0)
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0)
    ref = oracle.decode_attention(case.q_host[1:2], case.k[1:2].cpu(), case.v[1:2].cpu(), np.array([9]),
                                  n_pending=0)
    assert np.abs(out[1:2].double().cpu().numpy() - ref).max() <= TOL["bf16"]


def test_capacity_clamp_sets_flag_and_never_reads_past_cache(gpu):
    """seq_lens[b] == T_max: append refuses to write, decode clamps to T_max and
    flags; the output is the attention over the T_max stored rows."""
    dev = torch.device("cuda")
    t_max = 40
    case = DecodeCase(batch=1, n_q=2, n_kv=1, head_dim=64, dtype="fp16", lengths=[t_max], t_max=t_max,
                      tag="cap")
    k_before = case.k.clone()
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    kvc.append(case.k, case.v, case.seq_lens, case.k_new, case.v_new, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == kvc.DEVERR_CAPACITY
    assert torch.equal(case.k.view(torch.int16), k_before.view(torch.int16))
    status.zero_()
    ws = kvc.workspace(case.k, case.v, 2)
    out = torch.empty((1, 2, 64), device=dev)
    kvc.decode_attn(case.k, case.v, case.seq_lens, case.q, out, ws, n_pending=1, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == kvc.DEVERR_CAPACITY
    ref = oracle.decode_attention(case.q_host, case.k.cpu(), case.v.cpu(), np.array([t_max]), n_pending=0)
    assert np.abs(out.double().cpu().numpy() - ref).max() <= TOL["fp16"]
    # a length near 2^31 (its sum with n_pending passes int32) clamps the same way
    status.zero_()
    huge = torch.full_like(case.seq_lens, 2**31 - 1)
    out2 = torch.empty_like(out)
    kvc.decode_attn(case.k, case.v, huge, case.q, out2, ws, n_pending=1, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == kvc.DEVERR_CAPACITY
    assert torch.equal(out2, out)


def test_negative_length_is_flagged_and_treated_as_empty(gpu):
    dev = torch.device("cuda")
    case = DecodeCase(batch=1, n_q=2, n_kv=1, head_dim=128, dtype="bf16", lengths=[3], tag="neg")
    seq = torch.tensor([-5], dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = kvc.workspace(case.k, case.v, 2)
    out = torch.full((1, 2, 128), 3.0, device=dev)
    kvc.decode_attn(case.k, case.v, seq, case.q, out, ws, n_pending=0, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & kvc.DEVERR_BADLEN
    assert torch.all(out == 0)


@pytest.mark.parametrize("n_q", [8, 32])
def test_negative_length_in_the_fused_step_gives_a_zero_row(gpu, n_q):
    """The fused step with a negative length: nothing written, nothing
    attended, a zero row and KVC_DEVERR_BADLEN (group 4 on the 8-head-block
    kernel, group 32 on the wide-group kernel); the other sequence is right."""
    case = DecodeCase(batch=2, n_q=n_q, n_kv=1, head_dim=128, dtype="bf16", lengths=[40, 9], tag=f"negstep{n_q}",
                      device=gpu)
    k, v = case.oracle_inputs(0, 0)
    ref0 = oracle.decode_attention(case.q_host[0:1], k[None, None], v[None, None], np.array([40]), n_pending=1)[0]
    case.seq_lens.copy_(torch.tensor([40, -2], dtype=torch.int32))
    before = case.k[1].clone()
    ws = kvc.workspace(case.k, case.v, n_q)
    out = torch.full((2, n_q, 128), 3.0, device=gpu)
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    kvc.decode_step(case.k, case.v, case.seq_lens, case.k_new, case.v_new, case.q, out, ws, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & kvc.DEVERR_BADLEN
    assert torch.all(out[1] == 0)
    assert torch.equal(case.k[1].view(torch.int16), before.view(torch.int16))
    assert np.abs(out[0].double().cpu().numpy() - ref0).max() <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_output_in_cache_dtype_is_rne_of_fp32_output(gpu, dtype):
    """out_dtype = cache dtype gives exactly the fp32 result rounded to nearest
    even (torch's conversion is the independent reference for the rounding)."""
    case = DecodeCase(batch=3, n_q=8, n_kv=2, head_dim=128, dtype=dtype, lengths=[10, 500, 2000], tag="rne")
    out32, _ = _run(case)
    out16, _ = _run(case, out_dtype=synth.DTYPES[dtype])
    assert torch.equal(out16.cpu().view(torch.int16), out32.to(synth.DTYPES[dtype]).cpu().view(torch.int16))


def test_non_contiguous_cache_layout(gpu):
    """A [B, T, H, D] buffer viewed as [B, H, T, D] (strides passed through)."""
    case = DecodeCase(batch=3, n_q=8, n_kv=4, head_dim=128, dtype="fp16", lengths=[100, 3, 257],
                      tag="bthd", layout="bthd")
    out, _ = _run(case)
    _check_all(case, out)


def test_peaky_and_rising_scores(gpu):
    """Scores with a large spread (q scaled by 8) and keys whose scores rise
    along T, so the running max changes in every tile."""
    dev = torch.device("cuda")
    case = DecodeCase(batch=2, n_q=4, n_kv=1, head_dim=128, dtype="bf16", lengths=[1000, 333], tag="peaky")
    case.q = (case.q.float() * 8).to(torch.bfloat16)
    case.q_host = case.q.cpu()
    ramp = torch.linspace(0, 4, 1000, device=dev)[:, None]
    rising = (case.k[0, 0, :1000].float() * 0.1 + ramp * case.q[0, 0].float()[None] / 8).to(torch.bfloat16)
    case.k[0, 0, :1000] = rising
    case.host[(0, 0)] = (case.k[0, 0, :1000].cpu(),) + case.host[(0, 0)][1:]
    out, _ = _run(case)
    _check_all(case, out)


def test_explicit_scale(gpu):
    case = DecodeCase(batch=2, n_q=4, n_kv=2, head_dim=64, dtype="fp32", lengths=[50, 9], tag="scale")
    out, _ = _run(case, scale=0.3)
    _check_all(case, out, scale=0.3)


# ------------------------------------------- full-size shapes, sampled units --

def _full_size_case(name, rng_units=6):
    cfg = synth.CONFIGS[name]
    lens = cfg.lengths()
    picks = {(0, 0), (cfg.batch - 1, cfg.n_kv_heads - 1)}
    rng = np.random.default_rng(3)
    while len(picks) < rng_units:
        picks.add((int(rng.integers(cfg.batch)), int(rng.integers(cfg.n_kv_heads))))
    return cfg, DecodeCase(batch=cfg.batch, n_q=cfg.n_q_heads, n_kv=cfg.n_kv_heads, head_dim=cfg.head_dim,
                           dtype=cfg.dtype, lengths=lens, tag=name, host_rows=sorted(picks))


@pytest.mark.parametrize("name", ["mha_7b", "gqa_8b", "ragged_long", "gqa_70b", "mqa_70b"])
def test_full_size_layer_sampled_units(gpu, name):
    """One layer at the workload's full shape through the entry point the
    benchmark times, kvc_decode_step (append, then attend T_b + 1 tokens, in
    one launch: course notes "第 1 周 · Day 4" §1.3), with the split count the
    benchmark takes (the length-aware choice for the attended lengths). The
    oracle checks sampled (sequence, KV head) units, all query heads of each;
    the appended rows are checked bit for bit; and the unfused calls
    (kvc_append + kvc_decode_attn, same split count) give the same bits."""
    cfg, case = _full_size_case(name)
    dev = case.q.device
    attended = [int(n) + 1 for n in case.lengths]
    splits = kvc.decode_splits(case.k, case.v, case.n_q, lengths=attended)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = kvc.workspace(case.k, case.v, case.n_q, splits)
    out_step = torch.empty((case.batch, case.n_q, case.head_dim), dtype=torch.float32, device=dev)
    kvc.decode_step(case.k, case.v, case.seq_lens, case.k_new, case.v_new, case.q, out_step, ws,
                    n_splits=splits, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    worst = _check_all(case, out_step)
    for b, g in case.host:
        t = int(case.lengths[b])
        assert torch.equal(case.k[b, g, t].cpu().view(torch.int16), case.host[(b, g)][2].view(torch.int16))
        assert torch.equal(case.v[b, g, t].cpu().view(torch.int16), case.host[(b, g)][3].view(torch.int16))
    out, status2 = _run(case, n_splits=splits)     # appends the same rows again, then attends
    assert status2 == 0
    assert torch.equal(out, out_step)
    print(f"{name}: {splits} split(s), max-abs {worst:.3e} over {len(case.host)} units")


def test_length_aware_split_choice_on_a_very_uneven_batch(gpu):
    """One sequence far longer than the rest: the length-aware choice takes
    many splits (more than the length-blind rule), and the decode with that
    count matches the oracle on every unit."""
    lengths = [20000] + [40] * 7
    case = DecodeCase(batch=8, n_q=32, n_kv=8, head_dim=128, dtype="bf16", lengths=lengths, tag="uneven",
                      device=gpu)
    attended = [n + 1 for n in lengths]
    s_len = kvc.decode_splits(case.k, case.v, case.n_q, lengths=attended)
    s_blind = kvc.decode_splits(case.k, case.v, case.n_q)
    assert s_len > s_blind
    out, status = _run(case, n_splits=s_len)
    assert status == 0
    _check_all(case, out)


def test_many_splits_on_an_oversubscribed_grid(gpu):
    """512 (sequence, KV head) units at 32 splits each: 16,384 active
    workgroups, 32 times what the chip holds at once, so most merging
    workgroups wait on splits dispatched after them on other CUs. No wait
    may time out (status stays 0) and sampled units match the oracle."""
    lengths = synth.ragged_lengths(64, 3000, 4096, 11, "oversub").tolist()
    sample = [(0, 0), (13, 5), (40, 2), (63, 7)]
    case = DecodeCase(batch=64, n_q=32, n_kv=8, head_dim=128, dtype="bf16", lengths=lengths, tag="oversub",
                      device=gpu, host_rows=sample)
    out, status = _run(case, n_splits=32)
    assert status == 0
    grp = case.n_q // case.n_kv
    got = out.double().cpu().numpy()
    for b, g in sample:
        ref = _oracle_unit(case, b, g)
        assert np.abs(got[b, g * grp:(g + 1) * grp] - ref).max() <= TOL["bf16"]
