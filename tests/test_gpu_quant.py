"""GPU parity of the quantised cache (8-bit codes, one fp32 scale per token and
KV head) through the C ABI: codes and scales written by kvc_quant_append /
kvc_quant_prefill_fill bit-exact against oracle.quantize_rows, decode against
oracle.quant_decode_attention on the codes the device wrote, and the step
equal to append + decode bit for bit."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import kv_cache_append_amd as kvc
import oracle
import synth
from tests.gpu_cases import TOL

pytestmark = pytest.mark.gpu

OFMT = {"fp8": oracle.QFMT_FP8_E4M3, "int8": oracle.QFMT_INT8}
POISON_CODE = 0x7F   # NaN in E4M3; for int8 the NaN scales below poison the row


class QuantCase:
    """Codes [B, H_kv, T_max, D] and scales [B, H_kv, T_max], poisoned, with
    lengths[b] history rows per sequence quantised on the device by
    kvc_quant_prefill_fill; q, k_new, v_new in in_dtype."""

    def __init__(self, *, batch, n_q, n_kv, d, in_dtype, fmt, lengths, t_max=None, seed=31, tag="q",
                 device="cuda"):
        self.n_q, self.n_kv, self.d, self.in_dtype, self.fmt = n_q, n_kv, d, in_dtype, fmt
        self.lengths = np.asarray(lengths, dtype=np.int64)
        self.t_max = int(t_max if t_max is not None else int(self.lengths.max()) + 8)
        self.kc = torch.full((batch, n_kv, self.t_max, d), POISON_CODE, dtype=torch.uint8, device=device)
        self.vc = self.kc.clone()
        self.ks = torch.full((batch, n_kv, self.t_max), float("nan"), dtype=torch.float32, device=device)
        self.vs = self.ks.clone()
        self.desc = kvc.qcache_desc(self.kc, self.vc, self.ks, self.vs, kvc.QFMT[fmt], synth.DTYPES[in_dtype])
        rows = max(int(self.lengths.max()), 1)
        self.k_hist = synth.normal((batch, n_kv, rows, d), in_dtype, seed, tag, "K", device=device)
        self.v_hist = synth.normal((batch, n_kv, rows, d), in_dtype, seed, tag, "V", device=device)
        st = torch.zeros(1, dtype=torch.int32, device=device)
        for b in range(batch):
            n = int(self.lengths[b])
            if n == 0:
                continue
            one = torch.full((batch,), -1, dtype=torch.int32, device=device)   # others skipped (flagged)
            one[b] = 0
            kvc.quant_prefill_fill(self.desc, one, self.k_hist[:, :, :n].contiguous(),
                                   self.v_hist[:, :, :n].contiguous(), status=st)
        self.q = synth.normal((batch, n_q, d), in_dtype, seed, tag, "q", device=device)
        self.k_new = synth.normal((batch, n_kv, d), in_dtype, seed, tag, "kn", device=device)
        self.v_new = synth.normal((batch, n_kv, d), in_dtype, seed, tag, "vn", device=device)
        self.seq_lens = torch.tensor(self.lengths, dtype=torch.int32, device=device)
        torch.cuda.synchronize()

    def host(self):
        return (self.kc.cpu().numpy(), self.ks.cpu().numpy(), self.vc.cpu().numpy(), self.vs.cpu().numpy())

    def oracle_decode(self, n_pending=1):
        kc, ks, vc, vs = self.host()
        return oracle.quant_decode_attention(self.q.cpu(), kc, ks, vc, vs, self.lengths, OFMT[self.fmt],
                                             n_pending=n_pending)

    def decode(self, n_pending=1, n_splits=0, out_dtype=torch.float32, status=None):
        out = torch.empty(self.q.shape, dtype=out_dtype, device=self.q.device)
        ws = kvc.quant_workspace(self.desc, self.n_q, n_splits)
        kvc.quant_decode_attn(self.desc, self.seq_lens, self.q, out, ws, n_pending=n_pending, n_splits=n_splits,
                              status=status)
        torch.cuda.synchronize()
        return out


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("in_dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_quant_fill_and_append_bitwise(gpu, fmt, in_dtype, d):
    """Codes and scales of every written row equal oracle.quantize_rows of the
    same input bits; the appended row lands at slot seq_lens[b]; slots not
    written keep their poison."""
    c = QuantCase(batch=3, n_q=2, n_kv=2, d=d, in_dtype=in_dtype, fmt=fmt, lengths=[0, 5, 33], t_max=40,
                  tag=f"qf{fmt}{in_dtype}{d}")
    st = torch.zeros(1, dtype=torch.int32, device=gpu)
    kvc.quant_append(c.desc, c.seq_lens, c.k_new, c.v_new, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    kc, ks, vc, vs = c.host()
    of = OFMT[fmt]
    for src, codes, scales in ((c.k_hist, kc, ks), (c.v_hist, vc, vs)):
        hist = src.cpu()
        for b, n in enumerate(c.lengths):
            if n:
                want_c, want_s = oracle.quantize_rows(hist[b, :, :n], of)
                assert np.array_equal(codes[b, :, :n], want_c)
                assert np.array_equal(scales[b, :, :n].view(np.uint32), want_s.view(np.uint32))
    for new, codes, scales in ((c.k_new, kc, ks), (c.v_new, vc, vs)):
        want_c, want_s = oracle.quantize_rows(new.cpu(), of)
        for b, n in enumerate(c.lengths):
            assert np.array_equal(codes[b, :, n], want_c[b])
            assert np.array_equal(scales[b, :, n].view(np.uint32), want_s[b].view(np.uint32))
            assert (codes[b, :, n + 1:] == POISON_CODE).all() and np.isnan(scales[b, :, n + 1:]).all()


def test_quant_zero_row_and_extremes(gpu):
    """A row of zeros gets scale 0 and zero codes; a row with one large value
    and tiny others exercises saturation-free top codes and E4M3 subnormals."""
    for fmt in ("fp8", "int8"):
        c = QuantCase(batch=1, n_q=2, n_kv=2, d=128, in_dtype="fp32", fmt=fmt, lengths=[0], t_max=4,
                      tag=f"qz{fmt}")
        kn = torch.zeros((1, 2, 128), device=gpu)
        kn[0, 1, 3] = 1000.0
        kn[0, 1, 4:40] = torch.linspace(-3e-3, 3e-3, 36, device=gpu)
        kvc.quant_append(c.desc, c.seq_lens, kn, kn)
        torch.cuda.synchronize()
        kc, ks, _, _ = c.host()
        want_c, want_s = oracle.quantize_rows(kn.cpu(), OFMT[fmt])
        assert ks[0, 0, 0] == 0 and not kc[0, 0, 0].any()
        assert np.array_equal(kc[0, :, 0], want_c[0]) and np.array_equal(ks[0, :, 0], want_s[0])


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("q_dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (32, 8), (8, 8), (64, 8), (16, 1), (64, 1), (32, 2)])
def test_quant_decode_matches_oracle(gpu, fmt, q_dtype, hq, hkv):
    c = QuantCase(batch=5, n_q=hq, n_kv=hkv, d=128, in_dtype=q_dtype, fmt=fmt, lengths=[0, 1, 37, 300, 1100],
                  tag=f"qd{fmt}{q_dtype}{hq}{hkv}")
    kvc.quant_append(c.desc, c.seq_lens, c.k_new, c.v_new)
    got = c.decode(n_pending=1).double().cpu().numpy()
    assert not np.isnan(got).any()
    assert np.abs(got - c.oracle_decode(n_pending=1)).max() <= TOL[q_dtype]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("hq,hkv", [(64, 1), (32, 2)])
@pytest.mark.parametrize("n_splits", [0, 1, 2, 3])
def test_quant_decode_wide_groups(gpu, fmt, d, hq, hkv, n_splits):
    """Groups of 16+ query heads per KV head run on the wide-group kernel's
    8-bit mode (codes widened to the queries' type in LDS, K scales on the
    scores, V scales on the weights): lengths on and around the 64-key tile
    and empty sequences, one, two (last-split merge), three (spread merge) or
    the library's number of splits, pending rows 0 and 1."""
    q_dtype = "fp16" if d == 64 else "bf16"
    c = QuantCase(batch=6, n_q=hq, n_kv=hkv, d=d, in_dtype=q_dtype, fmt=fmt, lengths=[0, 1, 63, 64, 65, 700],
                  tag=f"qw{fmt}{d}{hq}{hkv}")
    for n_pending in (0, 1):
        if n_pending:
            kvc.quant_append(c.desc, c.seq_lens, c.k_new, c.v_new)
        st = torch.zeros(1, dtype=torch.int32, device=gpu)
        got = c.decode(n_pending=n_pending, n_splits=n_splits, status=st).double().cpu().numpy()
        assert int(st.item()) == 0
        assert np.isfinite(got).all()
        assert np.abs(got - c.oracle_decode(n_pending=n_pending)).max() <= TOL[q_dtype]


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_quant_decode_other_head_dims(gpu, fmt, d):
    c = QuantCase(batch=3, n_q=8, n_kv=2, d=d, in_dtype="bf16", fmt=fmt, lengths=[17, 400, 1024],
                  tag=f"qdd{fmt}{d}")
    got = c.decode(n_pending=0).double().cpu().numpy()
    assert np.abs(got - c.oracle_decode(n_pending=0)).max() <= TOL["bf16"]


@pytest.mark.parametrize("n_splits", [1, 3, 16])
def test_quant_split_counts_and_determinism(gpu, n_splits):
    c = QuantCase(batch=3, n_q=32, n_kv=8, d=128, in_dtype="bf16", fmt="fp8", lengths=[5, 700, 2000],
                  tag=f"qs{n_splits}")
    a = c.decode(n_pending=0, n_splits=n_splits)
    b = c.decode(n_pending=0, n_splits=n_splits)
    assert torch.equal(a, b)
    assert np.abs(a.double().cpu().numpy() - c.oracle_decode(n_pending=0)).max() <= TOL["bf16"]


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (64, 1)])     # the decode kernel (fused); the wide-group kernel
def test_quant_step_equals_append_plus_decode(gpu, fmt, hq, hkv):
    """20 steps: kvc_quant_decode_step leaves the same codes/scales and gives
    the same output bits as kvc_quant_append + kvc_quant_decode_attn."""
    c = QuantCase(batch=3, n_q=hq, n_kv=hkv, d=128, in_dtype="bf16", fmt=fmt, lengths=[0, 30, 250], t_max=280,
                  tag=f"qst{fmt}{hq}")
    kc2, vc2, ks2, vs2 = c.kc.clone(), c.vc.clone(), c.ks.clone(), c.vs.clone()
    d2 = kvc.qcache_desc(kc2, vc2, ks2, vs2, kvc.QFMT[fmt], torch.bfloat16)
    seq2 = c.seq_lens.clone()
    ws1, ws2 = kvc.quant_workspace(c.desc, hq), kvc.quant_workspace(d2, hq)
    for step in range(20):
        kn = synth.normal((3, hkv, 128), "bf16", step, "qst", "kn", device=gpu)
        vn = synth.normal((3, hkv, 128), "bf16", step, "qst", "vn", device=gpu)
        q = synth.normal((3, hq, 128), "bf16", step, "qst", "q", device=gpu)
        o1 = torch.empty((3, hq, 128), device=gpu)
        kvc.quant_decode_step(c.desc, c.seq_lens, kn, vn, q, o1, ws1)
        kvc.seq_lens_advance(c.seq_lens)
        kvc.quant_append(d2, seq2, kn, vn)
        o2 = torch.empty((3, hq, 128), device=gpu)
        kvc.quant_decode_attn(d2, seq2, q, o2, ws2, n_pending=1)
        kvc.seq_lens_advance(seq2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
    assert torch.equal(c.kc, kc2) and torch.equal(c.vc, vc2)
    assert torch.equal(torch.nan_to_num(c.ks), torch.nan_to_num(ks2))


def test_quant_out_in_query_dtype_is_rounded_fp32(gpu):
    c = QuantCase(batch=2, n_q=8, n_kv=2, d=128, in_dtype="fp16", fmt="int8", lengths=[50, 400], tag="qod")
    f32 = c.decode(n_pending=0)
    half = c.decode(n_pending=0, out_dtype=torch.float16)
    assert torch.equal(half, f32.to(torch.float16))


def test_quant_flags_capacity_and_negative_lengths(gpu):
    c = QuantCase(batch=3, n_q=4, n_kv=2, d=128, in_dtype="bf16", fmt="fp8", lengths=[10, 20, 30], t_max=32,
                  tag="qflag")
    before = c.kc.clone()
    st = torch.zeros(1, dtype=torch.int32, device=gpu)
    blk = synth.normal((3, 2, 4, 128), "bf16", 1, "qflag", "blk", device=gpu)
    kvc.quant_prefill_fill(c.desc, c.seq_lens, blk, blk, status=st)      # sequence 2: 30 + 4 > 32
    torch.cuda.synchronize()
    assert int(st.item()) & kvc.DEVERR_CAPACITY
    assert torch.equal(c.kc[2], before[2])
    c.seq_lens[1] = -4
    st.zero_()
    got = c.decode(n_pending=0, status=st)
    assert int(st.item()) & kvc.DEVERR_BADLEN
    assert torch.count_nonzero(got[1]) == 0


def test_quant_decode_at_gqa_8b_shape_sampled(gpu):
    """The 8B GQA decode shape (B=16, 32/8 heads, D=128, T=2048) on an fp8
    cache with bf16 queries and the library's split choice, on sampled
    sequences."""
    c = QuantCase(batch=16, n_q=32, n_kv=8, d=128, in_dtype="bf16", fmt="fp8", lengths=[2048] * 16, t_max=2049,
                  tag="q8b")
    kvc.quant_append(c.desc, c.seq_lens, c.k_new, c.v_new)
    got = c.decode(n_pending=1).double().cpu().numpy()
    kc, ks, vc, vs = c.host()
    q = c.q.cpu()
    for b in (0, 7, 15):
        ref = oracle.quant_decode_attention(q[b:b + 1], kc[b:b + 1], ks[b:b + 1], vc[b:b + 1], vs[b:b + 1],
                                            np.array([2048]), oracle.QFMT_FP8_E4M3, n_pending=1)
        assert np.abs(got[b:b + 1] - ref).max() <= TOL["bf16"]


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_quant_decode_at_mqa_70b_shape_sampled(gpu, fmt):
    """The 70B MQA decode shape (B=32, 64 query heads on one KV head, D=128,
    T=8192) on an 8-bit cache with bf16 queries, the timed step
    (kvc_quant_decode_step: the append, then the wide-group kernel) with the
    library's split choice, on sampled sequences."""
    c = QuantCase(batch=32, n_q=64, n_kv=1, d=128, in_dtype="bf16", fmt=fmt, lengths=[8192] * 32, t_max=8193,
                  tag=f"q70m{fmt}")
    out = torch.empty(c.q.shape, device=gpu)
    st = torch.zeros(1, dtype=torch.int32, device=gpu)
    ws = kvc.quant_workspace(c.desc, 64)
    kvc.quant_decode_step(c.desc, c.seq_lens, c.k_new, c.v_new, c.q, out, ws, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    got = out.double().cpu().numpy()
    kc, ks, vc, vs = c.host()
    q = c.q.cpu()
    for b in (0, 13, 31):
        ref = oracle.quant_decode_attention(q[b:b + 1], kc[b:b + 1], ks[b:b + 1], vc[b:b + 1], vs[b:b + 1],
                                            np.array([8192]), OFMT[fmt], n_pending=1)
        assert np.abs(got[b:b + 1] - ref).max() <= TOL["bf16"]


@pytest.mark.parametrize("fmt,bound", [("fp8", 0.1), ("int8", 0.03)])
def test_quant_decode_stays_close_to_the_unquantised_decode(gpu, fmt, bound):
    """A sanity bound, not parity: attention over the quantised cache stays
    within a loose distance of attention over the original rows."""
    c = QuantCase(batch=2, n_q=8, n_kv=2, d=128, in_dtype="bf16", fmt=fmt, lengths=[300, 900], tag=f"qe{fmt}")
    got = c.decode(n_pending=0).double().cpu().numpy()
    for b, n in enumerate(c.lengths):
        ref = oracle.decode_attention(c.q[b:b + 1].cpu(), c.k_hist[b:b + 1, :, :n].cpu(),
                                      c.v_hist[b:b + 1, :, :n].cpu(), np.array([n]), n_pending=0)
        assert np.abs(got[b:b + 1] - ref).max() < bound
