"""GPU parity of the paged cache (page pool + per-sequence page table) through
the C ABI: paged fill/append bit-exact against the oracle, paged decode
against oracle.paged_decode_attention and bit-identical to the contiguous
decode of the same logical cache, and the fused paged step."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import kv_cache_append_amd as kvc
import oracle
import synth
from tests.gpu_cases import TOL, poison_

pytestmark = pytest.mark.gpu


def _table(batch, per_seq, n_pages, seed, device):
    """A random permutation of pool pages handed out to the sequences."""
    perm = np.random.default_rng(seed).permutation(n_pages)[:batch * per_seq]
    return torch.tensor(perm.reshape(batch, per_seq), dtype=torch.int32, device=device)


class PagedCase:
    """A contiguous logical cache (the reference) and the same rows scattered
    into a NaN-poisoned page pool through a random page table with kvc_paged_prefill_fill."""

    def __init__(self, *, batch, n_q, n_kv, d, dtype, lengths, page, spare_pages=5, seed=21, tag="pg",
                 device="cuda", token_major=False, cap_tokens=None):
        self.n_q, self.n_kv, self.dtype, self.page = n_q, n_kv, dtype, page
        self.lengths = torch.as_tensor(lengths, dtype=torch.int32)
        cap = cap_tokens if cap_tokens is not None else int(self.lengths.max()) + 8
        self.per_seq = -(-cap // page)
        self.t_max = self.per_seq * page
        self.n_pages = batch * self.per_seq + spare_pages
        tdt = synth.DTYPES[dtype]
        if token_major:   # pool stored [n_pages, P, H_kv, D], viewed as [n_pages, H_kv, P, D]
            self.kp = torch.empty((self.n_pages, page, n_kv, d), dtype=tdt, device=device).transpose(1, 2)
            self.vp = torch.empty((self.n_pages, page, n_kv, d), dtype=tdt, device=device).transpose(1, 2)
        else:
            self.kp = torch.empty((self.n_pages, n_kv, page, d), dtype=tdt, device=device)
            self.vp = torch.empty_like(self.kp)
        poison_(self.kp)
        poison_(self.vp)
        self.table = _table(batch, self.per_seq, self.n_pages, seed, device)
        # contiguous reference cache with the same logical rows
        self.k = poison_(torch.empty((batch, n_kv, self.t_max, d), dtype=tdt, device=device))
        self.v = poison_(torch.empty_like(self.k))
        rows = max(int(self.lengths.max()), 1)
        self.kfull = synth.normal((batch, n_kv, rows, d), dtype, seed, tag, "K", device=device)
        self.vfull = synth.normal((batch, n_kv, rows, d), dtype, seed, tag, "V", device=device)
        zero = torch.zeros(batch, dtype=torch.int32, device=device)
        for b in range(batch):
            n = int(self.lengths[b])
            self.k[b, :, :n] = self.kfull[b, :, :n]
            self.v[b, :, :n] = self.vfull[b, :, :n]
        # scatter through the ABI, one sequence length at a time (lengths differ)
        for b in range(batch):
            n = int(self.lengths[b])
            if n == 0:
                continue
            one = torch.zeros(batch, dtype=torch.int32, device=device)
            one.fill_(self.t_max)         # other sequences: past capacity, skipped (and flagged)
            one[b] = 0
            st = torch.zeros(1, dtype=torch.int32, device=device)
            kvc.paged_prefill_fill(self.kp, self.vp, self.table, one, self.kfull[:, :, :n].contiguous(),
                                   self.vfull[:, :, :n].contiguous(), status=st)
        del zero
        self.q = synth.normal((batch, n_q, d), dtype, seed, tag, "q", device=device)
        self.k_new = synth.normal((batch, n_kv, d), dtype, seed, tag, "kn", device=device)
        self.v_new = synth.normal((batch, n_kv, d), dtype, seed, tag, "vn", device=device)
        self.seq_lens = self.lengths.to(device)
        torch.cuda.synchronize()


def _paged_out(c: PagedCase, n_pending=1, n_splits=0, status=None):
    out = torch.empty((c.q.shape[0], c.n_q, c.q.shape[2]), device=c.q.device)
    ws = kvc.paged_workspace(c.kp, c.vp, c.table, c.n_q, n_splits)
    kvc.paged_decode_attn(c.kp, c.vp, c.table, c.seq_lens, c.q, out, ws, n_pending=n_pending, n_splits=n_splits,
                          status=status)
    torch.cuda.synchronize()
    return out


def _contig_out(c: PagedCase, n_pending=1, n_splits=0):
    out = torch.empty((c.q.shape[0], c.n_q, c.q.shape[2]), device=c.q.device)
    ws = kvc.workspace(c.k, c.v, c.n_q, n_splits)
    kvc.decode_attn(c.k, c.v, c.seq_lens, c.q, out, ws, n_pending=n_pending, n_splits=n_splits)
    torch.cuda.synchronize()
    return out


def test_paged_fill_places_rows_through_the_table(gpu):
    c = PagedCase(batch=3, n_q=4, n_kv=2, d=128, dtype="bf16", lengths=[20, 0, 77], page=16, tag="pgfill")
    table = c.table.cpu().tolist()
    kp = c.kp.cpu().float().numpy()
    for b in range(3):
        n = int(c.lengths[b])
        view = oracle.paged_view(kp, table, n, lengths=[n] * 3)[b]
        assert np.array_equal(view, c.kfull[b, :, :n].cpu().float().numpy())


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("page", [16, 64, 256])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (32, 8), (8, 8), (16, 1), (8, 1), (32, 2), (64, 1), (128, 1), (512, 2)])
def test_paged_decode_matches_oracle_and_contiguous(gpu, dtype, page, hq, hkv):
    c = PagedCase(batch=3, n_q=hq, n_kv=hkv, d=128, dtype=dtype, lengths=[0, 300, 1100], page=page,
                  tag=f"pg{dtype}{page}{hq}{hkv}")
    # the block just appended is the slot after the cached rows: fill it in both caches
    lens1 = c.seq_lens
    kvc.paged_append(c.kp, c.vp, c.table, lens1, c.k_new, c.v_new)
    kvc.append(c.k, c.v, lens1, c.k_new, c.v_new)
    got = _paged_out(c)
    ref_c = _contig_out(c)
    # paging changes where rows live, not the result: the same kernel (the
    # wide-group kernel from 8 query heads per KV head on) gives the same bits
    assert torch.equal(got, ref_c)
    table = c.table.cpu().tolist()
    ref = oracle.paged_decode_attention(c.q.cpu(), c.kp.cpu(), c.vp.cpu(), table, c.lengths.numpy(), n_pending=1)
    assert np.abs(got.double().cpu().numpy() - ref).max() <= TOL[dtype]


@pytest.mark.parametrize("n_splits", [1, 3, 16])
@pytest.mark.parametrize("hq", [8, 32])
def test_paged_split_counts_and_token_major_pool(gpu, n_splits, hq):
    c = PagedCase(batch=2, n_q=hq, n_kv=2, d=128, dtype="bf16", lengths=[513, 40], page=32,
                  tag=f"pgs{n_splits}{hq}", token_major=True)
    got = _paged_out(c, n_pending=0, n_splits=n_splits)
    assert torch.equal(got, _contig_out(c, n_pending=0, n_splits=n_splits))


@pytest.mark.parametrize("d,hq", [(64, 8), (256, 8), (64, 32)])
def test_paged_other_head_dims(gpu, d, hq):
    c = PagedCase(batch=2, n_q=hq, n_kv=2, d=d, dtype="fp16", lengths=[100, 700], page=16, tag=f"pgd{d}{hq}")
    assert torch.equal(_paged_out(c, n_pending=0), _contig_out(c, n_pending=0))


@pytest.mark.parametrize("hq,hkv", [(8, 2), (64, 1), (256, 1)])
def test_paged_step_equals_append_plus_decode_over_many_steps(gpu, hq, hkv):
    """Fused paged step, 40 steps crossing page boundaries (P = 16): cache and
    output bit-identical to paged append + paged decode, and the pool matches
    the oracle's paged append. 64 and 256 query heads on one KV head run on
    the wide-group kernel (256: two pair blocks, the first writing the row)."""
    c = PagedCase(batch=3, n_q=hq, n_kv=hkv, d=128, dtype="bf16", lengths=[5, 31, 200], page=16,
                  tag=f"pgstep{hq}", cap_tokens=260)
    kp2, vp2 = c.kp.clone(), c.vp.clone()
    seq2 = c.seq_lens.clone()
    ws1 = kvc.paged_workspace(c.kp, c.vp, c.table, hq)
    ws2 = kvc.paged_workspace(c.kp, c.vp, c.table, hq)
    table = c.table.cpu().tolist()
    for step in range(40):
        kn = synth.normal((3, hkv, 128), "bf16", step, "pgstep", "kn", device=gpu)
        vn = synth.normal((3, hkv, 128), "bf16", step, "pgstep", "vn", device=gpu)
        q = synth.normal((3, hq, 128), "bf16", step, "pgstep", "q", device=gpu)
        before = (c.kp.cpu().float().numpy(), c.vp.cpu().float().numpy(), c.seq_lens.cpu().numpy())
        o1 = torch.empty((3, hq, 128), device=gpu)
        kvc.paged_decode_step(c.kp, c.vp, c.table, c.seq_lens, kn, vn, q, o1, ws1)
        kvc.seq_lens_advance(c.seq_lens)
        kvc.paged_append(kp2, vp2, c.table, seq2, kn, vn)
        o2 = torch.empty((3, hq, 128), device=gpu)
        kvc.paged_decode_attn(kp2, vp2, c.table, seq2, q, o2, ws2, n_pending=1)
        kvc.seq_lens_advance(seq2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
        if step % 13 == 0:
            kw, vw, _ = oracle.paged_append(before[0], before[1], table, before[2], kn.cpu().float().numpy(),
                                            vn.cpu().float().numpy())
            assert np.array_equal(np.nan_to_num(c.kp.cpu().float().numpy(), nan=7e7), np.nan_to_num(kw, nan=7e7))
    assert torch.equal(c.kp.view(torch.int16), kp2.view(torch.int16))


@pytest.mark.parametrize("dtype,d", [("fp32", 4), ("fp16", 40), ("bf16", 128)])
def test_paged_append_bitwise_any_dtype(gpu, dtype, d):
    c = PagedCase(batch=3, n_q=2, n_kv=2, d=d, dtype=dtype, lengths=[0, 15, 16], page=16, tag=f"pga{dtype}{d}")
    before_k, before_v = c.kp.cpu(), c.vp.cpu()
    kvc.paged_append(c.kp, c.vp, c.table, c.seq_lens, c.k_new, c.v_new)
    torch.cuda.synchronize()
    kw, vw, flagged = oracle.paged_append(before_k.float().numpy(), before_v.float().numpy(), c.table.cpu().tolist(),
                                          c.lengths.numpy(), c.k_new.cpu().float().numpy(),
                                          c.v_new.cpu().float().numpy())
    assert not flagged.any()
    got = c.kp.cpu().float().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(kw))
    assert np.array_equal(np.nan_to_num(got), np.nan_to_num(kw))


@pytest.mark.parametrize("hq", [4, 32])
def test_bad_page_is_flagged_and_not_written(gpu, hq):
    c = PagedCase(batch=2, n_q=hq, n_kv=2, d=128, dtype="bf16", lengths=[16, 3], page=16, tag=f"pgbad{hq}")
    c.table[0, 1] = c.n_pages + 5                   # slot 16 of sequence 0 points outside the pool
    before = c.kp.clone()
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    kvc.paged_append(c.kp, c.vp, c.table, c.seq_lens, c.k_new, c.v_new, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & kvc.DEVERR_PAGE
    t1 = int(c.table[1, 0])
    changed = (c.kp.view(torch.int16) != before.view(torch.int16)).nonzero()
    assert set(changed[:, 0].tolist()) == {t1}       # only sequence 1's page was written
    status.zero_()
    _paged_out(c, n_pending=1, status=status)         # sequence 0 reads its bad page as zeros, reported
    assert int(status.item()) & kvc.DEVERR_PAGE
