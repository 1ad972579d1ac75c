"""kvc_decode_step_noalloc (the decode step for callers that cannot allocate:
the split exchange lives in the library's own device array) against
kvc_decode_step with a caller's workspace, through the C ABI: two calls in a
row, the second with a smaller input (another geometry on the same array),
each bit-identical to the workspace entry point with the same split count
(same kernels) and within the bar of the fp64 oracle."""

import ctypes

import numpy as np
import pytest
import torch

import kv_cache_append_amd as kvc
import oracle
from tests.gpu_cases import TOL, DecodeCase

pytestmark = pytest.mark.gpu


def _noalloc(case: DecodeCase, out, n_splits, status):
    kvc.decode_step_noalloc(case.k, case.v, case.seq_lens, case.k_new, case.v_new, case.q, out, n_splits=n_splits,
                            status=status)


@pytest.mark.parametrize("shapes", [
    # (batch, n_q, n_kv, lengths, splits): a large call, then a smaller one
    ((16, 32, 8, [2048] * 16, 0), (3, 8, 2, [5, 300, 77], 3)),
    ((8, 64, 1, [4096] * 8, 0), (2, 32, 1, [100, 1500], 2)),         # wide-group kernel
    ((4, 256, 1, [900] * 4, 0), (2, 160, 1, [100, 1500], 3)),        # wide-group kernel, two pair blocks
])
def test_noalloc_step_equals_workspace_step(gpu, shapes):
    for i, (b, nq, nkv, lens, splits) in enumerate(shapes):
        a = DecodeCase(batch=b, n_q=nq, n_kv=nkv, head_dim=128, dtype="bf16", lengths=lens, tag=f"na{i}{nq}",
                       device=gpu)
        w = DecodeCase(batch=b, n_q=nq, n_kv=nkv, head_dim=128, dtype="bf16", lengths=lens, tag=f"na{i}{nq}",
                       device=gpu)
        s = splits or kvc.decode_splits(w.k, w.v, nq)
        out_a = torch.empty((b, nq, 128), device=gpu)
        out_w = torch.empty_like(out_a)
        st_a = torch.zeros(1, dtype=torch.int32, device=gpu)
        st_w = torch.zeros(1, dtype=torch.int32, device=gpu)
        _noalloc(a, out_a, s, st_a)
        ws = kvc.workspace(w.k, w.v, nq, s)
        kvc.decode_step(w.k, w.v, w.seq_lens, w.k_new, w.v_new, w.q, out_w, ws, n_splits=s, status=st_w)
        torch.cuda.synchronize()
        assert int(st_a.item()) == 0 and int(st_w.item()) == 0
        assert torch.equal(out_a, out_w)
        assert torch.equal(a.k.view(torch.int16), w.k.view(torch.int16))
        assert torch.equal(a.v.view(torch.int16), w.v.view(torch.int16))
        grp = nq // nkv
        got = out_a.double().cpu().numpy()
        for (bb, g) in list(a.host)[:4]:
            k, v = a.oracle_inputs(bb, g)
            ref = oracle.decode_attention(a.q_host[bb:bb + 1, g * grp:(g + 1) * grp], k[None, None], v[None, None],
                                          np.array([lens[bb]]), n_pending=1)[0]
            assert np.abs(got[bb, g * grp:(g + 1) * grp] - ref).max() <= TOL["bf16"]


def test_noalloc_rejects_calls_past_its_array(gpu):
    """A call whose partial results do not fit in the array is refused with
    KVC_ERR_WORKSPACE before anything is enqueued (nothing allocated)."""
    case = DecodeCase(batch=64, n_q=64, n_kv=1, head_dim=128, dtype="bf16", lengths=[300] * 64, tag="nabig",
                      device=gpu)
    out = torch.empty((64, 64, 128), device=gpu)
    lib = kvc.load()
    c = kvc.cache_desc(case.k, case.v)
    vp = ctypes.c_void_p
    rc = lib.kvc_decode_step_noalloc(ctypes.byref(c), vp(case.seq_lens.data_ptr()), vp(case.k_new.data_ptr()),
                                     vp(case.v_new.data_ptr()), case.k_new.stride(0), case.k_new.stride(1),
                                     vp(case.q.data_ptr()), 64, ctypes.c_float(0.0883883), vp(out.data_ptr()), 0, 64,
                                     None, vp(torch.cuda.current_stream().cuda_stream))
    assert rc == 6     # KVC_ERR_WORKSPACE: 64 x 64 x 64 splits x 128 x 4 B of partials is past 16 MiB


def test_noalloc_wide_calls_across_group_sizes(gpu):
    """Wide-group calls whose head-block count changes between calls: the
    merge words of a (sequence, KV head) stay at one place in the array while
    its flag row moves with the geometry, so the spread merge's claims must be
    compared with an epoch kept beside them. Every call, after three calls of
    another geometry, equals the workspace entry point bit for bit and is
    within the oracle's bar."""
    lens = [700, 1300, 64, 999]
    for i, grp in enumerate([16, 16, 16, 64, 16, 32]):
        nq = 2 * grp
        a = DecodeCase(batch=4, n_q=nq, n_kv=2, head_dim=128, dtype="bf16", lengths=lens, tag=f"nag{i}", device=gpu)
        w = DecodeCase(batch=4, n_q=nq, n_kv=2, head_dim=128, dtype="bf16", lengths=lens, tag=f"nag{i}", device=gpu)
        out_a = torch.full((4, nq, 128), float("nan"), device=gpu)
        out_w = torch.empty_like(out_a)
        st_a = torch.zeros(1, dtype=torch.int32, device=gpu)
        st_w = torch.zeros(1, dtype=torch.int32, device=gpu)
        _noalloc(a, out_a, 4, st_a)
        ws = kvc.workspace(w.k, w.v, nq, 4)
        kvc.decode_step(w.k, w.v, w.seq_lens, w.k_new, w.v_new, w.q, out_w, ws, n_splits=4, status=st_w)
        torch.cuda.synchronize()
        print(f"call {i}: group {grp}", flush=True)
        assert int(st_a.item()) == 0 and int(st_w.item()) == 0
        assert torch.equal(out_a, out_w)
        got = out_a.double().cpu().numpy()
        for (bb, g) in [(0, 1), (1, 0), (3, 1)]:
            k, v = a.oracle_inputs(bb, g)
            ref = oracle.decode_attention(a.q_host[bb:bb + 1, g * grp:(g + 1) * grp], k[None, None], v[None, None],
                                          np.array([lens[bb]]), n_pending=1)[0]
            assert np.abs(got[bb, g * grp:(g + 1) * grp] - ref).max() <= TOL["bf16"]
