"""kvc_decode_step (append fused into the decode launch), multi-step use of one
workspace, and replay of a captured HIP graph of whole decode steps."""

import numpy as np
import pytest
import torch

import kv_cache_append_amd as kvc
import oracle
import synth
from tests.gpu_cases import TOL, DecodeCase

pytestmark = pytest.mark.gpu

INT_VIEW = {"fp32": torch.int32, "fp16": torch.int16, "bf16": torch.int16}


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("n_q,n_kv", [(8, 2), (4, 4), (16, 1)])
def test_step_equals_append_then_decode(gpu, dtype, n_q, n_kv):
    """Same cache bytes (every slot, poison included) and bit-identical outputs
    as kvc_append followed by kvc_decode_attn(n_pending=1)."""
    lens = [0, 1, 63, 64, 65, 300, 1000]
    a = DecodeCase(batch=len(lens), n_q=n_q, n_kv=n_kv, head_dim=128, dtype=dtype, lengths=lens, tag="stepeq")
    b = DecodeCase(batch=len(lens), n_q=n_q, n_kv=n_kv, head_dim=128, dtype=dtype, lengths=lens, tag="stepeq")
    ws_a = kvc.workspace(a.k, a.v, n_q)
    ws_b = kvc.workspace(b.k, b.v, n_q)
    out_a = torch.empty((a.batch, n_q, 128), device=gpu)
    out_b = torch.empty_like(out_a)
    kvc.append(a.k, a.v, a.seq_lens, a.k_new, a.v_new)
    kvc.decode_attn(a.k, a.v, a.seq_lens, a.q, out_a, ws_a, n_pending=1)
    kvc.decode_step(b.k, b.v, b.seq_lens, b.k_new, b.v_new, b.q, out_b, ws_b)
    torch.cuda.synchronize()
    iv = INT_VIEW[dtype]
    assert torch.equal(a.k.view(iv), b.k.view(iv)) and torch.equal(a.v.view(iv), b.v.view(iv))
    assert torch.equal(out_a, out_b)
    grp = n_q // n_kv
    got = out_b.double().cpu().numpy()
    for (bb, g) in b.host:
        k, v = b.oracle_inputs(bb, g)
        ref = oracle.decode_attention(b.q_host[bb:bb + 1, g * grp:(g + 1) * grp], k[None, None], v[None, None],
                                      np.array([lens[bb]]), n_pending=1)[0]
        assert np.abs(got[bb, g * grp:(g + 1) * grp] - ref).max() <= TOL[dtype]


def _host_layer(k, v, lens):
    return k.cpu().clone(), v.cpu().clone()


def test_many_steps_many_layers_one_workspace(gpu):
    """Three layers, eight steps, one shared workspace (its merge epochs move
    on with every launch and no flag is ever cleared); every output against
    the oracle on host copies that follow the appends."""
    L, B, hq, hkv, d = 3, 4, 8, 2, 128
    lens0 = [5, 130, 0, 513]
    t_max = max(lens0) + 9
    caches = [DecodeCase(batch=B, n_q=hq, n_kv=hkv, head_dim=d, dtype="bf16", lengths=lens0, t_max=t_max,
                         tag=f"ml{l}") for l in range(L)]
    host = [(c.k.cpu().clone(), c.v.cpu().clone()) for c in caches]
    seq = torch.tensor(lens0, dtype=torch.int32, device=gpu)
    ws = kvc.workspace(caches[0].k, caches[0].v, hq)
    lens = np.array(lens0)
    for step in range(8):
        outs = []
        for l, c in enumerate(caches):
            kn = synth.normal((B, hkv, d), "bf16", 9, "ml", l, step, "k", device=gpu)
            vn = synth.normal((B, hkv, d), "bf16", 9, "ml", l, step, "v", device=gpu)
            q = synth.normal((B, hq, d), "bf16", 9, "ml", l, step, "q", device=gpu)
            out = torch.empty((B, hq, d), device=gpu)
            kvc.decode_step(c.k, c.v, seq, kn, vn, q, out, ws)
            outs.append((out, q.cpu(), kn.cpu(), vn.cpu()))
        kvc.seq_lens_advance(seq, 1)
        torch.cuda.synchronize()
        # two splits per (sequence, KV head) here; sequences 1 and 3 merge in
        # every call (3 layers per step), 0 and 2 are short enough for one
        # split: each merge raised the publisher's flag to the block's epoch
        # + 1 and then advanced the epoch (word 1), and nothing else moved
        words = ws[:64].view(torch.int32).cpu().view(B * hkv, 2)
        merges = [L * (step + 1) if b in (1, 3) else 0 for b in range(B) for _ in range(hkv)]
        assert words[:, 1].tolist() == merges and words[:, 0].tolist() == merges
        for l, (out, q, kn, vn) in enumerate(outs):
            hk, hv = host[l]
            for bb in range(B):
                hk[bb, :, lens[bb]] = kn[bb]
                hv[bb, :, lens[bb]] = vn[bb]
            ref = oracle.decode_attention(q, hk, hv, lens, n_pending=1)
            assert np.abs(out.double().cpu().numpy() - ref).max() <= TOL["bf16"], (step, l)
        lens = lens + 1
    assert seq.tolist() == list(lens)


def test_workspace_reused_across_shapes(gpu):
    """A workspace sized for the larger of two shapes serves both, alternately,
    when it is zero-filled again at each change of geometry."""
    big = DecodeCase(batch=6, n_q=32, n_kv=8, head_dim=128, dtype="fp16", lengths=[700] * 6, tag="wsbig")
    small = DecodeCase(batch=2, n_q=4, n_kv=1, head_dim=128, dtype="fp16", lengths=[90, 2000], tag="wssmall")
    n = max(kvc.decode_workspace_bytes(big.k, big.v, 32), kvc.decode_workspace_bytes(small.k, small.v, 4))
    ws = torch.zeros(n, dtype=torch.uint8, device=gpu)
    for rep in range(3):
        for c, hq in ((big, 32), (small, 4)):
            ws.zero_()
            out = torch.empty((c.batch, hq, 128), device=gpu)
            kvc.decode_attn(c.k, c.v, c.seq_lens, c.q, out, ws, n_pending=0)
            torch.cuda.synchronize()
            grp = hq // c.n_kv
            for (bb, g) in list(c.host)[:4]:
                k_old, v_old, _, _ = c.host[(bb, g)]
                ref = oracle.decode_attention(c.q_host[bb:bb + 1, g * grp:(g + 1) * grp], k_old[None, None],
                                              v_old[None, None], np.array([int(c.lengths[bb])]), n_pending=0)[0]
                assert np.abs(out[bb, g * grp:(g + 1) * grp].double().cpu().numpy() - ref).max() <= TOL["fp16"]


def test_step_full_cache_is_flagged_and_not_written(gpu):
    t_max = 50
    c = DecodeCase(batch=2, n_q=4, n_kv=2, head_dim=128, dtype="bf16", lengths=[t_max, 10], t_max=t_max, tag="full")
    before = c.k.clone()
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    ws = kvc.workspace(c.k, c.v, 4)
    out = torch.empty((2, 4, 128), device=gpu)
    kvc.decode_step(c.k, c.v, c.seq_lens, c.k_new, c.v_new, c.q, out, ws, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == kvc.DEVERR_CAPACITY
    assert torch.equal(c.k[0].view(torch.int16), before[0].view(torch.int16))      # full: untouched
    assert torch.equal(c.k[1, :, 10].view(torch.int16), c.k_new[1].view(torch.int16))
    ref = oracle.decode_attention(c.q_host[:1], before[:1].cpu(), c.v[:1].cpu(), np.array([t_max]), n_pending=0)
    assert np.abs(out[:1].double().cpu().numpy() - ref).max() <= TOL["bf16"]


def _graph_setup(device, tag):
    L, B, hq, hkv, d = 4, 3, 16, 4, 128
    lens = [200, 7, 1000]
    cases = [DecodeCase(batch=B, n_q=hq, n_kv=hkv, head_dim=d, dtype="bf16", lengths=lens, t_max=1040,
                        tag=f"{tag}{l}") for l in range(L)]
    seq = torch.tensor(lens, dtype=torch.int32, device=device)
    ws = kvc.workspace(cases[0].k, cases[0].v, hq)
    outs = [torch.zeros((B, hq, d), device=device) for _ in range(L)]
    return cases, seq, ws, outs


def _one_step(cases, seq, ws, outs):
    for c, out in zip(cases, outs):
        kvc.decode_step(c.k, c.v, seq, c.k_new, c.v_new, c.q, out, ws)
    kvc.seq_lens_advance(seq, 1)


def test_hip_graph_replay_matches_eager(gpu):
    """A captured graph of whole steps (4 layers + advance), replayed 6 times
    with eager work and synchronisations between replays, gives the same bits
    as the same steps launched eagerly on an identical copy."""
    eager = _graph_setup(gpu, "g")
    graphed = _graph_setup(gpu, "g")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            _one_step(*graphed)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    # capture did not run the kernels: the graphed copy still equals the initial state
    assert graphed[1].tolist() == [200, 7, 1000]
    for rep in range(6):
        _one_step(*eager)
        g.replay()
        junk = torch.randn(1000, device=gpu).sum()      # unrelated eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert eager[1].tolist() == graphed[1].tolist()
        for oe, og in zip(eager[3], graphed[3]):
            assert torch.equal(oe, og), rep
        for ce, cg in zip(eager[0], graphed[0]):
            assert torch.equal(ce.k.view(torch.int16), cg.k.view(torch.int16))


def test_workspace_stays_usable_after_a_merge_gives_up(gpu):
    """The split merge's wait is bounded: a merger that gives up reports
    KVC_DEVERR_SYNC and that call's outputs are not valid. The test hook
    sets the bound to a single poll, so mergers that find a partner's flag not
    yet raised give up at once; their partners raise the flag afterwards, in
    the same launch. The next calls on the same workspace, with the default
    bound and other queries, must wait for their own partners (a late flag
    holds the previous epoch's value) and match the oracle with no status bit."""
    lens = [2048] * 16
    case = DecodeCase(batch=16, n_q=32, n_kv=8, head_dim=128, dtype="bf16", lengths=lens, tag="syncrec",
                      device=gpu, host_rows=[(0, 0), (7, 3), (15, 7)])
    kvc.append(case.k, case.v, case.seq_lens, case.k_new, case.v_new)
    ws = kvc.workspace(case.k, case.v, case.n_q, 2)
    out = torch.empty((case.batch, case.n_q, 128), device=gpu)
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    qs = [synth.normal((case.batch, case.n_q, 128), "bf16", 7, "syncrec", "q", i, device=gpu) for i in range(4)]
    prev = kvc.debug_set_merge_spin_limit(0)
    gave_up = 0
    try:
        for i in range(8):                    # until some merge gives up
            status.zero_()
            kvc.decode_attn(case.k, case.v, case.seq_lens, qs[i % 2], out, ws, n_pending=1, n_splits=2,
                            status=status)
            torch.cuda.synchronize()
            if int(status.item()) & kvc.DEVERR_SYNC:
                gave_up = i + 1
                break
    finally:
        kvc.debug_set_merge_spin_limit(prev)
    print(f"a merge gave up on call {gave_up}" if gave_up else "no merge gave up in 8 calls")
    grp = case.n_q // case.n_kv
    for q in qs[2:]:                           # queries no earlier call used
        status.zero_()
        kvc.decode_attn(case.k, case.v, case.seq_lens, q, out, ws, n_pending=1, n_splits=2, status=status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        got = out.double().cpu().numpy()
        qh = q.cpu()
        for (b, g) in case.host:
            k, v = case.oracle_inputs(b, g)
            ref = oracle.decode_attention(qh[b:b + 1, g * grp:(g + 1) * grp], k[None, None], v[None, None],
                                          np.array([lens[b]]), n_pending=1)[0]
            assert np.abs(got[b, g * grp:(g + 1) * grp] - ref).max() <= TOL["bf16"]
