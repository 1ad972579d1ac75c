"""kvc_append / kvc_prefill_fill / kvc_seq_lens_advance: bit-exact against the
oracle's append model (course notes §3.1 update; glossary path B). Caches
start with a canary pattern; every slot the oracle does not write must keep
its canary bits."""

import numpy as np
import pytest
import torch

import kv_cache_append_amd as kvc
import oracle
import synth

pytestmark = pytest.mark.gpu

INT_VIEW = {"fp32": torch.int32, "fp16": torch.int16, "bf16": torch.int16}


def _canary(shape, dtype, device, layout="bhtd"):
    """Distinct bit patterns per element (a recognisable, non-NaN canary)."""
    n = int(np.prod(shape))
    idt = INT_VIEW[dtype]
    bits = (torch.arange(n, dtype=torch.int64, device=device) * 2654435761 % 15000 + 1000).to(idt)
    t = bits.view(synth.DTYPES[dtype]).reshape(shape)
    if layout == "bthd":
        b, h, tt, d = shape
        t = t.reshape(b, tt, h, d).transpose(1, 2)   # same values, [B,T,H,D] storage
    return t


def _bits(t, dtype):
    return t.contiguous().view(INT_VIEW[dtype]).cpu().numpy()


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("head_dim", [4, 64, 128, 3])
@pytest.mark.parametrize("layout", ["bhtd", "bthd"])
def test_append_bitwise(gpu, dtype, head_dim, layout):
    dev = torch.device("cuda")
    b, h, t_max = 5, 3, 9
    lens = np.array([0, 4, 8, 9, 12], dtype=np.int32)      # the last two overflow
    kc = _canary((b, h, t_max, head_dim), dtype, dev, layout)
    vc = _canary((b, h, t_max, head_dim), dtype, dev, layout)
    kn = synth.normal((b, h, head_dim), dtype, 1, "kn", head_dim, device=dev)
    vn = synth.normal((b, h, head_dim), dtype, 1, "vn", head_dim, device=dev)
    ref_k, ref_v, ovf = oracle.append(_bits(kc, dtype), _bits(vc, dtype), lens, _bits(kn, dtype), _bits(vn, dtype))
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    kvc.append(kc, vc, torch.from_numpy(lens).to(dev), kn, vn, status=status)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(kc, dtype), ref_k)
    assert np.array_equal(_bits(vc, dtype), ref_v)
    assert int(status.item()) == (kvc.DEVERR_CAPACITY if ovf.any() else 0)


def test_append_from_strided_source(gpu):
    """k_new / v_new as a view of a fused [B, 2, H, D] projection output."""
    dev = torch.device("cuda")
    b, h, t_max, d = 4, 8, 6, 128
    kc = torch.zeros((b, h, t_max, d), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    kv = synth.normal((b, 2, h, d), "bf16", 2, "kv", device=dev)
    lens = torch.tensor([0, 1, 2, 5], dtype=torch.int32, device=dev)
    kvc.append(kc, vc, lens, kv[:, 0], kv[:, 1])
    torch.cuda.synchronize()
    for i, p in enumerate(lens.tolist()):
        assert torch.equal(kc[i, :, p].view(torch.int16), kv[i, 0].view(torch.int16))
        assert torch.equal(vc[i, :, p].view(torch.int16), kv[i, 1].view(torch.int16))
        others = [s for s in range(t_max) if s != p]
        assert torch.all(kc[i, :, others].view(torch.int16) == 0)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_prefill_fill_bitwise_and_chunked(gpu, dtype):
    """One fill of 7 tokens equals fills of 3 then 4 (chunked prefill); a fill
    that would pass T_max is refused and flagged."""
    dev = torch.device("cuda")
    b, h, t_max, d = 3, 2, 12, 128
    src = synth.normal((b, h, 7, d), dtype, 3, "src", device=dev)
    src_v = synth.normal((b, h, 7, d), dtype, 3, "srcv", device=dev)
    lens0 = np.array([0, 2, 6], dtype=np.int32)          # 6 + 7 > 12: overflow
    kc = _canary((b, h, t_max, d), dtype, dev).clone()
    vc = _canary((b, h, t_max, d), dtype, dev).clone()
    ref_k, ref_v, ovf = oracle.prefill_fill(_bits(kc, dtype), _bits(vc, dtype), lens0, _bits(src, dtype),
                                            _bits(src_v, dtype))
    assert list(ovf) == [False, False, True]
    k1, v1 = kc.clone(), vc.clone()
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    kvc.prefill_fill(k1, v1, torch.from_numpy(lens0).to(dev), src, src_v, status=status)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(k1, dtype), ref_k) and np.array_equal(_bits(v1, dtype), ref_v)
    assert int(status.item()) == kvc.DEVERR_CAPACITY
    # chunked: 3 tokens, advance, 4 tokens (non-contiguous source slices)
    k2, v2 = kc.clone(), vc.clone()
    lens = torch.tensor([0, 2, 2], dtype=torch.int32, device=dev)
    kvc.prefill_fill(k2, v2, lens, src[:, :, :3], src_v[:, :, :3])
    kvc.seq_lens_advance(lens, 3)
    kvc.prefill_fill(k2, v2, lens, src[:, :, 3:], src_v[:, :, 3:])
    torch.cuda.synchronize()
    assert lens.tolist() == [3, 5, 5]
    r_k, r_v, _ = oracle.prefill_fill(_bits(kc, dtype), _bits(vc, dtype), np.array([0, 2, 2]), _bits(src, dtype),
                                      _bits(src_v, dtype))
    assert np.array_equal(_bits(k2, dtype), r_k) and np.array_equal(_bits(v2, dtype), r_v)


def test_past_rows_stay_bit_identical_as_sequence_grows(gpu):
    """Course notes §1.2: once written, k_j and v_j never change; 20 appends
    leave every earlier row's bits as written."""
    dev = torch.device("cuda")
    b, h, t_max, d = 2, 4, 24, 128
    kc = torch.zeros((b, h, t_max, d), dtype=torch.float16, device=dev)
    vc = torch.zeros_like(kc)
    lens = torch.zeros(b, dtype=torch.int32, device=dev)
    rows = []
    for step in range(20):
        kn = synth.normal((b, h, d), "fp16", 4, "grow", step, device=dev)
        vn = synth.normal((b, h, d), "fp16", 4, "growv", step, device=dev)
        kvc.append(kc, vc, lens, kn, vn)
        kvc.seq_lens_advance(lens, 1)
        rows.append((kn, vn))
        torch.cuda.synchronize()
        for j, (kj, vj) in enumerate(rows):
            assert torch.equal(kc[:, :, j].view(torch.int16), kj.view(torch.int16))
            assert torch.equal(vc[:, :, j].view(torch.int16), vj.view(torch.int16))
    assert lens.tolist() == [20, 20]


def test_zero_batch_and_zero_tokens_are_no_ops(gpu):
    dev = torch.device("cuda")
    kc = torch.zeros((0, 2, 4, 8), device=dev)
    kvc.append(kc, kc.clone(), torch.zeros(0, dtype=torch.int32, device=dev),
               torch.zeros((0, 2, 8), device=dev), torch.zeros((0, 2, 8), device=dev))
    k1 = torch.zeros((1, 2, 4, 8), device=dev)
    kvc.prefill_fill(k1, k1.clone(), torch.zeros(1, dtype=torch.int32, device=dev),
                     torch.ones((1, 2, 0, 8), device=dev), torch.ones((1, 2, 0, 8), device=dev))
    torch.cuda.synchronize()
    assert torch.all(k1 == 0)
