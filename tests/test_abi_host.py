"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and its host-only logic (validation before any launch, the
cache-bytes formula, status strings, workspace sizing) behaves as documented."""

import csv
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvc.h")


def _lib():
    import kv_cache_append_amd as kvc
    if not os.path.exists(kvc.LIB_PATH):
        pytest.fail("libkvc.so is not built (run __graft_entry__.build())")
    return kvc, kvc.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z_]+)\s*\(", text)))


def test_header_declarations_match_binding_list():
    import kv_cache_append_amd as kvc
    assert _declared() == sorted(kvc.EXPORTS)


def test_library_exports_every_declared_symbol():
    kvc, lib = _lib()
    out = subprocess.run(["nm", "-D", "--defined-only", kvc.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(kvc_\w+)$", out, flags=re.M))
    for name in _declared():
        assert name in exported, name
        assert hasattr(lib, name)


def test_library_is_built_for_gfx950():
    """The offload bundle inside libkvc.so (built here from our sources) targets gfx950."""
    kvc, _ = _lib()
    blob = open(kvc.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def _rows():
    path = os.path.join(ROOT, "tests", "golden", "capacity_values.csv")
    with open(path) as f:
        return list(csv.DictReader([ln for ln in f if not ln.startswith("#")]))


def test_cache_bytes_matches_printed_values():
    """kvc_cache_bytes against every size the pages print (same golden file
    that pins the oracle)."""
    kvc, lib = _lib()
    units = {"B": 1, "KiB": 2**10, "MiB": 2**20, "GiB": 2**30}
    code = {2: kvc.KVC_F16, 4: kvc.KVC_F32}
    for row in _rows():
        b = int(row["batch"])
        lens = (ctypes.c_int32 * b)(*([int(row["seq_len"])] * b))
        got = lib.kvc_cache_bytes(int(row["n_layers"]), int(row["n_kv_heads"]), int(row["head_dim"]),
                                  code[int(row["elem_bytes"])], lens, b)
        want = float(row["value"]) * units[row["unit"]]
        tol = float(row["rel_tol"])
        assert abs(got - want) <= tol * want, row["citation"]


def test_cache_bytes_invalid_inputs_return_zero():
    _, lib = _lib()
    lens = (ctypes.c_int32 * 2)(5, -1)
    assert lib.kvc_cache_bytes(1, 1, 8, 0, lens, 2) == 0          # negative length
    assert lib.kvc_cache_bytes(1, 1, 8, 9, lens, 1) == 0          # unknown dtype
    assert lib.kvc_cache_bytes(1, 1, 8, 2, None, 1) == 0          # NULL lengths
    assert lib.kvc_cache_bytes(1, 1, 8, 2, None, 0) == 0          # empty batch


def test_status_strings():
    kvc, lib = _lib()
    for code, name in kvc.STATUS.items():
        assert lib.kvc_status_str(code).decode().startswith(name)


def _desc(kvc, **kw):
    base = dict(k=64, v=128, batch=2, n_kv_heads=2, max_len=16, head_dim=128, dtype=kvc.KVC_BF16,
                reserved0=0, stride_b=2 * 16 * 128, stride_h=16 * 128, stride_t=128)
    base.update(kw)
    return kvc.CacheDesc(**base)


FAKE = ctypes.c_void_p(4096)  # never dereferenced: every case below fails validation first


@pytest.mark.parametrize("kw,code", [
    (dict(k=None), 1), (dict(dtype=7), 3), (dict(n_kv_heads=0), 2), (dict(head_dim=0), 2),
    (dict(stride_t=64), 2), (dict(reserved0=1), 2), (dict(k=66), 4), (dict(stride_t=129), 4),
])
def test_decode_validation_rejects_before_launch(kw, code):
    kvc, lib = _lib()
    c = _desc(kvc, **kw)
    rc = lib.kvc_decode_attn(ctypes.byref(c), FAKE, 1, FAKE, 4, 0.1, FAKE, 0, FAKE, 1 << 30, 0, None, None)
    assert rc == code


def test_decode_validation_gqa_workspace_unsupported():
    kvc, lib = _lib()
    c = _desc(kvc)
    big = 1 << 30
    assert lib.kvc_decode_attn(ctypes.byref(c), FAKE, 1, FAKE, 3, 0.1, FAKE, 0, FAKE, big, 0, None, None) == 5
    assert lib.kvc_decode_attn(ctypes.byref(c), FAKE, 1, FAKE, 0, 0.1, FAKE, 0, FAKE, big, 0, None, None) == 5
    need = lib.kvc_decode_workspace_bytes(ctypes.byref(c), 4, 0)
    assert need > 0
    assert lib.kvc_decode_attn(ctypes.byref(c), FAKE, 1, FAKE, 4, 0.1, FAKE, 0, FAKE, need - 1, 0,
                               None, None) == 6
    assert lib.kvc_decode_attn(ctypes.byref(c), FAKE, 1, FAKE, 4, 0.1, FAKE, 0, None, need, 0, None, None) == 6
    odd = _desc(kvc, head_dim=96, stride_t=96, stride_h=16 * 96, stride_b=2 * 16 * 96)
    assert lib.kvc_decode_attn(ctypes.byref(odd), FAKE, 1, FAKE, 4, 0.1, FAKE, 0, FAKE, big, 0, None, None) == 7
    assert lib.kvc_decode_attn(ctypes.byref(c), FAKE, 1, FAKE, 4, 0.1, FAKE, kvc.KVC_F16, FAKE, big, 0,
                               None, None) == 3     # out dtype must be fp32 or the cache dtype
    assert lib.kvc_decode_attn(ctypes.byref(c), None, 1, FAKE, 4, 0.1, FAKE, 0, FAKE, big, 0, None, None) == 1
    for bad in (0.0, -0.1, float("inf"), float("nan"), 3e38):   # scale must be finite and > 0
        assert lib.kvc_decode_attn(ctypes.byref(c), FAKE, 1, FAKE, 4, bad, FAKE, 0, FAKE, big, 0,
                                   None, None) == 7


def test_workspace_size_formula():
    """Workspace = uint32 ready flags [B * H_kv * head blocks, S] + the
    wide-group merge words (64 uint32 per (sequence, KV head)) + fp32
    partial outputs [B, H_q, S, D] + (reference, sum) pairs, each region
    rounded up to 256 bytes."""
    kvc, lib = _lib()
    c = _desc(kvc)
    for s in (1, 3, 16, 100):
        rows = 2 * 4 * s
        flags = -(-2 * 2 * s * 4 // 256) * 256
        sync = -(-2 * 2 * 256 // 256) * 256
        want = flags + sync + -(-rows * 128 * 4 // 256) * 256 + -(-rows * 8 // 256) * 256
        assert lib.kvc_decode_workspace_bytes(ctypes.byref(c), 4, s) == want
    auto = lib.kvc_decode_splits(ctypes.byref(c), 4)
    assert auto >= 1
    assert lib.kvc_decode_workspace_bytes(ctypes.byref(c), 4, 0) == lib.kvc_decode_workspace_bytes(
        ctypes.byref(c), 4, auto)
    assert lib.kvc_decode_workspace_bytes(ctypes.byref(c), 3, 0) == 0


def test_auto_splits_cover_the_chip():
    """The library's split choice aims at about one workgroup per CU (256 CUs),
    with chunks of at least 256 tokens."""
    kvc, lib = _lib()

    def splits(batch, n_kv, n_q, max_len):
        c = _desc(kvc, batch=batch, n_kv_heads=n_kv, max_len=max_len, stride_t=128,
                  stride_h=max_len * 128, stride_b=n_kv * max_len * 128)
        return lib.kvc_decode_splits(ctypes.byref(c), n_q)

    assert splits(16, 8, 32, 2049) == 2          # 128 units of 4 heads
    assert splits(1, 32, 32, 4097) == 8          # 32 single-head units
    assert splits(32, 8, 64, 8193) == 1          # 256 units
    assert splits(24, 32, 32, 6001) == 1         # 768 units
    assert splits(1, 2, 4, 13) == 1              # short cache: one chunk
    assert splits(1, 1, 1, 1 << 20) == 256       # capped at KVC_MAX_SPLITS
    for args in [(16, 8, 32, 2049), (1, 32, 32, 4097), (2, 2, 4, 700)]:
        s = splits(*args)
        assert s == 1 or -(-args[3] // s) >= 256


@pytest.mark.parametrize("call", ["append", "fill"])
def test_copy_validation(call):
    kvc, lib = _lib()
    bad = _desc(kvc, n_kv_heads=-1)
    ok = _desc(kvc)
    if call == "append":
        assert lib.kvc_append(ctypes.byref(bad), FAKE, FAKE, FAKE, 256, 128, None, None) == 2
        assert lib.kvc_append(ctypes.byref(ok), None, FAKE, FAKE, 256, 128, None, None) == 1
        assert lib.kvc_append(ctypes.byref(ok), FAKE, FAKE, FAKE, 256, 64, None, None) == 2
        assert lib.kvc_append(None, FAKE, FAKE, FAKE, 256, 128, None, None) == 1
        empty = _desc(kvc, batch=0)
        assert lib.kvc_append(ctypes.byref(empty), None, None, None, 0, 0, None, None) == 0
    else:
        assert lib.kvc_prefill_fill(ctypes.byref(ok), FAKE, FAKE, FAKE, 0, 0, 0, -1, None, None) == 2
        assert lib.kvc_prefill_fill(ctypes.byref(ok), FAKE, FAKE, FAKE, 0, 0, 0, 0, None, None) == 0
        assert lib.kvc_prefill_fill(ctypes.byref(ok), FAKE, None, FAKE, 0, 0, 0, 3, None, None) == 1
        assert lib.kvc_prefill_fill(ctypes.byref(ok), FAKE, FAKE, FAKE, 0, 0, 64, 3, None, None) == 2


def test_advance_validation():
    _, lib = _lib()
    assert lib.kvc_seq_lens_advance(None, -1, 1, None) == 2
    assert lib.kvc_seq_lens_advance(None, 0, 1, None) == 0
    assert lib.kvc_seq_lens_advance(None, 4, 1, None) == 1


def test_decode_step_validation():
    kvc, lib = _lib()
    c = _desc(kvc)
    big = 1 << 30
    args = lambda kn, vn, sb, sh: (ctypes.byref(c), FAKE, kn, vn, sb, sh, FAKE, 4, 0.1, FAKE, 0, FAKE, big, 0,
                                   None, None)
    assert lib.kvc_decode_step(*args(None, FAKE, 256, 128)) == 1
    assert lib.kvc_decode_step(*args(FAKE, None, 256, 128)) == 1
    assert lib.kvc_decode_step(*args(ctypes.c_void_p(4104), FAKE, 256, 128)) == 4   # k_new not 16-byte aligned
    assert lib.kvc_decode_step(*args(FAKE, FAKE, 256, 132)) == 4                     # stride_h * 2 B not /16
    assert lib.kvc_decode_step(*args(FAKE, FAKE, 256, 64)) == 2                      # heads overlap


def test_split_count_limit():
    kvc, lib = _lib()
    c = _desc(kvc)
    assert lib.kvc_decode_workspace_bytes(ctypes.byref(c), 4, 256) > 0
    assert lib.kvc_decode_workspace_bytes(ctypes.byref(c), 4, 257) == 0
    assert lib.kvc_decode_attn(ctypes.byref(c), FAKE, 1, FAKE, 4, 0.1, FAKE, 0, FAKE, 1 << 30, 257, None, None) == 2


def test_block_validation_and_workspace():
    """kvc_block_attn: t_q < 1 is a shape error, grouping as for decode, and
    its workspace is the decode workspace of t_q * n_q virtual heads."""
    kvc, lib = _lib()
    c = _desc(kvc)
    big = 1 << 30
    assert lib.kvc_block_attn(ctypes.byref(c), FAKE, 0, FAKE, 4, 0.1, FAKE, 0, FAKE, big, 0, None, None) == 2
    assert lib.kvc_block_attn(ctypes.byref(c), FAKE, 3, FAKE, 3, 0.1, FAKE, 0, FAKE, big, 0, None, None) == 5
    assert lib.kvc_block_attn(None, FAKE, 3, FAKE, 4, 0.1, FAKE, 0, FAKE, big, 0, None, None) == 1
    assert lib.kvc_block_attn(ctypes.byref(c), FAKE, 3, FAKE, 4, -1.0, FAKE, 0, FAKE, big, 0, None, None) == 7
    for t_q in (1, 3, 8):
        for s in (0, 1, 5):
            assert lib.kvc_block_workspace_bytes(ctypes.byref(c), 4, t_q, s) == \
                lib.kvc_decode_workspace_bytes(ctypes.byref(c), 4 * t_q, s)
    assert lib.kvc_block_workspace_bytes(ctypes.byref(c), 4, 0, 0) == 0
    assert lib.kvc_block_workspace_bytes(ctypes.byref(c), 3, 2, 0) == 0
    need = lib.kvc_block_workspace_bytes(ctypes.byref(c), 4, 3, 0)
    assert lib.kvc_block_attn(ctypes.byref(c), FAKE, 3, FAKE, 4, 0.1, FAKE, 0, FAKE, need - 1, 0, None, None) == 6


def test_block_step_validation_rejects_before_launch():
    """kvc_block_step: the fill's and the attention's host checks, on both
    of its routes (one fused launch for 16-byte aligned rows on the
    wide-group kernel; otherwise fill, then attention, both checked before
    either is enqueued). Every case fails before a launch."""
    kvc, lib = _lib()
    c = _desc(kvc)
    big = 1 << 30
    odd = ctypes.c_void_p(4096 + 2)          # element-aligned, not 16-byte aligned: the two-launch route

    def f(cache=ctypes.byref(c), t_q=4, kn=FAKE, vn=FAKE, sb=1024, sh=512, st=128, nq=4, scale=0.1, ws=big):
        return lib.kvc_block_step(cache, FAKE, t_q, kn, vn, sb, sh, st, FAKE, nq, scale, FAKE, 0, FAKE, ws, 0,
                                  None, None)

    assert f(cache=None) == 1                                   # no cache
    assert f(t_q=0) == 2                                        # t_q < 1
    assert f(kn=None) == 1 and f(vn=None) == 1                  # no rows to append
    assert f(sb=-1) == 2                                        # negative stride
    assert f(st=64) == 2                                        # rows of a block overlap
    assert f(kn=ctypes.c_void_p(4097)) == 4                     # not element-aligned
    for kn in (FAKE, odd):                                      # both routes
        assert f(kn=kn, nq=3) == 5                              # 3 query heads over 2 KV heads
        assert f(kn=kn, scale=-1.0) == 7                        # scale must be positive
        need = lib.kvc_block_workspace_bytes(ctypes.byref(c), 4, 4, 0)
        assert f(kn=kn, ws=need - 1) == 6                       # workspace too small


def test_split_read_validation_and_workspace():
    """kvc_split_read (the decode launch's loads and split exchange, no
    arithmetic): host checks fail before a launch; the workspace holds the
    flags (256-byte aligned) and 2 KB per (unit, split)."""
    kvc, lib = _lib()
    c = _desc(kvc)
    ws = lib.kvc_split_read_workspace_bytes(ctypes.byref(c), 3)
    assert ws == 256 + 4 * 3 * 2048                            # 2 x 2 units, 3 splits
    assert lib.kvc_split_read_workspace_bytes(ctypes.byref(c), 0) == 0
    assert lib.kvc_split_read_workspace_bytes(ctypes.byref(c), 257) == 0
    big = 1 << 30
    f = lambda cc, splits=3, out=FAKE, wsp=FAKE, n=big: lib.kvc_split_read(cc, FAKE, splits, out, wsp, n, None)
    assert f(None) == 1 and f(ctypes.byref(c), out=None) == 1
    assert f(ctypes.byref(c), splits=0) == 2
    assert f(ctypes.byref(c), n=ws - 1) == 6
    assert f(ctypes.byref(c), wsp=ctypes.c_void_p(4096 + 16)) == 4     # workspace not 256-byte aligned
    small = _desc(kvc, head_dim=8, stride_b=2 * 16 * 8, stride_h=16 * 8, stride_t=8)   # 16-byte rows
    assert f(ctypes.byref(small)) == 7
    bad = _desc(kvc, dtype=9)
    assert f(ctypes.byref(bad)) == 3


def test_prefill_validation_rejects_before_launch():
    """kvc_prefill_attn: every case below fails on the host before a launch."""
    kvc, lib = _lib()
    c = _desc(kvc)
    f = lib.kvc_prefill_attn
    assert f(None, FAKE, 3, FAKE, 4, 0.1, FAKE, 0, None, None) == 1                       # no cache
    assert f(ctypes.byref(c), FAKE, 0, FAKE, 4, 0.1, FAKE, 0, None, None) == 2             # t_q < 1
    assert f(ctypes.byref(c), FAKE, 3, FAKE, 3, 0.1, FAKE, 0, None, None) == 5             # 3 % 2 heads
    assert f(ctypes.byref(c), FAKE, 3, FAKE, 4, 0.1, FAKE, kvc.KVC_F16, None, None) == 3   # out dtype
    assert f(ctypes.byref(c), FAKE, 3, FAKE, 4, -1.0, FAKE, 0, None, None) == 7            # scale
    assert f(ctypes.byref(c), FAKE, 3, FAKE, 4, float("inf"), FAKE, 0, None, None) == 7
    c32 = _desc(kvc, dtype=kvc.KVC_F32)                                                  # fp32 cache
    assert f(ctypes.byref(c32), FAKE, 3, FAKE, 4, 0.1, FAKE, 0, None, None) == 7
    c96 = _desc(kvc, head_dim=96, stride_b=2 * 16 * 96, stride_h=16 * 96, stride_t=96)    # head dim 96
    assert f(ctypes.byref(c96), FAKE, 3, FAKE, 4, 0.1, FAKE, 0, None, None) == 7
    assert f(ctypes.byref(c), None, 3, FAKE, 4, 0.1, FAKE, 0, None, None) == 1             # no seq_lens
    assert f(ctypes.byref(c), FAKE, 3, ctypes.c_void_p(4104), 4, 0.1, FAKE, 0, None, None) == 4   # q alignment
    assert f(ctypes.byref(c), FAKE, 3, FAKE, 4, 0.1, ctypes.c_void_p(4098), 0, None, None) == 4   # out alignment
    huge = _desc(kvc, max_len=1 << 23, stride_b=2 * (1 << 23) * 128, stride_h=(1 << 23) * 128)
    assert f(ctypes.byref(huge), FAKE, 3, FAKE, 4, 0.1, FAKE, 0, None, None) == 2          # 32-bit offsets
    empty = _desc(kvc, batch=0)
    assert f(ctypes.byref(empty), None, 3, None, 4, 0.1, None, 0, None, None) == 0         # nothing to do


def _pdesc(kvc, **kw):
    base = dict(k_pages=64, v_pages=128, block_table=256, batch=2, n_kv_heads=2, page_size=16, head_dim=128,
                dtype=kvc.KVC_BF16, n_pages=10, pages_per_seq=4, table_stride=4, stride_page=2 * 16 * 128,
                stride_h=16 * 128, stride_t=128)
    base.update(kw)
    return kvc.PagedCacheDesc(**base)


def test_paged_validation_and_workspace():
    """Paged calls: page size a power of two (>= 16 for decode), table present,
    non-overlapping page geometry; decode only on 16-bit caches with head_dim
    a multiple of 32; workspace equals the contiguous one of the same batch,
    heads and capacity."""
    kvc, lib = _lib()
    big = 1 << 30
    ok = _pdesc(kvc)

    def dec(d):
        return lib.kvc_paged_decode_attn(ctypes.byref(d), FAKE, 1, FAKE, 4, 0.1, FAKE, 0, FAKE, big, 0, None, None)

    assert dec(_pdesc(kvc, page_size=24)) == 2
    assert dec(_pdesc(kvc, page_size=8, stride_h=8 * 128, stride_page=2 * 8 * 128)) == 7
    assert dec(_pdesc(kvc, block_table=None)) == 1
    assert dec(_pdesc(kvc, table_stride=3)) == 2
    assert dec(_pdesc(kvc, stride_h=100 * 128 // 100)) == 2          # heads overlap rows of a page
    assert dec(_pdesc(kvc, dtype=kvc.KVC_F32, stride_page=2 * 16 * 128, stride_h=16 * 128)) == 7
    # fill/append take P = 8: validation passes and stops at the missing seq_lens (nothing launched)
    assert lib.kvc_paged_append(ctypes.byref(_pdesc(kvc, page_size=8, stride_h=8 * 128, stride_page=2048)),
                                None, FAKE, FAKE, 256, 128, None, None) == 1
    assert lib.kvc_paged_append(None, FAKE, FAKE, FAKE, 256, 128, None, None) == 1
    contig = _desc(kvc, batch=2, n_kv_heads=2, max_len=64, stride_t=128, stride_h=64 * 128, stride_b=2 * 64 * 128)
    for s in (0, 1, 3):
        assert lib.kvc_paged_decode_workspace_bytes(ctypes.byref(ok), 4, s) == \
            lib.kvc_decode_workspace_bytes(ctypes.byref(contig), 4, s)


def _qdesc(kvc, **kw):
    """A valid kvc_qcache_t over fake device addresses (never dereferenced):
    B=2, H_kv=2, T_max=64, D=128, fp8 codes, bf16 rows/queries."""
    f = dict(k=4096, v=8192, k_scale=12288, v_scale=16384, batch=2, n_kv_heads=2, max_len=64, head_dim=128,
             format=kvc.QFMT_FP8_E4M3, in_dtype=kvc.KVC_BF16, stride_b=2 * 64 * 128, stride_h=64 * 128,
             stride_t=128, scale_stride_b=2 * 64, scale_stride_h=64)
    f.update(kw)
    return kvc.QCacheDesc(**f)


def test_quant_validation_and_workspace():
    """Quantised calls: format and dtype codes, head dims 64/128/256, scale
    and code pointers present, 16-byte code strides, non-overlapping scale
    rows, fp16/bf16 queries for decode; the decode workspace equals the
    contiguous cache's of the same geometry. Every case fails before launch."""
    kvc, lib = _lib()
    big = 1 << 30

    def dec(d, n_q=4, scale=0.1, out_dtype=0, ws_bytes=big, splits=0):
        return lib.kvc_quant_decode_attn(ctypes.byref(d), FAKE, 1, FAKE, n_q, scale, FAKE, out_dtype, FAKE, ws_bytes,
                                         splits, None, None)

    assert dec(_qdesc(kvc, format=2)) == 3
    assert dec(_qdesc(kvc, in_dtype=7)) == 3
    assert dec(_qdesc(kvc, in_dtype=kvc.KVC_F32)) == 7                # fp32 queries: not for decode
    assert dec(_qdesc(kvc, head_dim=96, stride_t=96, stride_h=64 * 96, stride_b=2 * 64 * 96)) == 7
    assert dec(_qdesc(kvc, k_scale=None)) == 1
    assert dec(_qdesc(kvc, stride_t=136)) == 4                        # not a multiple of 16 bytes
    assert dec(_qdesc(kvc, k=4100)) == 4
    assert dec(_qdesc(kvc, scale_stride_h=32)) == 2                   # scale rows of two heads overlap
    assert dec(_qdesc(kvc, stride_t=64)) == 2                         # rows overlap
    assert dec(_qdesc(kvc), n_q=3) == 5
    assert dec(_qdesc(kvc), scale=-1.0) == 7
    assert dec(_qdesc(kvc), out_dtype=kvc.KVC_F16) == 3               # out must be fp32 or the query type
    assert dec(_qdesc(kvc), splits=257) == 2
    need = lib.kvc_quant_decode_workspace_bytes(ctypes.byref(_qdesc(kvc)), 4, 0)
    assert dec(_qdesc(kvc), ws_bytes=need - 1) == 6
    contig = _desc(kvc, batch=2, n_kv_heads=2, max_len=64, stride_t=128, stride_h=64 * 128, stride_b=2 * 64 * 128)
    for s in (0, 1, 3):
        assert lib.kvc_quant_decode_workspace_bytes(ctypes.byref(_qdesc(kvc)), 4, s) == \
            lib.kvc_decode_workspace_bytes(ctypes.byref(contig), 4, s)
    assert lib.kvc_quant_decode_workspace_bytes(ctypes.byref(_qdesc(kvc, in_dtype=kvc.KVC_F32)), 4, 0) == 0
    # append / fill: fp32 rows are accepted, so validation passes and stops at the missing seq_lens
    assert lib.kvc_quant_append(ctypes.byref(_qdesc(kvc, in_dtype=kvc.KVC_F32)), None, FAKE, FAKE, 256, 128,
                                None, None) == 1
    assert lib.kvc_quant_append(None, FAKE, FAKE, FAKE, 256, 128, None, None) == 1
    assert lib.kvc_quant_prefill_fill(ctypes.byref(_qdesc(kvc)), FAKE, FAKE, FAKE, 0, 0, 0, -1, None, None) == 2
    assert lib.kvc_quant_prefill_fill(ctypes.byref(_qdesc(kvc)), FAKE, FAKE, FAKE, 0, 0, 0, 0, None, None) == 0
    assert lib.kvc_quant_prefill_fill(ctypes.byref(_qdesc(kvc)), FAKE, FAKE, FAKE, 0, 0, 64, 3, None, None) == 2
    # the step validates the attention arguments before it enqueues the append
    step = lambda **kw: lib.kvc_quant_decode_step(ctypes.byref(_qdesc(kvc)), FAKE, FAKE, FAKE, 256, 128, FAKE,
                                                  kw.get("n_q", 4), 0.1, FAKE, 0, FAKE, kw.get("ws", big), 0,
                                                  None, None)
    assert step(n_q=3) == 5
    assert step(ws=need - 1) == 6


def test_splits_for_lengths_model_choices():
    """The length-aware split choice on the bench workloads' geometries: the
    counts measured fastest on MI355X (all equal to the length-blind rule,
    the ragged batch included: one split measured 5 % faster than six), and
    more splits than the length-blind rule when a few sequences are far
    longer than the rest."""
    import synth
    kvc, lib = _lib()

    def pick(b, h, t, d, dt, nq, lens):
        c = _desc(kvc, batch=b, n_kv_heads=h, max_len=t, head_dim=d, dtype=dt, stride_t=d, stride_h=t * d,
                  stride_b=h * t * d)
        arr = (ctypes.c_int32 * len(lens))(*[int(x) for x in lens])
        return lib.kvc_decode_splits_for_lengths(ctypes.byref(c), nq, arr), lib.kvc_decode_splits(ctypes.byref(c), nq)

    assert pick(16, 8, 2100, 128, kvc.KVC_BF16, 32, [2049] * 16) == (2, 2)
    assert pick(1, 32, 4130, 128, kvc.KVC_F16, 32, [4097]) == (8, 8)
    assert pick(32, 8, 8300, 128, kvc.KVC_BF16, 64, [8193] * 32) == (1, 1)
    # 64 query heads on one KV head run on the wide-group kernel, one
    # workgroup per (sequence, KV head) and split: 32 units need 8 splits
    assert pick(32, 1, 8300, 128, kvc.KVC_BF16, 64, [8193] * 32) == (8, 8)
    ragged = synth.CONFIGS["ragged_long"].lengths(7).numpy() + 1
    assert pick(24, 32, 6100, 128, kvc.KVC_F16, 32, ragged) == (1, 1)
    assert pick(24, 32, 4096, 128, kvc.KVC_F16, 32, [min(int(x), 4096) for x in ragged]) == (1, 1)   # ring, W=4096
    got, default = pick(8, 8, 61000, 128, kvc.KVC_BF16, 32, [60000] + [100] * 7)   # one long sequence
    assert default == 4 and got >= 16
    got, default = pick(32, 8, 61000, 128, kvc.KVC_BF16, 32, [60000] * 2 + [2000] * 30)
    assert default == 1 and got >= 8
    c = _desc(kvc)
    arr = (ctypes.c_int32 * 8)(*([100] * 8))
    assert lib.kvc_decode_splits_for_lengths(ctypes.byref(c), 3, arr) == 0       # not a GQA multiple
    assert lib.kvc_decode_splits_for_lengths(ctypes.byref(c), 4, None) == 0


def test_offset_bound_of_a_slice():
    """The kernels address a (sequence, KV head) slice with 32-bit offsets:
    (T_max + 2048) * stride_t * s must stay below 2^31. At the bound the call
    gets as far as the workspace check; one token past it is KVC_ERR_SHAPE.
    Neither launches (the workspace is absent)."""
    kvc, lib = _lib()
    top = (2**31 - 1) // 256 - 2048
    for t_max, want in ((top, 6), (top + 1, 2)):
        c = _desc(kvc, batch=1, n_kv_heads=1, max_len=t_max, stride_t=128, stride_h=t_max * 128, stride_b=t_max * 128)
        assert lib.kvc_decode_attn(ctypes.byref(c), FAKE, 1, FAKE, 4, 0.1, FAKE, 0, None, 0, 0, None, None) == want
