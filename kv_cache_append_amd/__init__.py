"""Python binding of libkvc (KV-cache append + single-query decode attention on
MI355X / gfx950).

Argument marshalling only: every step runs in the HIP kernels of libkvc.so,
reached through its C ABI (include/kvc.h) with ctypes. PyTorch supplies device
memory and the current HIP stream. There is no fallback: if the library is not
built, every call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; KVC_LIBRARY may name another build of the same sources.
LIB_PATH = os.environ.get("KVC_LIBRARY") or os.path.join(_PKG, "libkvc.so")

KVC_F32, KVC_F16, KVC_BF16 = 0, 1, 2
DTYPE_CODE = {torch.float32: KVC_F32, torch.float16: KVC_F16, torch.bfloat16: KVC_BF16}
DEVERR_CAPACITY = 1
DEVERR_BADLEN = 2
DEVERR_SYNC = 4
DEVERR_PAGE = 8
QFMT_FP8_E4M3, QFMT_INT8 = 0, 1
QFMT = {"fp8": QFMT_FP8_E4M3, "int8": QFMT_INT8}

STATUS = {
    0: "KVC_OK", 1: "KVC_ERR_NULL", 2: "KVC_ERR_SHAPE", 3: "KVC_ERR_DTYPE", 4: "KVC_ERR_ALIGN",
    5: "KVC_ERR_GQA", 6: "KVC_ERR_WORKSPACE", 7: "KVC_ERR_UNSUPPORTED", 8: "KVC_ERR_HIP",
}

# Every symbol include/kvc.h declares.
EXPORTS = ("kvc_append", "kvc_prefill_fill", "kvc_decode_workspace_bytes", "kvc_decode_splits",
           "kvc_decode_attn", "kvc_decode_step", "kvc_decode_step_advance", "kvc_decode_step_noalloc",
           "kvc_decode_splits_for_lengths", "kvc_block_attn", "kvc_block_workspace_bytes", "kvc_block_step",
           "kvc_prefill_attn",
           "kvc_paged_append", "kvc_paged_prefill_fill", "kvc_paged_decode_workspace_bytes",
           "kvc_paged_decode_attn", "kvc_paged_decode_step",
           "kvc_ring_append", "kvc_ring_prefill_fill", "kvc_ring_decode_attn", "kvc_ring_decode_step",
           "kvc_quant_append", "kvc_quant_prefill_fill", "kvc_quant_decode_workspace_bytes",
           "kvc_quant_decode_attn", "kvc_quant_decode_step",
           "kvc_seq_lens_advance", "kvc_cache_bytes", "kvc_status_str", "kvc_stream_read_sink_bytes",
           "kvc_stream_read", "kvc_split_read_workspace_bytes", "kvc_split_read", "kvc_debug_set_merge_spin_limit")


class KvcError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS.get(code, code)}")


class CacheDesc(ctypes.Structure):
    """Mirror of kvc_cache_t."""
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("max_len", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("reserved0", ctypes.c_int32),
        ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64), ("stride_t", ctypes.c_int64),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load libkvc.so (built in-tree by __graft_entry__.build()); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, sz, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float
    cp = ctypes.POINTER(CacheDesc)
    lib.kvc_append.argtypes = [cp, vp, vp, vp, i64, i64, vp, vp]
    lib.kvc_append.restype = i32
    lib.kvc_prefill_fill.argtypes = [cp, vp, vp, vp, i64, i64, i64, i32, vp, vp]
    lib.kvc_prefill_fill.restype = i32
    lib.kvc_decode_workspace_bytes.argtypes = [cp, i32, i32]
    lib.kvc_decode_workspace_bytes.restype = sz
    lib.kvc_decode_splits.argtypes = [cp, i32]
    lib.kvc_decode_splits.restype = i32
    lib.kvc_decode_splits_for_lengths.argtypes = [cp, i32, ctypes.POINTER(i32)]
    lib.kvc_decode_splits_for_lengths.restype = i32
    lib.kvc_decode_attn.argtypes = [cp, vp, i32, vp, i32, f32, vp, i32, vp, sz, i32, vp, vp]
    lib.kvc_decode_attn.restype = i32
    lib.kvc_decode_step.argtypes = [cp, vp, vp, vp, i64, i64, vp, i32, f32, vp, i32, vp, sz, i32, vp, vp]
    lib.kvc_decode_step.restype = i32
    lib.kvc_block_attn.argtypes = [cp, vp, i32, vp, i32, f32, vp, i32, vp, sz, i32, vp, vp]
    lib.kvc_block_attn.restype = i32
    lib.kvc_block_step.argtypes = [cp, vp, i32, vp, vp, i64, i64, i64, vp, i32, f32, vp, i32, vp, sz, i32, vp, vp]
    lib.kvc_block_step.restype = i32
    lib.kvc_block_workspace_bytes.argtypes = [cp, i32, i32, i32]
    lib.kvc_block_workspace_bytes.restype = sz
    lib.kvc_prefill_attn.argtypes = [cp, vp, i32, vp, i32, f32, vp, i32, vp, vp]
    lib.kvc_prefill_attn.restype = i32
    pp = ctypes.POINTER(PagedCacheDesc)
    lib.kvc_paged_append.argtypes = [pp, vp, vp, vp, i64, i64, vp, vp]
    lib.kvc_paged_append.restype = i32
    lib.kvc_paged_prefill_fill.argtypes = [pp, vp, vp, vp, i64, i64, i64, i32, vp, vp]
    lib.kvc_paged_prefill_fill.restype = i32
    lib.kvc_paged_decode_workspace_bytes.argtypes = [pp, i32, i32]
    lib.kvc_paged_decode_workspace_bytes.restype = sz
    lib.kvc_paged_decode_attn.argtypes = [pp, vp, i32, vp, i32, f32, vp, i32, vp, sz, i32, vp, vp]
    lib.kvc_paged_decode_attn.restype = i32
    lib.kvc_paged_decode_step.argtypes = [pp, vp, vp, vp, i64, i64, vp, i32, f32, vp, i32, vp, sz, i32, vp, vp]
    lib.kvc_paged_decode_step.restype = i32
    lib.kvc_ring_append.argtypes = [cp, vp, vp, vp, i64, i64, vp, vp]
    lib.kvc_ring_append.restype = i32
    lib.kvc_ring_prefill_fill.argtypes = [cp, vp, vp, vp, i64, i64, i64, i32, vp, vp]
    lib.kvc_ring_prefill_fill.restype = i32
    lib.kvc_ring_decode_attn.argtypes = [cp, vp, i32, vp, i32, f32, vp, i32, vp, sz, i32, vp, vp]
    lib.kvc_ring_decode_attn.restype = i32
    lib.kvc_ring_decode_step.argtypes = [cp, vp, vp, vp, i64, i64, vp, i32, f32, vp, i32, vp, sz, i32, vp, vp]
    lib.kvc_ring_decode_step.restype = i32
    qp = ctypes.POINTER(QCacheDesc)
    lib.kvc_quant_append.argtypes = [qp, vp, vp, vp, i64, i64, vp, vp]
    lib.kvc_quant_append.restype = i32
    lib.kvc_quant_prefill_fill.argtypes = [qp, vp, vp, vp, i64, i64, i64, i32, vp, vp]
    lib.kvc_quant_prefill_fill.restype = i32
    lib.kvc_quant_decode_workspace_bytes.argtypes = [qp, i32, i32]
    lib.kvc_quant_decode_workspace_bytes.restype = sz
    lib.kvc_quant_decode_attn.argtypes = [qp, vp, i32, vp, i32, f32, vp, i32, vp, sz, i32, vp, vp]
    lib.kvc_quant_decode_attn.restype = i32
    lib.kvc_quant_decode_step.argtypes = [qp, vp, vp, vp, i64, i64, vp, i32, f32, vp, i32, vp, sz, i32, vp, vp]
    lib.kvc_quant_decode_step.restype = i32
    lib.kvc_stream_read_sink_bytes.argtypes = [i32]
    lib.kvc_stream_read_sink_bytes.restype = sz
    lib.kvc_stream_read.argtypes = [vp, sz, vp, i32, vp]
    lib.kvc_stream_read.restype = i32
    lib.kvc_split_read_workspace_bytes.argtypes = [cp, i32]
    lib.kvc_split_read_workspace_bytes.restype = sz
    lib.kvc_split_read.argtypes = [cp, vp, i32, vp, vp, sz, vp]
    lib.kvc_split_read.restype = i32
    lib.kvc_seq_lens_advance.argtypes = [vp, i32, i32, vp]
    lib.kvc_seq_lens_advance.restype = i32
    lib.kvc_cache_bytes.argtypes = [i32, i32, i32, i32, ctypes.POINTER(i32), i32]
    lib.kvc_cache_bytes.restype = ctypes.c_uint64
    lib.kvc_status_str.argtypes = [i32]
    lib.kvc_status_str.restype = ctypes.c_char_p
    lib.kvc_debug_set_merge_spin_limit.argtypes = [i32]
    lib.kvc_debug_set_merge_spin_limit.restype = i32
    lib.kvc_decode_step_advance.argtypes = [cp, vp, vp, vp, vp, i64, i64, vp, i32, f32, vp, i32, vp, sz, i32, vp, vp]
    lib.kvc_decode_step_advance.restype = i32
    lib.kvc_decode_step_noalloc.argtypes = [cp, vp, vp, vp, i64, i64, vp, i32, f32, vp, i32, i32, vp, vp]
    lib.kvc_decode_step_noalloc.restype = i32
    _lib = lib
    return lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(code: int, where: str):
    if code != 0:
        raise KvcError(code, where)


class PagedCacheDesc(ctypes.Structure):
    """Mirror of kvc_paged_cache_t."""
    _fields_ = [
        ("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
        ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("n_pages", ctypes.c_int32),
        ("pages_per_seq", ctypes.c_int32), ("table_stride", ctypes.c_int32),
        ("stride_page", ctypes.c_int64), ("stride_h", ctypes.c_int64), ("stride_t", ctypes.c_int64),
    ]


def paged_desc(k_pages: torch.Tensor, v_pages: torch.Tensor, block_table: torch.Tensor) -> PagedCacheDesc:
    """kvc_paged_cache_t for page pools [n_pages, H_kv, P, D] (any strides with
    D contiguous) and an int32 device page table [B, pages_per_seq]."""
    if k_pages.shape != v_pages.shape or k_pages.stride() != v_pages.stride() or k_pages.dim() != 4:
        raise ValueError("page pools must be 4-D [n_pages, H_kv, P, D] with equal shape and strides")
    if k_pages.shape[3] > 1 and k_pages.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be int32 [B, pages_per_seq] with contiguous rows")
    n_pages, h, psz, d = k_pages.shape
    sp, sh, st, _ = k_pages.stride()
    b, per_seq = block_table.shape
    return PagedCacheDesc(k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(), b, h, psz, d,
                          DTYPE_CODE[k_pages.dtype], n_pages, per_seq, block_table.stride(0), sp, sh, st)


class QCacheDesc(ctypes.Structure):
    """Mirror of kvc_qcache_t."""
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("max_len", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("format", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
        ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64), ("stride_t", ctypes.c_int64),
        ("scale_stride_b", ctypes.c_int64), ("scale_stride_h", ctypes.c_int64),
    ]


def qcache_desc(k_codes: torch.Tensor, v_codes: torch.Tensor, k_scale: torch.Tensor, v_scale: torch.Tensor,
                fmt: int, in_dtype: torch.dtype) -> QCacheDesc:
    """kvc_qcache_t for uint8 code tensors [B, H_kv, T_max, D] and float32 scale
    tensors [B, H_kv, T_max] (token axis contiguous); fmt is QFMT_FP8_E4M3 or
    QFMT_INT8, in_dtype the dtype of the appended rows and of the queries."""
    if k_codes.shape != v_codes.shape or k_codes.stride() != v_codes.stride() or k_codes.dim() != 4:
        raise ValueError("K and V codes must be 4-D with equal shape and strides")
    if k_codes.dtype != torch.uint8 or v_codes.dtype != torch.uint8:
        raise ValueError("codes must be uint8")
    if k_codes.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    b, h, t, d = k_codes.shape
    if k_scale.shape != (b, h, t) or v_scale.shape != (b, h, t) or k_scale.stride() != v_scale.stride():
        raise ValueError("scales must be [B, H_kv, T_max] with equal strides")
    if k_scale.dtype != torch.float32 or v_scale.dtype != torch.float32 or (t > 1 and k_scale.stride(2) != 1):
        raise ValueError("scales must be float32 with a contiguous token axis")
    sb, sh, st, _ = k_codes.stride()
    return QCacheDesc(k_codes.data_ptr(), v_codes.data_ptr(), k_scale.data_ptr(), v_scale.data_ptr(), b, h, t, d,
                      int(fmt), DTYPE_CODE[in_dtype], sb, sh, st, k_scale.stride(0), k_scale.stride(1))


def cache_desc(k: torch.Tensor, v: torch.Tensor) -> CacheDesc:
    """kvc_cache_t for one layer's K and V tensors [B, H_kv, T_max, D] (any
    strides with D contiguous; K and V must share shape, strides and dtype)."""
    if k.shape != v.shape or k.stride() != v.stride() or k.dtype != v.dtype or k.dim() != 4:
        raise ValueError("K and V must be 4-D with equal shape, strides and dtype")
    if k.dtype not in DTYPE_CODE:
        raise ValueError(f"unsupported cache dtype {k.dtype}")
    if k.shape[3] > 1 and k.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    b, h, t, d = k.shape
    sb, sh, st, _ = k.stride()
    return CacheDesc(k.data_ptr(), v.data_ptr(), b, h, t, d, DTYPE_CODE[k.dtype], 0, sb, sh, st)


def append(k_cache, v_cache, seq_lens, k_new, v_new, status=None, stream=None, desc=None):
    """kvc_append: write k_new/v_new [B, H_kv, D] at slot seq_lens[b]."""
    lib = load()
    c = desc if desc is not None else cache_desc(k_cache, v_cache)
    if k_new.stride() != v_new.stride() or k_new.dim() != 3:
        raise ValueError("k_new and v_new must be [B, H_kv, D] with equal strides")
    _check(lib.kvc_append(ctypes.byref(c), _ptr(seq_lens), _ptr(k_new), _ptr(v_new),
                          k_new.stride(0), k_new.stride(1), _ptr(status), _stream(stream)), "kvc_append")


def prefill_fill(k_cache, v_cache, seq_lens, k, v, status=None, stream=None):
    """kvc_prefill_fill: write k/v [B, H_kv, T_new, D] at slots [seq_lens[b], +T_new)."""
    lib = load()
    c = cache_desc(k_cache, v_cache)
    if k.stride() != v.stride() or k.dim() != 4:
        raise ValueError("k and v must be [B, H_kv, T_new, D] with equal strides")
    _check(lib.kvc_prefill_fill(ctypes.byref(c), _ptr(seq_lens), _ptr(k), _ptr(v),
                                k.stride(0), k.stride(1), k.stride(2), k.shape[2],
                                _ptr(status), _stream(stream)), "kvc_prefill_fill")


def decode_workspace_bytes(k_cache, v_cache, n_q_heads: int, n_splits: int = 0) -> int:
    c = cache_desc(k_cache, v_cache)
    return int(load().kvc_decode_workspace_bytes(ctypes.byref(c), n_q_heads, n_splits))


def workspace(k_cache, v_cache, n_q_heads: int, n_splits: int = 0) -> torch.Tensor:
    """A zero-filled device workspace for the decode calls (zero once; the
    calls leave it reusable)."""
    n = decode_workspace_bytes(k_cache, v_cache, n_q_heads, n_splits)
    if n == 0:
        raise ValueError("invalid cache/head arguments for a decode workspace")
    return torch.zeros(n, dtype=torch.uint8, device=k_cache.device)


def block_workspace(k_cache, v_cache, n_q_heads: int, t_q: int, n_splits: int = 0) -> torch.Tensor:
    """A zero-filled device workspace for kvc_block_attn with this geometry."""
    c = cache_desc(k_cache, v_cache)
    n = int(load().kvc_block_workspace_bytes(ctypes.byref(c), n_q_heads, t_q, n_splits))
    if n == 0:
        raise ValueError("invalid cache/head/block arguments for a block workspace")
    return torch.zeros(n, dtype=torch.uint8, device=k_cache.device)


def decode_splits(k_cache, v_cache, n_q_heads: int, lengths=None, desc=None) -> int:
    """kvc_decode_splits, or kvc_decode_splits_for_lengths when the attended
    lengths (one per sequence, host values) are given."""
    c = desc if desc is not None else cache_desc(k_cache, v_cache)
    if lengths is None:
        return int(load().kvc_decode_splits(ctypes.byref(c), n_q_heads))
    lens = [int(x) for x in lengths]
    if len(lens) != c.batch:
        raise ValueError("one length per sequence")
    arr = (ctypes.c_int32 * max(1, len(lens)))(*lens)
    return int(load().kvc_decode_splits_for_lengths(ctypes.byref(c), n_q_heads, arr))


def decode_attn(k_cache, v_cache, seq_lens, q, out, workspace, n_pending: int = 1, scale=None,
                n_splits: int = 0, status=None, stream=None, desc=None):
    """kvc_decode_attn: out[b,h] = softmax(scale q.K^T) V over seq_lens[b]+n_pending tokens."""
    lib = load()
    c = desc if desc is not None else cache_desc(k_cache, v_cache)
    if scale is None:
        scale = 1.0 / float(q.shape[-1]) ** 0.5
    if not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous [B, H_q, D]")
    out_code = DTYPE_CODE[out.dtype]
    _check(lib.kvc_decode_attn(ctypes.byref(c), _ptr(seq_lens), n_pending, _ptr(q), q.shape[1],
                               float(scale), _ptr(out), out_code, _ptr(workspace),
                               workspace.numel() * workspace.element_size(), n_splits,
                               _ptr(status), _stream(stream)), "kvc_decode_attn")


def decode_step(k_cache, v_cache, seq_lens, k_new, v_new, q, out, workspace, scale=None, n_splits: int = 0,
                status=None, stream=None, desc=None, seq_lens_next=None):
    """kvc_decode_step: append k_new/v_new at slot seq_lens[b] and attend
    seq_lens[b] + 1 tokens, in one launch. With seq_lens_next (another int32
    [B] device array), kvc_decode_step_advance: the same launch also writes
    seq_lens_next[b] = seq_lens[b] + 1 (the last layer of a step)."""
    lib = load()
    c = desc if desc is not None else cache_desc(k_cache, v_cache)
    if scale is None:
        scale = 1.0 / float(q.shape[-1]) ** 0.5
    if not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous [B, H_q, D]")
    if k_new.stride() != v_new.stride() or k_new.dim() != 3:
        raise ValueError("k_new and v_new must be [B, H_kv, D] with equal strides")
    if seq_lens_next is not None:
        _check(lib.kvc_decode_step_advance(ctypes.byref(c), _ptr(seq_lens), _ptr(seq_lens_next), _ptr(k_new),
                                           _ptr(v_new), k_new.stride(0), k_new.stride(1), _ptr(q), q.shape[1],
                                           float(scale), _ptr(out), DTYPE_CODE[out.dtype], _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), n_splits, _ptr(status),
                                           _stream(stream)), "kvc_decode_step_advance")
        return
    _check(lib.kvc_decode_step(ctypes.byref(c), _ptr(seq_lens), _ptr(k_new), _ptr(v_new), k_new.stride(0),
                               k_new.stride(1), _ptr(q), q.shape[1], float(scale), _ptr(out),
                               DTYPE_CODE[out.dtype], _ptr(workspace), workspace.numel() * workspace.element_size(),
                               n_splits, _ptr(status), _stream(stream)), "kvc_decode_step")


def decode_step_noalloc(k_cache, v_cache, seq_lens, k_new, v_new, q, out, scale=None, n_splits: int = 0,
                        status=None, stream=None, desc=None):
    """kvc_decode_step_noalloc: kvc_decode_step with the split exchange in the
    library's own device array instead of a workspace (nothing allocated)."""
    lib = load()
    c = desc if desc is not None else cache_desc(k_cache, v_cache)
    if scale is None:
        scale = 1.0 / float(q.shape[-1]) ** 0.5
    if not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous [B, H_q, D]")
    if k_new.stride() != v_new.stride() or k_new.dim() != 3:
        raise ValueError("k_new and v_new must be [B, H_kv, D] with equal strides")
    _check(lib.kvc_decode_step_noalloc(ctypes.byref(c), _ptr(seq_lens), _ptr(k_new), _ptr(v_new), k_new.stride(0),
                                       k_new.stride(1), _ptr(q), q.shape[1], float(scale), _ptr(out),
                                       DTYPE_CODE[out.dtype], n_splits, _ptr(status), _stream(stream)),
           "kvc_decode_step_noalloc")


def block_attn(k_cache, v_cache, seq_lens, q, out, workspace, scale=None, n_splits: int = 0, status=None,
               stream=None, desc=None):
    """kvc_block_attn: q [B, t_q, H_q, D]; query i of sequence b attends
    slots 0..seq_lens[b]+i (lower-right causal mask); out like q."""
    lib = load()
    c = desc if desc is not None else cache_desc(k_cache, v_cache)
    if scale is None:
        scale = 1.0 / float(q.shape[-1]) ** 0.5
    if not (q.is_contiguous() and out.is_contiguous()) or q.dim() != 4:
        raise ValueError("q and out must be contiguous [B, t_q, H_q, D]")
    _check(lib.kvc_block_attn(ctypes.byref(c), _ptr(seq_lens), q.shape[1], _ptr(q), q.shape[2], float(scale),
                              _ptr(out), DTYPE_CODE[out.dtype], _ptr(workspace),
                              workspace.numel() * workspace.element_size(), n_splits, _ptr(status),
                              _stream(stream)), "kvc_block_attn")


def block_step(k_cache, v_cache, seq_lens, k_new, v_new, q, out, workspace, scale=None, n_splits: int = 0,
               status=None, stream=None, desc=None):
    """kvc_block_step: write k_new/v_new [B, H_kv, t_q, D] at slots
    [seq_lens[b], +t_q), then block_attn over them (one launch where the
    wide-group kernel serves the block)."""
    lib = load()
    c = desc if desc is not None else cache_desc(k_cache, v_cache)
    if scale is None:
        scale = 1.0 / float(q.shape[-1]) ** 0.5
    if not (q.is_contiguous() and out.is_contiguous()) or q.dim() != 4:
        raise ValueError("q and out must be contiguous [B, t_q, H_q, D]")
    if k_new.dim() != 4 or k_new.stride() != v_new.stride() or k_new.stride(3) != 1:
        raise ValueError("k_new and v_new must be [B, H_kv, t_q, D] with equal strides and D contiguous")
    _check(lib.kvc_block_step(ctypes.byref(c), _ptr(seq_lens), q.shape[1], _ptr(k_new), _ptr(v_new),
                              k_new.stride(0), k_new.stride(1), k_new.stride(2), _ptr(q), q.shape[2], float(scale),
                              _ptr(out), DTYPE_CODE[out.dtype], _ptr(workspace),
                              workspace.numel() * workspace.element_size(), n_splits, _ptr(status),
                              _stream(stream)), "kvc_block_step")


def prefill_attn(k_cache, v_cache, seq_lens, q, out, scale=None, status=None, stream=None, desc=None):
    """kvc_prefill_attn: as block_attn (query i of sequence b attends slots
    0..seq_lens[b]+i), tiled on the matrix cores for long blocks; no workspace."""
    lib = load()
    c = desc if desc is not None else cache_desc(k_cache, v_cache)
    if scale is None:
        scale = 1.0 / float(q.shape[-1]) ** 0.5
    if not (q.is_contiguous() and out.is_contiguous()) or q.dim() != 4:
        raise ValueError("q and out must be contiguous [B, t_q, H_q, D]")
    _check(lib.kvc_prefill_attn(ctypes.byref(c), _ptr(seq_lens), q.shape[1], _ptr(q), q.shape[2], float(scale),
                                _ptr(out), DTYPE_CODE[out.dtype], _ptr(status), _stream(stream)), "kvc_prefill_attn")


def paged_prefill_fill(k_pages, v_pages, block_table, seq_lens, k, v, status=None, stream=None):
    """kvc_paged_prefill_fill: k/v [B, H_kv, T_new, D] to logical slots [seq_lens[b], +T_new)."""
    c = paged_desc(k_pages, v_pages, block_table)
    if k.stride() != v.stride() or k.dim() != 4:
        raise ValueError("k and v must be [B, H_kv, T_new, D] with equal strides")
    _check(load().kvc_paged_prefill_fill(ctypes.byref(c), _ptr(seq_lens), _ptr(k), _ptr(v), k.stride(0),
                                         k.stride(1), k.stride(2), k.shape[2], _ptr(status), _stream(stream)),
           "kvc_paged_prefill_fill")


def paged_append(k_pages, v_pages, block_table, seq_lens, k_new, v_new, status=None, stream=None):
    """kvc_paged_append: k_new/v_new [B, H_kv, D] to logical slot seq_lens[b]."""
    c = paged_desc(k_pages, v_pages, block_table)
    if k_new.stride() != v_new.stride() or k_new.dim() != 3:
        raise ValueError("k_new and v_new must be [B, H_kv, D] with equal strides")
    _check(load().kvc_paged_append(ctypes.byref(c), _ptr(seq_lens), _ptr(k_new), _ptr(v_new), k_new.stride(0),
                                   k_new.stride(1), _ptr(status), _stream(stream)), "kvc_paged_append")


def paged_workspace(k_pages, v_pages, block_table, n_q_heads: int, n_splits: int = 0) -> torch.Tensor:
    c = paged_desc(k_pages, v_pages, block_table)
    n = int(load().kvc_paged_decode_workspace_bytes(ctypes.byref(c), n_q_heads, n_splits))
    if n == 0:
        raise ValueError("invalid paged cache/head arguments for a decode workspace")
    return torch.zeros(n, dtype=torch.uint8, device=k_pages.device)


def paged_decode_attn(k_pages, v_pages, block_table, seq_lens, q, out, workspace, n_pending: int = 1, scale=None,
                      n_splits: int = 0, status=None, stream=None):
    c = paged_desc(k_pages, v_pages, block_table)
    if scale is None:
        scale = 1.0 / float(q.shape[-1]) ** 0.5
    if not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous [B, H_q, D]")
    _check(load().kvc_paged_decode_attn(ctypes.byref(c), _ptr(seq_lens), n_pending, _ptr(q), q.shape[1],
                                        float(scale), _ptr(out), DTYPE_CODE[out.dtype], _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), n_splits, _ptr(status),
                                        _stream(stream)), "kvc_paged_decode_attn")


def paged_decode_step(k_pages, v_pages, block_table, seq_lens, k_new, v_new, q, out, workspace, scale=None,
                      n_splits: int = 0, status=None, stream=None):
    c = paged_desc(k_pages, v_pages, block_table)
    if scale is None:
        scale = 1.0 / float(q.shape[-1]) ** 0.5
    if not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous [B, H_q, D]")
    if k_new.stride() != v_new.stride() or k_new.dim() != 3:
        raise ValueError("k_new and v_new must be [B, H_kv, D] with equal strides")
    _check(load().kvc_paged_decode_step(ctypes.byref(c), _ptr(seq_lens), _ptr(k_new), _ptr(v_new), k_new.stride(0),
                                        k_new.stride(1), _ptr(q), q.shape[1], float(scale), _ptr(out),
                                        DTYPE_CODE[out.dtype], _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), n_splits, _ptr(status),
                                        _stream(stream)), "kvc_paged_decode_step")


def ring_append(k_cache, v_cache, seq_lens, k_new, v_new, status=None, stream=None):
    """kvc_ring_append: token number seq_lens[b] into slot seq_lens[b] % W (W = T_max)."""
    c = cache_desc(k_cache, v_cache)
    if k_new.stride() != v_new.stride() or k_new.dim() != 3:
        raise ValueError("k_new and v_new must be [B, H_kv, D] with equal strides")
    _check(load().kvc_ring_append(ctypes.byref(c), _ptr(seq_lens), _ptr(k_new), _ptr(v_new), k_new.stride(0),
                                  k_new.stride(1), _ptr(status), _stream(stream)), "kvc_ring_append")


def ring_prefill_fill(k_cache, v_cache, seq_lens, k, v, status=None, stream=None):
    """kvc_ring_prefill_fill: k/v [B, H_kv, T_new, D] as token numbers seq_lens[b].. into the ring."""
    c = cache_desc(k_cache, v_cache)
    if k.stride() != v.stride() or k.dim() != 4:
        raise ValueError("k and v must be [B, H_kv, T_new, D] with equal strides")
    _check(load().kvc_ring_prefill_fill(ctypes.byref(c), _ptr(seq_lens), _ptr(k), _ptr(v), k.stride(0),
                                        k.stride(1), k.stride(2), k.shape[2], _ptr(status), _stream(stream)),
           "kvc_ring_prefill_fill")


def ring_decode_attn(k_cache, v_cache, seq_lens, q, out, workspace, n_pending: int = 1, scale=None,
                     n_splits: int = 0, status=None, stream=None):
    c = cache_desc(k_cache, v_cache)
    if scale is None:
        scale = 1.0 / float(q.shape[-1]) ** 0.5
    if not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous [B, H_q, D]")
    _check(load().kvc_ring_decode_attn(ctypes.byref(c), _ptr(seq_lens), n_pending, _ptr(q), q.shape[1],
                                       float(scale), _ptr(out), DTYPE_CODE[out.dtype], _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), n_splits, _ptr(status),
                                       _stream(stream)), "kvc_ring_decode_attn")


def ring_decode_step(k_cache, v_cache, seq_lens, k_new, v_new, q, out, workspace, scale=None, n_splits: int = 0,
                     status=None, stream=None):
    c = cache_desc(k_cache, v_cache)
    if scale is None:
        scale = 1.0 / float(q.shape[-1]) ** 0.5
    if not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous [B, H_q, D]")
    if k_new.stride() != v_new.stride() or k_new.dim() != 3:
        raise ValueError("k_new and v_new must be [B, H_kv, D] with equal strides")
    _check(load().kvc_ring_decode_step(ctypes.byref(c), _ptr(seq_lens), _ptr(k_new), _ptr(v_new), k_new.stride(0),
                                       k_new.stride(1), _ptr(q), q.shape[1], float(scale), _ptr(out),
                                       DTYPE_CODE[out.dtype], _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), n_splits, _ptr(status),
                                       _stream(stream)), "kvc_ring_decode_step")


def seq_lens_advance(seq_lens, n: int = 1, stream=None):
    _check(load().kvc_seq_lens_advance(_ptr(seq_lens), seq_lens.numel(), n, _stream(stream)),
           "kvc_seq_lens_advance")


def cache_bytes(n_layers: int, n_kv_heads: int, head_dim: int, dtype: torch.dtype, lengths) -> int:
    lens = [int(x) for x in lengths]
    arr = (ctypes.c_int32 * max(1, len(lens)))(*lens)
    return int(load().kvc_cache_bytes(n_layers, n_kv_heads, head_dim, DTYPE_CODE[dtype], arr, len(lens)))


def status_str(code: int) -> str:
    return load().kvc_status_str(code).decode()


def debug_set_merge_spin_limit(spins: int) -> int:
    """kvc_debug_set_merge_spin_limit (a test hook): polls before the split
    merge stops waiting and reports KVC_DEVERR_SYNC; returns the previous value."""
    return int(load().kvc_debug_set_merge_spin_limit(int(spins)))


# ------------------------------------------------------------ quantised cache --

def quant_append(qc: QCacheDesc, seq_lens, k_new, v_new, status=None, stream=None):
    """kvc_quant_append: quantise k_new/v_new [B, H_kv, D] into slot seq_lens[b]."""
    if k_new.stride() != v_new.stride() or k_new.dim() != 3:
        raise ValueError("k_new and v_new must be [B, H_kv, D] with equal strides")
    _check(load().kvc_quant_append(ctypes.byref(qc), _ptr(seq_lens), _ptr(k_new), _ptr(v_new), k_new.stride(0),
                                   k_new.stride(1), _ptr(status), _stream(stream)), "kvc_quant_append")


def quant_prefill_fill(qc: QCacheDesc, seq_lens, k, v, status=None, stream=None):
    """kvc_quant_prefill_fill: quantise k/v [B, H_kv, T_new, D] into slots [seq_lens[b], +T_new)."""
    if k.stride() != v.stride() or k.dim() != 4:
        raise ValueError("k and v must be [B, H_kv, T_new, D] with equal strides")
    _check(load().kvc_quant_prefill_fill(ctypes.byref(qc), _ptr(seq_lens), _ptr(k), _ptr(v), k.stride(0),
                                         k.stride(1), k.stride(2), k.shape[2], _ptr(status), _stream(stream)),
           "kvc_quant_prefill_fill")


def quant_workspace(qc: QCacheDesc, n_q_heads: int, n_splits: int = 0, device="cuda") -> torch.Tensor:
    """A zero-filled device workspace for the quantised decode calls."""
    n = int(load().kvc_quant_decode_workspace_bytes(ctypes.byref(qc), n_q_heads, n_splits))
    if n == 0:
        raise ValueError("invalid quantised cache/head arguments for a decode workspace")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def quant_decode_attn(qc: QCacheDesc, seq_lens, q, out, workspace, n_pending: int = 1, scale=None, n_splits: int = 0,
                      status=None, stream=None):
    """kvc_quant_decode_attn over the values the codes stand for."""
    if scale is None:
        scale = 1.0 / float(q.shape[-1]) ** 0.5
    if not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous [B, H_q, D]")
    _check(load().kvc_quant_decode_attn(ctypes.byref(qc), _ptr(seq_lens), n_pending, _ptr(q), q.shape[1],
                                        float(scale), _ptr(out), DTYPE_CODE[out.dtype], _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), n_splits, _ptr(status),
                                        _stream(stream)), "kvc_quant_decode_attn")


def quant_decode_step(qc: QCacheDesc, seq_lens, k_new, v_new, q, out, workspace, scale=None, n_splits: int = 0,
                      status=None, stream=None):
    """kvc_quant_decode_step: quantised append of the step's rows, then decode (n_pending = 1)."""
    if scale is None:
        scale = 1.0 / float(q.shape[-1]) ** 0.5
    if not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous [B, H_q, D]")
    if k_new.stride() != v_new.stride() or k_new.dim() != 3:
        raise ValueError("k_new and v_new must be [B, H_kv, D] with equal strides")
    _check(load().kvc_quant_decode_step(ctypes.byref(qc), _ptr(seq_lens), _ptr(k_new), _ptr(v_new),
                                        k_new.stride(0), k_new.stride(1), _ptr(q), q.shape[1], float(scale),
                                        _ptr(out), DTYPE_CODE[out.dtype], _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), n_splits, _ptr(status),
                                        _stream(stream)), "kvc_quant_decode_step")


def split_read_workspace(k_cache, v_cache, n_splits: int, desc=None) -> torch.Tensor:
    """Zero-filled workspace for kvc_split_read (one per geometry)."""
    lib = load()
    c = desc if desc is not None else cache_desc(k_cache, v_cache)
    n = int(lib.kvc_split_read_workspace_bytes(ctypes.byref(c), n_splits))
    if n == 0:
        raise KvcError(2, "kvc_split_read_workspace_bytes")
    return torch.zeros(n, dtype=torch.uint8, device=k_cache.device if k_cache is not None else "cuda")


def split_read(k_cache, v_cache, seq_lens, n_splits: int, out, workspace, stream=None, desc=None):
    """kvc_split_read: the decode launch's loads and split exchange without
    its arithmetic; out is [units, 128] 16-byte words (2 KB per (sequence, KV
    head) unit), the XOR fold of every word the unit's rows hold."""
    lib = load()
    c = desc if desc is not None else cache_desc(k_cache, v_cache)
    _check(lib.kvc_split_read(ctypes.byref(c), _ptr(seq_lens), n_splits, _ptr(out), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream)), "kvc_split_read")


def stream_read_rate(n_bytes: int = 4 << 30, grids=(512, 2048, 8192), reps: int = 5, device="cuda") -> float:
    """Best streaming-read rate in GB/s of kvc_stream_read over an n_bytes
    device buffer across the given grid sizes (per grid: one warm-up launch,
    then `reps` launches timed with HIP events on the launching stream)."""
    lib = load()
    buf = torch.empty(n_bytes, dtype=torch.uint8, device=device)
    sink = torch.empty(int(lib.kvc_stream_read_sink_bytes(max(grids))), dtype=torch.uint8, device=device)
    stream = torch.cuda.current_stream()
    best = 0.0
    for n_wg in grids:
        run = lambda: _check(lib.kvc_stream_read(_ptr(buf), n_bytes, _ptr(sink), n_wg, _stream(stream)),
                             "kvc_stream_read")
        run()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        best = max(best, n_bytes / (e0.elapsed_time(e1) / reps / 1e3) / 1e9)
    del buf, sink
    return best


def stream_read_launch_rate(launch_bytes: int, n_bytes: int = 4 << 30, grids=(256, 512, 1024), launches: int = 64,
                            device="cuda") -> float:
    """Best rate in GB/s of kvc_stream_read launches that each read
    launch_bytes (a multiple of 16) back to back, every launch a different
    region of an n_bytes buffer (at least two regions, so no launch finds its
    bytes in a cache), across the given grid sizes; timed with HIP events
    over `launches` launches per grid after one warm-up pass. This is what a
    kernel that only streams the same bytes in one launch reaches, fixed
    launch costs included."""
    if launch_bytes <= 0 or launch_bytes % 16:
        raise ValueError("launch_bytes must be a positive multiple of 16")
    lib = load()
    regions = max(2, n_bytes // launch_bytes)
    buf = torch.empty(regions * launch_bytes, dtype=torch.uint8, device=device)
    sink = torch.empty(int(lib.kvc_stream_read_sink_bytes(max(grids))), dtype=torch.uint8, device=device)
    stream = torch.cuda.current_stream()
    base = buf.data_ptr()
    best = 0.0
    for n_wg in grids:
        def run(i):
            _check(lib.kvc_stream_read(ctypes.c_void_p(base + (i % regions) * launch_bytes), launch_bytes,
                                       _ptr(sink), n_wg, _stream(stream)), "kvc_stream_read")
        for i in range(regions):
            run(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(launches):
            run(i)
        e1.record(stream)
        torch.cuda.synchronize()
        best = max(best, launch_bytes / (e0.elapsed_time(e1) / launches / 1e3) / 1e9)
    del buf, sink
    return best
