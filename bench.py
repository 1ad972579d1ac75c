"""Decode-step benchmark: achieved HBM GB/s of KV-cache decode attention.

One step is the whole per-layer incremental-decode path over all L layers of
one batch: for every layer kvc_decode_step (the new token's k, v written into
slot T_b and every query head attending T_b + 1 tokens, one launch), the last
layer's launch (kvc_decode_step_advance) also writing seq_lens + 1 for the next
step into a second length array (steps alternate the two arrays). The value is
KV bytes read per step, 2*L*H_kv*D*s*sum_b(T_b + 1), divided by the step time,
with every input already resident in HBM. The lengths are reset to the
workload's before the timed steps, so step k attends T_b + k + 1 tokens; the
byte count follows that exactly.

Prints ONE JSON line. Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attention achieved HBM GB/s (KV bytes read/step time) and % of peak"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
DOMINANT_KERNEL = "decode_kernel"
# each decode kernel's sources (a counter record is tied to its kernel's code)
KERNEL_SOURCES = {k: [os.path.join(ROOT, "kv_cache_append_amd", "csrc", f) for f in files]
                  for k, files in (("decode_kernel", ("kvc_kernels.hip", "kvc_internal.h")),
                                   ("wide_decode_kernel", ("kvc_wide.hip", "kvc_tile.h", "kvc_internal.h")))}


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="gqa_8b")
    ap.add_argument("--also", default="ragged_long,mha_7b,gqa_70b,mqa_70b",
                    help="comma-separated workloads measured in the same run after --config, each with its own "
                         "value, step time and roofline in the line's 'workloads' list ('none' to skip)")
    ap.add_argument("--splits", type=int, default=0, help="decode splits (0 = library choice)")
    ap.add_argument("--paged", type=int, default=0,
                    help="page size P: time the decode step on page pools through a page table "
                         "(kvc_paged_decode_step) instead of contiguous caches")
    ap.add_argument("--ring", type=int, default=0,
                    help="window W: time the decode step on ring caches of W slots (kvc_ring_decode_step, "
                         "sliding-window attention over the most recent W tokens) instead of full caches")
    ap.add_argument("--quant", choices=["fp8", "int8"], default=None,
                    help="time the decode step on a quantised cache (8-bit codes + per-token fp32 scales; "
                         "kvc_quant_decode_step) instead of the 16-bit cache")
    ap.add_argument("--layout", choices=["bhtd", "bthd"], default="bhtd",
                    help="cache storage order: [B, H_kv, T, D] (head-major) or [B, T, H_kv, D] (token-major, "
                         "viewed as [B, H_kv, T, D] through strides)")
    ap.add_argument("--page-order", choices=["random", "interleaved"], default="random",
                    help="paged caches: pages handed out in a random order, or interleaved by position "
                         "(page p of every sequence adjacent, as sequences growing together receive them)")
    ap.add_argument("--block-q", type=int, default=0,
                    help="time a block of N new tokens per sequence per layer (kvc_block_step: the block's "
                         "fill and its attention, e.g. a speculative verify step) instead of the decode step")
    ap.add_argument("--prefill", type=int, default=0,
                    help="time a prompt prefill of N tokens per sequence on the config's layer shape instead "
                         "of the decode step: per layer kvc_prefill_fill + kvc_prefill_attn (causal attention "
                         "on the matrix cores); one JSON line in TFLOP/s")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="wall-clock budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=7)
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU run: turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of a "
                         "--calib-copy-mib run into HBM bytes per decode launch, written to --pmc-out")
    ap.add_argument("--pmc-out", default=None, help="output JSON of --pmc-summary")
    ap.add_argument("--stream-gib", type=int, default=4,
                    help="GiB read by the streaming-read calibration (kvc_stream_read); 0 skips it")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB (a known-size reference "
                         "for HBM byte counters in a profiled run)")
    return ap.parse_args()


class Workload:
    """All L layers of one decode step, resident in HBM, with pre-marshalled
    C-ABI arguments (so the timed loop does no Python-side tensor work)."""

    def __init__(self, cfg, margin_tokens: int, seed: int, splits: int, block_q: int = 0, page: int = 0,
                 ring: int = 0, quant=None, layout: str = "bhtd", page_order: str = "random"):
        import torch
        import kv_cache_append_amd as kvc
        import synth

        self.cfg = cfg
        self.block_q = block_q        # 0: decode step; N: block of N new tokens per sequence
        self.page = page              # 0: contiguous caches; P: page pools of P-token pages
        self.ring = ring              # 0: full caches; W: ring caches of the most recent W tokens
        self.quant = quant            # None: 16-bit cache; "fp8" / "int8": 8-bit codes + per-token scales
        self.kvc = kvc
        self.lib = kvc.load()
        dev = torch.device("cuda:0")
        # device status word (KVC_DEVERR_* bits) passed to every call of the run
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.lengths = cfg.lengths(seed)
        self.t_max = ring if ring else int(self.lengths.max()) + margin_tokens + 1
        L, B, Hkv, Hq, D = cfg.n_layers, cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.head_dim
        tdt = synth.DTYPES[cfg.dtype]
        # contiguous 16-bit caches with 8..512 (query, head) pairs per KV head
        # and blocks of at most 64 queries run on the wide-group kernel; other
        # blocks of 8+ queries and 32+ pairs on the prefill kernel
        pairs = cfg.group * max(block_q, 1)
        sixteen = cfg.dtype in ("fp16", "bf16") and cfg.head_dim in (64, 128)
        self.block_prefill = (bool(block_q) and sixteen and block_q >= 8 and pairs >= 32
                              and not (8 <= pairs <= 512 and block_q <= 64))
        self.wide = not (page or ring or quant) and sixteen and 8 <= pairs <= 512 and not self.block_prefill
        self.fused_advance = not (block_q or page or ring or quant)   # (see below)
        if quant:
            self._init_quant(cfg, seed, splits, dev, tdt)
            return
        if page:
            # page pools per layer and one page table (a random permutation of
            # the pool's pages) shared by the layers, as a serving runtime keeps it
            per_seq = -(-self.t_max // page)
            self.t_max = per_seq * page
            n_pages = B * per_seq
            g = torch.Generator().manual_seed(synth.derive_seed(seed, cfg.name, "pages"))
            if page_order == "interleaved":   # page p of sequence b is pool page p * B + b
                perm = (torch.arange(per_seq).view(1, per_seq) * B + torch.arange(B).view(B, 1)).to(torch.int32)
            else:
                perm = torch.randperm(n_pages, generator=g).to(torch.int32)
            self.table = perm.reshape(B, per_seq).to(dev)
            self.k = torch.empty((L, n_pages, Hkv, page, D), dtype=tdt, device=dev)
        elif layout == "bthd":   # token-major storage, the heads of a token adjacent
            self.k = torch.empty((L, B, self.t_max, Hkv, D), dtype=tdt, device=dev).transpose(2, 3)
        else:
            self.k = torch.empty((L, B, Hkv, self.t_max, D), dtype=tdt, device=dev)
        self.v = torch.empty_like(self.k)
        for l in range(L):  # fill layer by layer (bounded fp32 temporaries)
            synth.normal(None, cfg.dtype, seed, cfg.name, l, "K", out=self.k[l])
            synth.normal(None, cfg.dtype, seed, cfg.name, l, "V", out=self.v[l])
        nq = max(block_q, 1)
        qs = (B, block_q, Hq, D) if block_q else (B, Hq, D)
        ks = (B, Hkv, block_q, D) if block_q else (B, Hkv, D)
        self.q = torch.stack([synth.normal(qs, cfg.dtype, seed, cfg.name, l, "q", device=dev) for l in range(L)])
        self.k_new = torch.stack([synth.normal(ks, cfg.dtype, seed, cfg.name, l, "k_new", device=dev)
                                  for l in range(L)])
        self.v_new = torch.stack([synth.normal(ks, cfg.dtype, seed, cfg.name, l, "v_new", device=dev)
                                  for l in range(L)])
        self.out = torch.empty((L,) + qs, dtype=torch.float32, device=dev)
        self.seq_lens = self.lengths.to(dev)
        # The decode step on contiguous 16-bit-or-fp32 caches ends with
        # kvc_decode_step_advance: the last layer's launch also writes the next
        # step's lengths into the other of two arrays (no separate advance
        # launch), so consecutive steps alternate the arrays.
        self.fused_advance = not (block_q or page or ring or quant)
        self.seq_lens_alt = torch.empty_like(self.seq_lens)
        if page:
            self.descs = [kvc.paged_desc(self.k[l], self.v[l], self.table) for l in range(L)]
        else:
            self.descs = [kvc.cache_desc(self.k[l], self.v[l]) for l in range(L)]
        # the library's split choice for the lengths the first timed step attends
        attended = self._attended_at_start()
        if not page:
            self.splits = splits if splits > 0 else kvc.decode_splits(self.k[0], self.v[0], Hq * nq, lengths=attended)
        if page:
            # the split choice of the contiguous cache with the same capacity
            logical = kvc.CacheDesc(self.k.data_ptr(), self.v.data_ptr(), B, Hkv, self.t_max, D,
                                    kvc.DTYPE_CODE[tdt], 0, Hkv * self.t_max * D, self.t_max * D, D)
            self.splits = splits if splits > 0 else kvc.decode_splits(None, None, Hq, lengths=attended,
                                                                      desc=logical)
            self.ws = kvc.paged_workspace(self.k[0], self.v[0], self.table, Hq, self.splits)
        elif block_q:
            self.ws = kvc.block_workspace(self.k[0], self.v[0], Hq, block_q, self.splits)
        else:
            self.ws = kvc.workspace(self.k[0], self.v[0], Hq, self.splits)
        self.scale = ctypes.c_float(1.0 / math.sqrt(D))
        torch.cuda.synchronize()

    def _init_quant(self, cfg, seed, splits, dev, tdt):
        """Codes [L, B, H_kv, T_max, D] and scales [L, B, H_kv, T_max], each
        layer quantised on the device from seeded N(0,1) rows of the
        workload's dtype by kvc_quant_prefill_fill."""
        import torch
        import synth
        kvc = self.kvc
        L, B, Hkv, Hq, D = cfg.n_layers, cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.head_dim
        T = self.t_max
        self.kc = torch.empty((L, B, Hkv, T, D), dtype=torch.uint8, device=dev)
        self.vc = torch.empty_like(self.kc)
        self.ks = torch.empty((L, B, Hkv, T), dtype=torch.float32, device=dev)
        self.vs = torch.empty_like(self.ks)
        fmt = kvc.QFMT[self.quant]
        self.descs = [kvc.qcache_desc(self.kc[l], self.vc[l], self.ks[l], self.vs[l], fmt, tdt) for l in range(L)]
        zero = torch.zeros(B, dtype=torch.int32, device=dev)
        krows = torch.empty((B, Hkv, T, D), dtype=tdt, device=dev)
        vrows = torch.empty_like(krows)
        for l in range(L):   # every slot of the layer, quantised from fresh rows
            synth.normal(None, cfg.dtype, seed, cfg.name, l, "K", out=krows)
            synth.normal(None, cfg.dtype, seed, cfg.name, l, "V", out=vrows)
            kvc.quant_prefill_fill(self.descs[l], zero, krows, vrows)
        del krows, vrows
        self.q = torch.stack([synth.normal((B, Hq, D), cfg.dtype, seed, cfg.name, l, "q", device=dev)
                              for l in range(L)])
        self.k_new = torch.stack([synth.normal((B, Hkv, D), cfg.dtype, seed, cfg.name, l, "k_new", device=dev)
                                  for l in range(L)])
        self.v_new = torch.stack([synth.normal((B, Hkv, D), cfg.dtype, seed, cfg.name, l, "v_new", device=dev)
                                  for l in range(L)])
        self.out = torch.empty((L, B, Hq, D), dtype=torch.float32, device=dev)
        self.seq_lens = self.lengths.to(dev)
        logical = kvc.CacheDesc(self.kc.data_ptr(), self.vc.data_ptr(), B, Hkv, T, D, kvc.DTYPE_CODE[tdt], 0,
                                Hkv * T * D, T * D, D)
        # the length-blind rule: the launch model behind the length-aware
        # choice is calibrated on the 16-bit kernels only
        self.splits = splits if splits > 0 else kvc.decode_splits(None, None, Hq, desc=logical)
        self.ws = kvc.quant_workspace(self.descs[0], Hq, self.splits)
        self.scale = ctypes.c_float(1.0 / math.sqrt(D))
        torch.cuda.synchronize()

    def _attended_at_start(self):
        """Tokens each sequence attends in the first step (host values)."""
        n = self.lengths.to("cpu").long() + max(self.block_q, 1)
        if self.ring:
            n = n.clamp(max=self.ring)
        return n.tolist()

    def reset_lengths(self):
        self.seq_lens.copy_(self.lengths.to(self.seq_lens.device))
        if hasattr(self, "seq_lens_alt"):
            self.seq_lens_alt.copy_(self.seq_lens)

    def layers(self, stream_handle, attn_only: bool = False, lens_in=None, lens_out=None):
        """Enqueue the per-layer decode launches of one step (lengths unchanged).
        attn_only (quantised cache): only the decode launch of each layer, which
        reads the same bytes as in the step (the slot it appends is attended).
        lens_in / lens_out: the step's length array and, for the last layer's
        kvc_decode_step_advance, the array the next step's lengths go to."""
        lib, cfg = self.lib, self.cfg
        vp = ctypes.c_void_p
        seq = vp((self.seq_lens if lens_in is None else lens_in).data_ptr())
        stat = vp(self.status.data_ptr())
        ws, wsb = vp(self.ws.data_ptr()), ctypes.c_size_t(self.ws.numel())
        sb, sh = self.k_new.stride(1), self.k_new.stride(2)
        st = vp(stream_handle)
        if self.block_q:
            n = self.block_q
            ks = self.k_new.stride()
            for l in range(cfg.n_layers):
                d = ctypes.byref(self.descs[l])
                rc = lib.kvc_block_step(d, seq, n, vp(self.k_new[l].data_ptr()), vp(self.v_new[l].data_ptr()),
                                        ks[1], ks[2], ks[3], vp(self.q[l].data_ptr()), cfg.n_q_heads, self.scale,
                                        vp(self.out[l].data_ptr()), 0, ws, wsb, self.splits, stat, st)
                if rc:
                    raise RuntimeError(f"libkvc returned {rc} at layer {l}")
            return
        if self.quant and attn_only:
            for l in range(cfg.n_layers):
                rc = lib.kvc_quant_decode_attn(ctypes.byref(self.descs[l]), seq, 1, vp(self.q[l].data_ptr()),
                                               cfg.n_q_heads, self.scale, vp(self.out[l].data_ptr()), 0, ws, wsb,
                                               self.splits, stat, st)
                if rc:
                    raise RuntimeError(f"libkvc returned {rc} at layer {l}")
            return
        step_fn = (lib.kvc_paged_decode_step if self.page else
                   lib.kvc_ring_decode_step if self.ring else
                   lib.kvc_quant_decode_step if self.quant else lib.kvc_decode_step)
        for l in range(cfg.n_layers):
            d = ctypes.byref(self.descs[l])
            if lens_out is not None and l == cfg.n_layers - 1:
                rc = lib.kvc_decode_step_advance(d, seq, vp(lens_out.data_ptr()), vp(self.k_new[l].data_ptr()),
                                                 vp(self.v_new[l].data_ptr()), sb, sh, vp(self.q[l].data_ptr()),
                                                 cfg.n_q_heads, self.scale, vp(self.out[l].data_ptr()), 0, ws, wsb,
                                                 self.splits, stat, st)
            else:
                rc = step_fn(d, seq, vp(self.k_new[l].data_ptr()), vp(self.v_new[l].data_ptr()), sb, sh,
                             vp(self.q[l].data_ptr()), cfg.n_q_heads, self.scale,
                             vp(self.out[l].data_ptr()), 0, ws, wsb, self.splits, stat, st)
            if rc:
                raise RuntimeError(f"libkvc returned {rc} at layer {l}")

    def step(self, stream_handle, parity: int = 0):
        """Enqueue one decode step: every layer, then seq_lens += 1 (in the
        last layer's launch when fused_advance: step `parity` 0 reads
        seq_lens and writes seq_lens_alt, parity 1 the reverse)."""
        if self.fused_advance:
            a, b = (self.seq_lens, self.seq_lens_alt) if parity % 2 == 0 else (self.seq_lens_alt, self.seq_lens)
            self.layers(stream_handle, lens_in=a, lens_out=b)
            return
        self.layers(stream_handle)
        seq = ctypes.c_void_p(self.seq_lens.data_ptr())
        if self.lib.kvc_seq_lens_advance(seq, self.cfg.batch, max(self.block_q, 1), ctypes.c_void_p(stream_handle)):
            raise RuntimeError("kvc_seq_lens_advance failed")

    def attended_tokens(self, step_index: int) -> int:
        """Tokens all sequences attend at step `step_index` from the reset
        lengths (a ring caps each sequence at its window)."""
        nq = max(self.block_q, 1)
        lens = self.lengths.to("cpu").long() + nq * (step_index + 1)
        if self.ring:
            lens = lens.clamp(max=self.ring)
        return int(lens.sum())

    def token_bytes(self) -> int:
        """K+V bytes of one token of one layer: 2 * H_kv * D * s, or for a
        quantised cache 2 * H_kv * (D code bytes + a 4-byte scale)."""
        row = self.cfg.head_dim + 4 if self.quant else self.cfg.head_dim * self.cfg.elem_bytes
        return 2 * self.cfg.n_kv_heads * row

    def kv_bytes(self, steps: int) -> int:
        """KV bytes read by `steps` steps starting from the reset lengths."""
        return self.cfg.n_layers * self.token_bytes() * sum(self.attended_tokens(k) for k in range(steps))

    def decode_launch_bytes(self, step_index: int) -> int:
        """Algorithmic K+V bytes one decode launch (one layer) reads at a step."""
        return self.token_bytes() * self.attended_tokens(step_index)


def _measure(w: Workload, steps: int, warmup: int, use_graph: bool):
    import torch

    stream = torch.cuda.current_stream()
    for i in range(max(warmup, 1)):
        w.step(stream.cuda_stream, i)
    torch.cuda.synchronize()
    # one HIP graph per step; with the fused advance two, one per direction
    # of the length arrays, replayed alternately
    graphs = None
    if use_graph:
        w.reset_lengths()
        torch.cuda.synchronize()
        graphs = []
        for parity in range(2 if w.fused_advance else 1):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                w.step(torch.cuda.current_stream().cuda_stream, parity)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(max(warmup, 1)):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()

    def run_step(i):
        if graphs is not None:
            graphs[i % len(graphs)].replay()
        else:
            w.step(stream.cuda_stream, i)

    # timed region: exactly `steps` steps from the reset lengths, back to back
    w.reset_lengths()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        run_step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = e0.elapsed_time(e1)
    # each step's own time, from a second pass over the same steps with an
    # event after every step (kept out of the timed region)
    w.reset_lengths()
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    marks[0].record()
    for i in range(steps):
        run_step(i)
        marks[i + 1].record()
    torch.cuda.synchronize()
    step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(steps)]
    # Average duration of one decode launch: the L per-layer launches alone
    # (lengths held, so every launch reads the same bytes), `reps` passes back
    # to back, bracketed by HIP events on the launching stream.
    w.reset_lengths()
    torch.cuda.synchronize()
    reps = max(2, min(steps, 10))
    layers_graph = None
    if use_graph:
        layers_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(layers_graph):
            w.layers(torch.cuda.current_stream().cuda_stream, attn_only=bool(w.quant))
        torch.cuda.synchronize()
        layers_graph.replay()
    else:
        w.layers(stream.cuda_stream, attn_only=bool(w.quant))
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        if layers_graph is not None:
            layers_graph.replay()
        else:
            w.layers(stream.cuda_stream, attn_only=bool(w.quant))
    e1.record()
    torch.cuda.synchronize()
    avg_launch_ms = e0.elapsed_time(e1) / (reps * w.cfg.n_layers)
    avg_launch_bytes = w.decode_launch_bytes(0)
    return ms_total, wall, avg_launch_ms, avg_launch_bytes, step_ms


def _split_read_ms(w: Workload, use_graph: bool, reps: int = 10):
    """Average duration in ms of one kvc_split_read launch -- the decode
    launch's workgroups, K/V loads and split exchange without the attention's
    arithmetic -- over the L layers' caches with the step's split count and
    the lengths the per-launch pass held, back to back (one HIP graph of the
    L launches), bracketed by HIP events on the launching stream."""
    import torch
    import kv_cache_append_amd as kvc
    cfg, lib, vp = w.cfg, w.lib, ctypes.c_void_p
    units = cfg.batch * cfg.n_kv_heads
    out = torch.empty(units * 2048, dtype=torch.uint8, device=w.k.device)
    ws = kvc.split_read_workspace(w.k[0], w.v[0], w.splits)
    seq = vp(w.seq_lens.data_ptr())

    def run(h):
        for l in range(cfg.n_layers):
            if lib.kvc_split_read(ctypes.byref(w.descs[l]), seq, w.splits, vp(out.data_ptr()), vp(ws.data_ptr()),
                                  ws.numel(), vp(h)):
                raise RuntimeError("kvc_split_read failed")

    stream = torch.cuda.current_stream()
    g = None
    if use_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    (g.replay() if g is not None else run(stream.cuda_stream))
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        (g.replay() if g is not None else run(stream.cuda_stream))
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * cfg.n_layers)


def _kernel_fingerprint(kernel: str) -> str:
    """SHA-256 of the kernel's sources with comments and whitespace removed,
    so that counter records stay tied to the code and not to its comments."""
    import re
    src = "".join(open(p).read() for p in KERNEL_SOURCES[kernel])
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = re.sub(r"\s+", " ", src).strip()
    return hashlib.sha256(src.encode()).hexdigest()


def _traffic(workload_name: str):
    """HBM bytes per decode launch from committed rocprofv3 counter runs, if
    they were taken on the current kernel code; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_code_sha256") != _kernel_fingerprint(rec.get("kernel", "decode_kernel")):
        return None
    return rec.get("hbm_bytes_per_launch")


def _pmc_summary(fetch_csv: str, write_csv: str, out_path: str, args):
    """HBM traffic of the decode kernel from rocprofv3 counters. FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) are each scaled by what they read for the
    device-to-device copy of --calib-copy-mib MiB in the same run (that copy
    reads and writes exactly that many bytes)."""
    import csv

    def per_kernel(path, counter):
        out = {"decode": [], "copy": []}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = ("decode" if ("decode_kernel" in name or "wide_decode_kernel" in name) else
                   "copy" if "copyBuffer" in name else None)
            if key:
                out[key].append(float(r["Counter_Value"]))
        return out

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    wr = per_kernel(write_csv, "WRITE_SIZE")
    if not (f["decode"] and f["copy"] and wr["decode"] and wr["copy"]):
        raise SystemExit("counter CSVs lack decode_kernel or copy dispatches")
    copy_bytes = args.calib_copy_mib << 20
    f_scale = copy_bytes / (max(f["copy"]) * 1024)
    w_scale = copy_bytes / (max(wr["copy"]) * 1024)
    fetch = sum(f["decode"]) / len(f["decode"]) * 1024 * f_scale
    write = sum(wr["decode"]) / len(wr["decode"]) * 1024 * w_scale
    import synth
    cfg = synth.CONFIGS[args.config]
    algo = 2 * cfg.n_kv_heads * cfg.head_dim * cfg.elem_bytes * (int(cfg.lengths(args.seed).long().sum()) + cfg.batch)
    kernel = ("wide_decode_kernel" if cfg.dtype in ("fp16", "bf16") and cfg.head_dim in (64, 128) and cfg.group >= 8
              else "decode_kernel")
    rec = {
        "workload": args.config,
        "kernel": kernel,
        "kernel_code_sha256": _kernel_fingerprint(kernel),
        "hbm_bytes_per_launch": int(round(fetch + write)),
        "fetch_bytes_per_launch": int(round(fetch)),
        "write_bytes_per_launch": int(round(write)),
        "algorithmic_kv_bytes_per_launch": algo,
        "fetch_scale": round(f_scale, 4),
        "write_scale": round(w_scale, 4),
        "calib_copy_bytes": copy_bytes,
        "decode_dispatches": len(f["decode"]),
    }
    with open(out_path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def _host_cpu() -> dict:
    """Cores this process may run on and the host CPU's model name."""
    try:
        cores = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        cores = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"affinity_cores": int(cores), "cpu_model": model}


def _cpu_baseline(cfg, seconds: float, seed: int):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload:
    whole layers of (sequence, KV head) units at the workload's shapes, timed
    until about `seconds` of wall clock. Reports KV GB/s of the oracle."""
    import numpy as np
    import torch
    import synth
    import oracle
    host = _host_cpu()
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    # the oracle's loop is one Python thread; its matrix-vector products run on
    # the BLAS pool, which cannot use more cores than the process may run on
    threads = max(1, min(blas_threads, host["affinity_cores"]))
    lengths = cfg.lengths(seed)
    done_bytes, units, t_spent = 0, 0, 0.0
    b = 0
    inputs = {}
    # (sequence, layer) slices in step order, repeated over later steps until
    # about `seconds` of oracle time (at most 100 steps); each sequence's
    # inputs are drawn once
    while t_spent < seconds and b < 100 * cfg.batch * cfg.n_layers:
        i = b % cfg.batch
        n = int(lengths[i]) + 1
        kv = cfg.n_kv_heads
        if i not in inputs:
            inputs[i] = (synth.normal((1, cfg.n_q_heads, cfg.head_dim), cfg.dtype, seed, "cpu", i, "q"),
                         synth.normal((1, kv, n, cfg.head_dim), cfg.dtype, seed, "cpu", i, "K"),
                         synth.normal((1, kv, n, cfg.head_dim), cfg.dtype, seed, "cpu", i, "V"))
        q, k, v = inputs[i]
        t0 = time.perf_counter()
        oracle.decode_attention(q, k, v, np.array([n - 1]), n_pending=1)
        t_spent += time.perf_counter() - t0
        done_bytes += 2 * kv * n * cfg.head_dim * cfg.elem_bytes
        units += kv
        b += 1
    del inputs
    return {
        "value": round(done_bytes / t_spent / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "affinity_cores": host["affinity_cores"],
        "cpu_model": host["cpu_model"],
        "blas_threads": int(blas_threads),
        "sample": f"{b} (sequence, layer) slices of {cfg.name} ({b / (cfg.batch * cfg.n_layers):.2f} steps), all "
                  f"{cfg.n_kv_heads} KV heads each ({units} (sequence, KV head) units, {cfg.group} query heads "
                  f"each, {done_bytes / 1e9:.3f} GB of K+V) in {t_spent:.1f} s; numpy fp64 on one Python thread, its matrix-vector "
                  f"products on {threads} BLAS threads ({host['affinity_cores']} cores in the process affinity mask, "
                  f"{host['cpu_model']})",
    }


def _run_config(name, args, with_cpu):
    import torch
    import synth
    cfg = synth.CONFIGS[name]
    nq = max(args.block_q, 1)
    margin = (max(args.steps, args.warmup) + 2) * nq
    if sum(bool(x) for x in (args.ring, args.block_q, args.paged, args.quant)) > 1:
        raise SystemExit("--ring, --block-q, --paged and --quant are separate modes")
    if args.layout != "bhtd" and (args.paged or args.quant):
        raise SystemExit("--layout applies to contiguous 16-bit caches")
    w = Workload(cfg, margin, args.seed, args.splits, args.block_q, args.paged, args.ring, args.quant, args.layout,
                 args.page_order)
    ms_total, wall, launch_ms, launch_bytes, step_ms = _measure(w, args.steps, args.warmup, not args.no_graph)
    # the same bytes per launch read by a kernel that only streams them
    import kv_cache_append_amd as kvc
    launch_read = (kvc.stream_read_launch_rate(int(launch_bytes) // 16 * 16, n_bytes=args.stream_gib << 30)
                   if args.stream_gib > 0 else None)
    # the same launches' loads and split exchange without the arithmetic
    # (contiguous caches, the decode step)
    split_read_ms = (None if (args.block_q or args.paged or args.ring or args.quant or args.layout != "bhtd")
                     else _split_read_ms(w, not args.no_graph))
    torch.cuda.synchronize()
    status = int(w.status.item())          # KVC_DEVERR_* bits of every call of the run (0 expected)
    step_sorted = sorted(step_ms)
    kv = w.kv_bytes(args.steps)
    gbs = kv / (ms_total / 1e3) / 1e9
    achieved = launch_bytes / (launch_ms / 1e3) / 1e9
    lens = w.lengths
    res = {
        "value": round(gbs, 2),
        "unit": "GB/s",
        "ms_per_step": round(ms_total / args.steps, 5),
        # each step's own time (HIP events between steps); steps later in the
        # run attend slightly more tokens
        "step_ms": {"median": round(step_sorted[len(step_sorted) // 2], 5), "min": round(step_sorted[0], 5),
                    "max": round(step_sorted[-1], 5)},
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 5),
        "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "steps_per_s": round(args.steps / (ms_total / 1e3), 2),
        "tokens_per_s": round(cfg.batch * args.steps / (ms_total / 1e3), 1),
        "kv_bytes_per_step": kv // args.steps,
        "status": status,
        "dtype": cfg.dtype,
        "config": {
            "workload": name, "description": cfg.description, "layers": cfg.n_layers, "batch": cfg.batch,
            "n_q_heads": cfg.n_q_heads, "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim,
            "cached_tokens_at_start": {"min": int(lens.min()), "max": int(lens.max()),
                                       "sum": int(lens.long().sum())},
            "splits": w.splits, "hip_graph": not args.no_graph,
            **({"query_block": args.block_q} if args.block_q else {}),
            **({"page_size": args.paged, "page_order": args.page_order} if args.paged else {}),
            **({"window": args.ring} if args.ring else {}),
            **({"layout": args.layout} if args.layout != "bhtd" else {}),
            **({"kv_format": args.quant, "kv_bytes_per_token_head": cfg.head_dim + 4} if args.quant else {}),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": (("wide_decode_kernel (kvc_block_step per layer: the block's fill and attention in one launch)"
                        if w.wide else "copy_rows_kernel + " + ("prefill_kernel" if w.block_prefill else "decode_kernel") +
                        " (kvc_block_step per layer: fill, then attention; time per layer covers both)")
                       if args.block_q else
                       "decode_kernel (kvc_ring_decode_step: ring append + windowed attention + merge, one "
                       "launch per layer)" if args.ring else
                       "decode_kernel on 8-bit codes (kvc_quant_decode_attn, timed alone; the step adds one "
                       "quantising append launch per layer)" if args.quant else
                       ("wide_decode_kernel" if w.wide else "decode_kernel") +
                       " (kvc_decode_step: append + attention + merge, one launch per layer; the last layer's "
                       "launch also advances the lengths)"),
            "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "launch_ms": round(launch_ms, 5), "launch_bytes": int(launch_bytes),
            **({"stream_read_gbs": round(args.stream_gbs, 1), "frac_of_stream": round(achieved / args.stream_gbs, 4)}
               if args.stream_gbs else {}),
            **({"split_read_us": round(split_read_ms * 1e3, 2),
                "frac_of_split_read": round(split_read_ms / launch_ms, 4)} if split_read_ms is not None else {}),
            **({"launch_read_gbs": round(launch_read, 1), "frac_of_launch_read": round(achieved / launch_read, 4)}
               if launch_read else {}),
            # counters are taken for the default mode (16-bit contiguous cache)
            "traffic": None if (args.block_q or args.paged or args.ring or args.quant) else _traffic(name),
        },
    }
    if with_cpu:
        res["cpu_baseline"] = _cpu_baseline(cfg, args.cpu_seconds, args.seed)
    del w
    torch.cuda.empty_cache()
    return res


MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0}   # MI355X dense matrix-core peak per 16-bit type


def _run_prefill(args) -> dict:
    """A prompt prefill on the config's layer shape: every sequence starts
    empty and takes --prefill N tokens. Per layer, kvc_prefill_fill writes the
    prompt's K/V into that layer's cache and kvc_prefill_attn computes the
    causal attention of its N queries. FLOPs count q.K and P.V (2 each per
    query, key and head-dim element) over the keys each query sees,
    N(N+1)/2 per (sequence, query head)."""
    import torch
    import kv_cache_append_amd as kvc
    import synth
    cfg = synth.CONFIGS[args.config]
    if cfg.dtype not in MFMA_PEAK_TFLOPS:
        raise SystemExit(f"--prefill needs a 16-bit cache ({cfg.name} is {cfg.dtype})")
    B, hq, hkv, d, n_layers, t = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_layers, args.prefill
    dev = torch.device("cuda:0")
    tdt = synth.DTYPES[cfg.dtype]
    k = [torch.empty((B, hkv, t, d), dtype=tdt, device=dev) for _ in range(n_layers)]
    v = [torch.empty_like(x) for x in k]
    k_src = synth.normal((B, hkv, t, d), cfg.dtype, args.seed, cfg.name, "prefill", "K", device=dev)
    v_src = synth.normal((B, hkv, t, d), cfg.dtype, args.seed, cfg.name, "prefill", "V", device=dev)
    q = synth.normal((B, t, hq, d), cfg.dtype, args.seed, cfg.name, "prefill", "q", device=dev)
    out = torch.empty_like(q)
    seq = torch.zeros(B, dtype=torch.int32, device=dev)
    descs = [kvc.cache_desc(k[i], v[i]) for i in range(n_layers)]

    def fill_all():
        for i in range(n_layers):
            kvc.prefill_fill(k[i], v[i], seq, k_src, v_src)

    def attn_all():
        for i in range(n_layers):
            kvc.prefill_attn(k[i], v[i], seq, q, out, desc=descs[i])

    for _ in range(args.warmup):
        fill_all()
        attn_all()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record()
    for s_ in range(args.steps):
        fill_all()
        attn_all()
        ev[s_ + 1].record()
    torch.cuda.synchronize()
    step_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    ms_total = ev[0].elapsed_time(ev[-1])
    reps = 3                                    # attention launches alone, for the roofline
    e0.record()
    for _ in range(reps):
        attn_all()
    e1.record()
    torch.cuda.synchronize()
    launch_ms = e0.elapsed_time(e1) / (reps * n_layers)
    flops_launch = 4.0 * d * hq * B * t * (t + 1) / 2
    ms_step = ms_total / args.steps
    value = flops_launch * n_layers / (ms_step * 1e-3) / 1e12
    achieved = flops_launch / (launch_ms * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[cfg.dtype]
    srt = sorted(step_ms)
    return {
        "metric": "prompt-prefill causal attention TFLOP/s (q.K and P.V FLOPs / step time)",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step,
        "step_ms": {"median": srt[len(srt) // 2], "min": srt[0], "max": srt[-1]},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) prompt q/K/V rounded to the cache dtype; no dataset)",
        "config": {"workload": f"{cfg.name} prompt prefill", "batch": B, "prompt_tokens": t, "n_layers": n_layers,
                   "n_q_heads": hq, "n_kv_heads": hkv, "head_dim": d,
                   "step": "per layer kvc_prefill_fill + kvc_prefill_attn"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": None, "launch_us": launch_ms * 1e3,
                     "flops_per_launch": flops_launch},
    }


def main():
    args = _parse()
    if args.pmc_summary:
        _pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.pmc_out or "traffic.json", args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): this build has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.prefill > 0:
        print(json.dumps(_run_prefill(args)), flush=True)
        return
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # the chip's streaming-read rate with the decode kernel's loads, over 4 GiB
    # (far past the on-chip caches): the achievable ceiling beside the 8 TB/s peak
    args.stream_gbs = None
    if args.stream_gib > 0:
        import kv_cache_append_amd as kvc
        args.stream_gbs = kvc.stream_read_rate(n_bytes=args.stream_gib << 30)
        torch.cuda.empty_cache()
    main_res = _run_config(args.config, args, with_cpu=not args.no_cpu_baseline)
    line = {
        "metric": METRIC,
        "value": main_res["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "step_ms": main_res["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": main_res["dtype"],
        "data": "synthetic (seeded N(0,1) q/K/V rounded to the cache dtype; no dataset)",
        "config": main_res["config"],
        "pct_of_peak": main_res["pct_of_peak"],
        "steps_per_s": main_res["steps_per_s"],
        "tokens_per_s": main_res["tokens_per_s"],
        "wall_ms_per_step": main_res["wall_ms_per_step"],
        "kv_bytes_per_step": main_res["kv_bytes_per_step"],
        "status": main_res["status"],
        "roofline": main_res["roofline"],
    }
    if "cpu_baseline" in main_res:
        line["cpu_baseline"] = main_res["cpu_baseline"]
    # the other workloads, each on its own resident caches (freed in between)
    others = [x for x in (args.also or "").split(",") if x and x != "none" and x != args.config]
    if others:
        line["workloads"] = []
        for name in others:
            r = _run_config(name, args, with_cpu=False)
            line["workloads"].append({"workload": name, **{k: r[k] for k in (
                "value", "unit", "ms_per_step", "step_ms", "pct_of_peak", "steps_per_s", "tokens_per_s",
                "kv_bytes_per_step", "status", "dtype", "config", "roofline")}})
    bad = [(e["config"]["workload"] if "config" in e else "?", e["status"])
           for e in [main_res] + line.get("workloads", []) if e["status"]]
    print(json.dumps(line), flush=True)
    if bad:
        print(f"device status bits set during the run: {bad}", file=sys.stderr)
        sys.exit(3)


if __name__ == "__main__":
    main()
