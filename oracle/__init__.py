"""Plain CPU fp64 oracle for the per-layer incremental decode step.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The GPU library
(``kv_cache_append_amd``) never imports, links or calls it, and this package
never imports the GPU library: the two share no code, only the seeded inputs
from ``synth``.

What it computes follows three web pages on the KV cache, cited by title and
section:

* [KVG]  glossary entry "KV 缓存" (llm-glossary.tokens-kit.com/terms/kv-cache/)
* [W1D4] course notes "第 1 周 · Day 4：KV Cache 与 MQA / GQA"
         (semidirectx.com/notes/courses/cme295/week1-day4/)
* [LA11] textbook section "11.7 KV Cache：形状、显存与带宽"
         (yongzhen.wang/Linear-Algebra-to-LLM/learn/m11/kv-cache/)

Every function here is pinned by a ``-m "not gpu"`` test against something other
than itself (closed forms, the pages' printed values, a library routine,
invariants or 50-digit brute force); none is "parity unpinned".
"""

from .kvc_oracle import (  # noqa: F401
    append,
    QFMT_FP8_E4M3,
    QFMT_INT8,
    QMAX,
    cache_bytes,
    causal_attention,
    chunk_attention,
    concat_append_positions,
    code_value,
    decode_attention,
    dequantize,
    e4m3_decode_one,
    e4m3_encode_one,
    int8_encode_one,
    kv_head_of,
    paged_append,
    paged_decode_attention,
    paged_prefill_fill,
    paged_slot,
    paged_view,
    prealloc_append_positions,
    prefill_fill,
    project,
    quant_append,
    quant_decode_attention,
    quant_prefill_fill,
    quantize_rows,
    ring_append,
    ring_decode_attention,
    ring_slot,
    toy_path_a,
    toy_path_b,
    widen,
)
