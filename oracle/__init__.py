"""CPU oracle for paged decode attention over a block-table KV cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls, links or
runs this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` do. It shares no code, header, table or
constant with the HIP library under ``paged_kv_decode_splitk_amd/``.

Everything here is plain NumPy. Attention is computed in float64 by the
textbook definition (gather the pages into contiguous K/V, dequantize, softmax,
weighted sum); the number formats and cache writes follow their definitions
value by value.

Sources (the three pages the method is taken from):

* metrale API page ``metrale_model_layers/layers/ops/prefill_attn_b.rs``,
  cited below as ``[metrale: <function>]`` after the launcher whose doc comment
  states the fact (``reshape_and_cache_nvfp4``, ``bf16_absmax``,
  ``paged_decode_attn_splitk_nvfp4``, ``paged_decode_attn_splitk_fp8``,
  ``paged_decode_attn_splitk_bf16``, ``paged_decode_attn_reduce_fp8``).
* AstrAI commit log for ``csrc/tests``, cited as ``[AstrAI log: <topic>]``.
* pegainfer issue #1008, cited as ``[pegainfer #1008: <section>]``.

Where the pages leave a step open, the reading taken is tagged ``(R<n>)``
with the same numbering the design notes use.

Pins: every function here is pinned by ``tests/test_oracle_*.py`` against
library routines (torch's float8_e4m3fn cast and decode, torch's
scaled_dot_product_attention in float64), brute-force searches and
invariants. No function is "parity unpinned".
"""
from .formats import (
    E4M3_MAX,
    E2M1_MAX,
    bf16_to_f64,
    e4m3_values,
    e4m3_decode,
    e4m3_encode,
    e2m1_values,
    e2m1_decode,
    e2m1_encode,
    nvfp4_encode_groups,
    nvfp4_decode_groups,
)
from .cache import (
    CacheGeometry,
    new_cache,
    reshape_and_cache,
    bf16_absmax,
    read_kv_rows,
)
from .attention import (
    window_start,
    paged_decode_attention,
    attention_rows,
    split_page_bound,
    split_partials,
    combine_partials,
    query_range,
    paged_prefill_attention,
    contiguous_kv_rows,
    contiguous_attention,
)

__all__ = [
    "E4M3_MAX", "E2M1_MAX", "bf16_to_f64", "e4m3_values", "e4m3_decode",
    "e4m3_encode", "e2m1_values", "e2m1_decode", "e2m1_encode",
    "nvfp4_encode_groups", "nvfp4_decode_groups", "CacheGeometry", "new_cache",
    "reshape_and_cache", "bf16_absmax", "read_kv_rows", "window_start",
    "paged_decode_attention", "attention_rows", "split_page_bound",
    "split_partials", "combine_partials", "query_range",
    "paged_prefill_attention", "contiguous_kv_rows", "contiguous_attention",
]
