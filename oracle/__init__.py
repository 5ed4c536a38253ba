"""fp64 CPU oracle for index-gathered sparse attention (TEST INFRASTRUCTURE).

This package is a plain, slow, obviously correct restatement of what the
GPU library computes. Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import it; the library and its Python binding never
do, and this package imports nothing from them. Its inputs come from the
seeded generators in ``gen`` (random draws only, no method arithmetic).

Modules
-------
attention   per-token sparse attention and ragged chunk prefill
union       union-of-G index build (sorted, deduplicated, ownership bits) and
            union attention
pages       decode-pool page mark and (masked) page split
fp8         the 656-byte FP8 MLA record and its dequantisation to bf16
decode      sparse MLA decode over the split pages of FP8 records
topk        the indexer's top-k selection from scores to index rows

Every function cites the passage of the pages it restates. Where the pages
leave a point open, the reading taken is stated at the function.

Parity status: every function here is pinned by CPU tests against
definitions outside this package (dense float64 attention in torch, mpmath
brute force, closed forms, Python-set semantics, numpy reshapes); none is
"parity unpinned".
"""
from .attention import bf16_to_f64, kv_rows_f64, sparse_attention, chunk_prefill, row_attention
from .union import union_build, union_attention, chunk_union_build, chunk_union_attention
from .pages import page_mark, page_split
from .fp8 import fp8_e4m3_to_f64, mla_fp8_rows_to_f64
from .decode import paged_decode, paged_record
from .topk import topk_select

__all__ = [
    "bf16_to_f64",
    "sparse_attention",
    "chunk_prefill",
    "row_attention",
    "kv_rows_f64",
    "union_build",
    "union_attention",
    "chunk_union_build",
    "chunk_union_attention",
    "fp8_e4m3_to_f64",
    "mla_fp8_rows_to_f64",
    "paged_decode",
    "paged_record",
    "topk_select",
    "page_mark",
    "page_split",
]
