"""Sparse MLA decode over the split pages (TEST INFRASTRUCTURE: oracle only).

sglang PR 32320 ("Only split touched SWA pages in FlashMLA page-split
kernel"): in every decode step the page split re-lays the pool in pages of
64 tokens, and the sparse MLA decode kernel that runs after it ("Accuracy
Tests", the profile table) attends over those pages. Its arithmetic is the
per-token sparse attention of attention.py: one query row per request, the
MLA head set over one latent row per token (576 wide, the first 512 columns
serving as V), each row the 656-byte FP8 record of fp8.py.

For request b, head h, with P = num_pages * page_tokens pool tokens:

    J   = { j : 0 <= idx[b, j] < P }       (and j < topk_len[b] when given)
    t   = idx[b, j]
    row = record at page t // page_tokens, byte (t % page_tokens) * row_bytes
    then O[b, h], LSE[b, h] as in attention.py over those rows, a duplicated
    index counting with its multiplicity

Readings (the pages give the decode kernel by name only):

* Token ids are the pool ids of the page mark, t = page * 256 + slot of the
  256-token source pages. The split sends rows [s * 64, (s + 1) * 64) of
  source page p to destination page p * 4 + s, so token t sits in
  destination page t // 64 at row t % 64.
* A token row is one FP8 MLA record (fp8.py). The 4-byte word stored per
  token after a page's rows (the pages call it a scale but give it no role
  in attention; the record carries the scales of all its FP8 values) is not
  read.
* Ids outside [0, P) are masked like -1; an empty support gives O = 0 and
  LSE = -inf.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .attention import bf16_to_f64, row_attention
from .fp8 import mla_fp8_rows_to_f64

RECORD_BYTES = 656
HEAD_DIM_V = 512


def paged_record(pool: np.ndarray, t: int, *, page_tokens: int,
                 row_bytes: int = RECORD_BYTES) -> np.ndarray:
    """The row_bytes of token t in a pool of pages (uint8 [pages, stride])."""
    page, row = divmod(int(t), page_tokens)
    return pool[page, row * row_bytes:(row + 1) * row_bytes]


def paged_decode(q: np.ndarray, pool: np.ndarray, idx: np.ndarray, *, page_tokens: int,
                 scale: float, topk_len: Optional[np.ndarray] = None,
                 row_bytes: int = RECORD_BYTES) -> Tuple[np.ndarray, np.ndarray]:
    """q bf16 bits [B, Hq, 576]; pool uint8 [num_pages, page_stride] (pages of
    page_tokens records of row_bytes, then the per-token words); idx int32
    [B, topk] pool token ids. Returns (O float64 [B, Hq, 512], LSE [B, Hq])."""
    B, Hq, _ = q.shape
    tokens = pool.shape[0] * page_tokens
    out = np.zeros((B, Hq, HEAD_DIM_V))
    lse = np.zeros((B, Hq))
    for b in range(B):
        limit = idx.shape[1] if topk_len is None else max(0, min(int(topk_len[b]), idx.shape[1]))
        tok = [int(t) for t in idx[b, :limit] if 0 <= t < tokens]
        rec = np.zeros((len(tok), row_bytes), dtype=np.uint8)
        for i, t in enumerate(tok):
            rec[i] = paged_record(pool, t, page_tokens=page_tokens, row_bytes=row_bytes)
        rows = mla_fp8_rows_to_f64(rec)
        out[b], lse[b] = row_attention(bf16_to_f64(q[b]), rows, rows[:, :HEAD_DIM_V], scale)
    return out, lse
