"""Indexer top-k selection (TEST INFRASTRUCTURE: oracle only).

sglang PR 37275, "Motivation": the indexer gives every query row a budget
of 2051 token slots (its top-k plus the compression ratio, minus one), and
a row that sees fewer tokens than that uses fewer slots; "Not covered": the
sparse kernels take the selected rows as they come. The scoring needs trained weights and stays outside; what is
restated here is the selection, from given fp32 scores to the int32 index
rows the attention entry points take.

For row t with visible length n_t (positions 0 .. n_t - 1 of the row's
scores; n_t = kv_len when no lengths are given):

    n_t <= k :  idx[t] = 0, 1, .., n_t - 1, then -1 up to k
    n_t >  k :  S_t = the k positions j < n_t of largest score[t, j], where
                a larger score wins and equal scores go to the lower position;
                idx[t] = S_t in ascending order

Readings (the pages name the selection but not its tie rule, its output
order or its padding beyond shorter rows using fewer slots):

* Ties in value go to the lower position; -0.0 and +0.0 are equal values
  (plain float comparison). Scores are never NaN.
* The selected positions are written in ascending order: the attention
  result does not depend on the order, the union build sorts its rows anyway,
  and ascending rows keep neighbouring rows' gathers close together.
* A row with n_t <= k selects every visible position and pads with -1, the
  padding the attention entry points skip.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def topk_select(scores: np.ndarray, k: int, row_len: Optional[np.ndarray] = None) -> np.ndarray:
    """scores float32 [T, kv]; row_len int [T] visible lengths (None = kv).
    Returns int32 [T, k]."""
    T, kv = scores.shape
    out = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        n = kv if row_len is None else max(0, min(int(row_len[t]), kv))
        if n <= k:
            out[t, :n] = np.arange(n, dtype=np.int32)
            continue
        v = scores[t, :n].astype(np.float64)                # exact widening
        order = np.lexsort((np.arange(n), -v))              # value down, then position up
        out[t] = np.sort(order[:k]).astype(np.int32)
    return out
