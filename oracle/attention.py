"""Per-token sparse attention in fp64 (TEST INFRASTRUCTURE: oracle only).

What is computed (sglang PR 37275, "Motivation" and the mechanism paragraph
under it; PR 32779, "Motivation"): each query row t selects its own top-k
token slots, given as int32 indices with -1 as padding; every query head h of
the KV group kvh scores the selected K rows, a softmax over those scores
weights the selected V rows, and the result is written per (row, head).

For row t of a request whose KV buffer holds kv_len tokens, and head h:

    kvh = h // group                      (contiguous GQA groups)
    J   = { j : 0 <= idx[t, j] < kv_len }  (and j < topk_len[t] when given)
    s_j = scale * <Q[t, h, :], K[idx[t, j], kvh, :]>
    m   = max_j s_j ;  w_j = exp(s_j - m) ;  l = sum_j w_j
    O[t, h, :] = sum_j w_j * V[idx[t, j], kvh, :] / l
    LSE[t, h]  = m + ln(l)

Readings where the pages are silent:

* An index outside [0, kv_len) is masked like -1 (the pages' tests cover
  negative and out-of-range selected indices without stating the
  semantics; the library never dereferences such a slot).
* An empty support gives O = 0 and LSE = -inf.
* A duplicated index counts with its multiplicity (PR 32779, "Accuracy
  Tests": on the per-token path a row selected twice counts twice).
* MLA latent rows: V is the first Dv columns of the K row (PR 32779, "Speed
  Tests": 576-wide rows, 512 used as V).
* No causal mask beyond the index set: the indexer owns causality.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def kv_rows_f64(rows: np.ndarray) -> np.ndarray:
    """K/V rows as float64: bf16 bit patterns (uint16) are widened exactly;
    rows already decoded to float64 (the FP8 MLA rows, see fp8.py) pass
    through."""
    rows = np.asarray(rows)
    return rows if rows.dtype == np.float64 else bf16_to_f64(rows)


def row_attention(q_heads: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray,
                  scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of a few query heads over an explicit list of rows.

    q_heads [H, Dqk], k_rows [n, Dqk], v_rows [n, Dv], all float64.
    Returns O [H, Dv] and LSE [H]; n == 0 gives zeros and -inf.
    """
    H = q_heads.shape[0]
    if k_rows.shape[0] == 0:
        return np.zeros((H, v_rows.shape[1])), np.full(H, -np.inf)
    s = scale * (q_heads @ k_rows.T)                  # [H, n]
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    l = w.sum(axis=1, keepdims=True)
    o = (w @ v_rows) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def _valid_slots(idx_row: np.ndarray, kv_len: int, limit: Optional[int]) -> np.ndarray:
    j = np.arange(idx_row.shape[0])
    ok = (idx_row >= 0) & (idx_row < kv_len)
    if limit is not None:
        ok &= j < limit
    return idx_row[ok].astype(np.int64)


def sparse_attention(q: np.ndarray, k: np.ndarray, v: Optional[np.ndarray],
                     idx: np.ndarray, *, num_kv_heads: int, scale: float,
                     kv_len: Optional[int] = None, head_dim_v: Optional[int] = None,
                     topk_len: Optional[np.ndarray] = None,
                     rows: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Sparse attention for the rows of one request (definition above).

    q    bf16 bits [T, Hq, Dqk]
    k    bf16 bits [kv, Hkv, Dqk]
    v    bf16 bits [kv, Hkv, Dv], or None: V = K[..., :head_dim_v]
    idx  int32 [T, topk]
    rows optional subset of row numbers to evaluate (others are not computed)

    Returns (O float64 [len(rows), Hq, Dv], LSE float64 [len(rows), Hq]).
    """
    T, Hq, _ = q.shape
    kv_len = k.shape[0] if kv_len is None else kv_len
    group = Hq // num_kv_heads
    if v is None:
        if head_dim_v is None:
            raise ValueError("head_dim_v is required when V lives in K")
        dv = head_dim_v
    else:
        dv = v.shape[2]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    out = np.zeros((len(rows), Hq, dv))
    lse = np.zeros((len(rows), Hq))
    for r, t in enumerate(rows):
        limit = None if topk_len is None else int(topk_len[t])
        tok = _valid_slots(idx[t], kv_len, limit)
        for kvh in range(num_kv_heads):
            kr = kv_rows_f64(k[tok, kvh, :])
            vr = kr[:, :dv] if v is None else kv_rows_f64(v[tok, kvh, :])
            heads = slice(kvh * group, (kvh + 1) * group)
            o, s = row_attention(bf16_to_f64(q[t, heads, :]), kr, vr, scale)
            out[r, heads] = o
            lse[r, heads] = s
    return out, lse


def chunk_prefill(q: np.ndarray, k: np.ndarray, v: Optional[np.ndarray],
                  idx: np.ndarray, cu_seqlens_q: np.ndarray, cu_seqlens_kv: np.ndarray,
                  *, num_kv_heads: int, scale: float, head_dim_v: Optional[int] = None,
                  rows: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Ragged chunk prefill (PR 37275, "Kernel measurements": the chunk kernel
    runs when a prompt continues a cached prefix, i.e. for each chunk past
    the first).

    Request r owns query rows [cu_seqlens_q[r], cu_seqlens_q[r+1]) and the KV
    tokens [cu_seqlens_kv[r], cu_seqlens_kv[r+1]) of the packed K/V buffers;
    its indices are local to that KV range. Each row is then the per-token
    definition over its own request's KV.
    """
    T = idx.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    dv = head_dim_v if v is None else v.shape[2]
    out = np.zeros((len(rows), q.shape[1], dv))
    lse = np.zeros((len(rows), q.shape[1]))
    req = np.searchsorted(cu_seqlens_q, rows, side="right") - 1
    for r in np.unique(req):
        sel = np.flatnonzero(req == r)
        lo, hi = int(cu_seqlens_kv[r]), int(cu_seqlens_kv[r + 1])
        o, s = sparse_attention(q, k[lo:hi], None if v is None else v[lo:hi], idx,
                                num_kv_heads=num_kv_heads, scale=scale,
                                kv_len=hi - lo, head_dim_v=head_dim_v, rows=rows[sel])
        out[sel] = o
        lse[sel] = s
    return out, lse
