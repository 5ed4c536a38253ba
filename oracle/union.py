"""Union-of-G index sets and union attention in fp64 (TEST INFRASTRUCTURE:
oracle only).

sglang PR 32779, "Modifications" (``--dsa-triton-union``): a group of G
neighbouring tokens gathers one common index set, and each gathered row
carries bits naming the tokens that selected it, so every token's softmax
runs over its own rows only and the output matches per-token attention. Each
group's set is formed by sorting every member's rows separately; a row enters
the set under the first member that selected it, and its bits name every
member that selected it. "Accuracy Tests" states the
contract the tests check: no row appears twice, a row's bits are the union
of its holders' bits, and -1 slots are left out.

Canonical layout (the pages fix the membership, not the storage; this is the
reading the library follows):

* group g covers rows g*G .. min(g*G+G, T)-1; the last group of a T % G != 0
  batch simply has fewer members, and absent members own nothing;
* union_idx[g] lists token 0's distinct valid indices ascending, then token
  1's indices that token 0 lacks, ascending, and so on; then -1 fill;
* union_bits[g, r] has bit j set iff member j selected union_idx[g, r]
  (bit 0 = the group's first token); 0 fill;
* union_len[g] is the number of listed rows;
* an index is valid iff 0 <= x < kv_len; duplicates within one token's row
  collapse to one entry.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .attention import bf16_to_f64, kv_rows_f64, row_attention


def union_build(idx: np.ndarray, kv_len: int, G: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Returns union_idx int32 [ceil(T/G), G*k], union_bits uint8 [same],
    union_len int32 [ceil(T/G)]."""
    T, k = idx.shape
    n_groups = (T + G - 1) // G
    union_idx = np.full((n_groups, G * k), -1, dtype=np.int32)
    union_bits = np.zeros((n_groups, G * k), dtype=np.uint8)
    union_len = np.zeros(n_groups, dtype=np.int32)
    for g in range(n_groups):
        members = range(g * G, min(g * G + G, T))
        sets = []
        for t in members:
            sets.append({int(x) for x in idx[t] if 0 <= int(x) < kv_len})
        emitted = []
        earlier = set()
        for s in sets:
            for x in sorted(s):
                if x not in earlier:
                    emitted.append(x)
            earlier |= s
        for r, x in enumerate(emitted):
            bits = 0
            for j, s in enumerate(sets):
                if x in s:
                    bits |= 1 << j
            union_idx[g, r] = x
            union_bits[g, r] = bits
        union_len[g] = len(emitted)
    return union_idx, union_bits, union_len


def union_attention(q: np.ndarray, k: np.ndarray, v, union_idx: np.ndarray,
                    union_bits: np.ndarray, union_len: np.ndarray, G: int, *,
                    num_kv_heads: int, scale: float, head_dim_v=None,
                    rows=None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of each token over the union rows whose ownership bit it
    holds (PR 32779, "Modifications"). Same per-(row, head) definition as
    the per-token oracle, with the support taken from the union set."""
    T, Hq, _ = q.shape
    group = Hq // num_kv_heads
    dv = head_dim_v if v is None else v.shape[2]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    out = np.zeros((len(rows), Hq, dv))
    lse = np.zeros((len(rows), Hq))
    for r, t in enumerate(rows):
        g, j = divmod(int(t), G)
        n = int(union_len[g])
        own = (union_bits[g, :n] >> j) & 1
        tok = union_idx[g, :n][own.astype(bool)].astype(np.int64)
        for kvh in range(num_kv_heads):
            kr = kv_rows_f64(k[tok, kvh, :])
            vr = kr[:, :dv] if v is None else kv_rows_f64(v[tok, kvh, :])
            heads = slice(kvh * group, (kvh + 1) * group)
            o, s = row_attention(bf16_to_f64(q[t, heads, :]), kr, vr, scale)
            out[r, heads] = o
            lse[r, heads] = s
    return out, lse


def chunk_union_build(idx: np.ndarray, cu_seqlens_q: np.ndarray, cu_seqlens_kv: np.ndarray,
                      G: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Union sets over ragged requests: the union of PR 32779 ("Modifications")
    applied to the requests of the chunk kernel (PR 37275, "Kernel
    measurements"). Request r owns rows [cu_q[r], cu_q[r+1]) and KV rows
    [cu_kv[r], cu_kv[r+1]); its groups are G consecutive rows of its own
    (the last one may be short), so no group spans two requests, and its
    indices are local to its KV range. Groups are listed request by request.

    Returns union_idx int32 [groups, G*k], union_bits uint8 [same],
    union_len int32 [groups] (request-local indices, the union_build layout
    within each group) and group_request int32 [groups]."""
    T, k = idx.shape
    parts_i, parts_b, parts_l, owner = [], [], [], []
    for r in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[r]), int(cu_seqlens_q[r + 1])
        if q1 <= q0:
            continue
        kv_len = int(cu_seqlens_kv[r + 1] - cu_seqlens_kv[r])
        ui, ub, ul = union_build(idx[q0:q1], kv_len, G)
        parts_i.append(ui)
        parts_b.append(ub)
        parts_l.append(ul)
        owner.append(np.full(len(ul), r, dtype=np.int32))
    if not parts_l:
        return (np.zeros((0, G * k), np.int32), np.zeros((0, G * k), np.uint8),
                np.zeros(0, np.int32), np.zeros(0, np.int32))
    return (np.concatenate(parts_i), np.concatenate(parts_b), np.concatenate(parts_l),
            np.concatenate(owner))


def chunk_union_attention(q: np.ndarray, k: np.ndarray, v, union_idx: np.ndarray,
                          union_bits: np.ndarray, union_len: np.ndarray,
                          group_request: np.ndarray, cu_seqlens_q: np.ndarray,
                          cu_seqlens_kv: np.ndarray, G: int, *, num_kv_heads: int,
                          scale: float, head_dim_v=None,
                          rows=None) -> Tuple[np.ndarray, np.ndarray]:
    """Union attention of each request's rows over its own groups' lists and
    its own KV range (the per-row definition of union_attention)."""
    T = q.shape[0]
    dv = head_dim_v if v is None else v.shape[2]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    out = np.zeros((len(rows), q.shape[1], dv))
    lse = np.zeros((len(rows), q.shape[1]))
    req = np.searchsorted(cu_seqlens_q, rows, side="right") - 1
    for r in np.unique(req):
        sel = np.flatnonzero(req == r)
        q0, q1 = int(cu_seqlens_q[r]), int(cu_seqlens_q[r + 1])
        lo, hi = int(cu_seqlens_kv[r]), int(cu_seqlens_kv[r + 1])
        g = np.flatnonzero(group_request == r)
        o, s = union_attention(q[q0:q1], k[lo:hi], None if v is None else v[lo:hi],
                               union_idx[g], union_bits[g], union_len[g], G,
                               num_kv_heads=num_kv_heads, scale=scale, head_dim_v=head_dim_v,
                               rows=rows[sel] - q0)
        out[sel] = o
        lse[sel] = s
    return out, lse
