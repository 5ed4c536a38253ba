"""Seeded synthetic inputs for index-gathered sparse attention.

This module only draws random numbers and lays them out. It holds none of the
attention, union or page arithmetic, so both the fp64 oracle and the GPU path
can take their inputs from here without sharing any of the method's code.

Workloads follow the shapes the pages measure:

* sglang PR 37275 ("[QSA] Tune sm120 sparse prefill geometry"), section
  "Kernel measurements": 8192 query rows, 2051 selected token slots per row,
  head dim 256, one KV head, group 6 or 12, bf16.
* sglang PR 32779 (DSA ``triton_sparse_mla``), section "Modifications": the
  calibrated random-walk index generator (each token copies the previous
  token's set with about 2% of the slots swapped, plus -1 padding while the
  visible context is shorter than top-k); section "Speed Tests": 8 heads,
  576-wide latent rows (512 used as V), top-k 2048.
* sglang PR 32320 ("Only split touched SWA pages"): 256-token source pages
  split into 64-token pages, only about 2 x batch pages referenced.

bf16 values are stored as ``uint16`` bit patterns (numpy has no bf16 type),
rounded to nearest-even from float32 N(0, 1) draws.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "AttnCase",
    "PageCase",
    "bf16_bits_rne",
    "normal_bf16",
    "uniform_distinct_indices",
    "random_walk_indices",
    "make_attn_case",
    "make_ragged_case",
    "make_page_case",
    "make_config",
    "CONFIG_NAMES",
    "sha256_manifest",
]

# Fraction of slots replaced from one token to the next in the random walk
# (PR 32779, "Modifications": about 2% of rows swapped per step).
WALK_SWAP_FRAC = 0.02

# Children of the root SeedSequence, one per independent stream.
_STREAM_Q, _STREAM_K, _STREAM_V, _STREAM_IDX, _STREAM_LEN, _STREAM_POOL = range(6)
_N_STREAMS = 6


def _streams(seed: int) -> List[np.random.Generator]:
    children = np.random.SeedSequence(seed).spawn(_N_STREAMS)
    return [np.random.Generator(np.random.PCG64(c)) for c in children]


def bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """bf16 bits of float32 N(0, 1) draws."""
    return bf16_bits_rne(rng.standard_normal(size=shape, dtype=np.float32))


def uniform_distinct_indices(rng: np.random.Generator, positions: np.ndarray,
                             k: int) -> np.ndarray:
    """Row r holds min(k, p+1) distinct positions drawn uniformly from [0, p]
    (p = positions[r]) in random order, then -1 padding."""
    out = np.full((len(positions), k), -1, dtype=np.int32)
    for r, p in enumerate(positions):
        n = min(k, int(p) + 1)
        out[r, :n] = rng.choice(int(p) + 1, size=n, replace=False)
    return out


def _draw_unselected(rng: np.random.Generator, sel: np.ndarray, visible: int,
                     n: int, n_selected: int) -> np.ndarray:
    """n distinct positions, uniform over [0, visible) minus the selected set."""
    free = visible - n_selected
    if free < 64 * n + 64:
        cand = np.flatnonzero(~sel[:visible])
        return rng.choice(cand, size=n, replace=False).astype(np.int32)
    got: List[int] = []
    seen = set()
    while len(got) < n:
        for c in rng.integers(0, visible, size=2 * n):
            c = int(c)
            if not sel[c] and c not in seen:
                seen.add(c)
                got.append(c)
                if len(got) == n:
                    break
    return np.asarray(got, dtype=np.int32)


def random_walk_indices(rng: np.random.Generator, positions: np.ndarray, k: int,
                        swap_frac: float = WALK_SWAP_FRAC) -> np.ndarray:
    """Calibrated random-walk top-k rows over consecutive query positions.

    * A row whose visible prefix [0, p] fits in k slots holds 0..p in order,
      then -1 padding.
    * The first row that does not fit draws k distinct positions uniformly
      from [0, p], in random order.
    * Every later row copies the previous row and replaces round(swap_frac*k)
      slots (chosen uniformly, without replacement) by positions drawn
      uniformly from the visible but unselected positions (the count is capped
      by how many such positions exist).
    """
    positions = np.asarray(positions, dtype=np.int64)
    T = len(positions)
    out = np.full((T, k), -1, dtype=np.int32)
    if T == 0:
        return out
    n_swap = int(round(swap_frac * k))
    sel = np.zeros(int(positions.max()) + 1, dtype=bool)
    cur: Optional[np.ndarray] = None
    for r in range(T):
        p = int(positions[r])
        visible = p + 1
        if visible <= k:
            out[r, :visible] = np.arange(visible, dtype=np.int32)
            if cur is not None:
                sel[cur] = False
                cur = None
            continue
        if cur is None:
            cur = rng.choice(visible, size=k, replace=False).astype(np.int32)
            sel[cur] = True
        else:
            ns = min(n_swap, visible - k)
            if ns > 0:
                slots = rng.choice(k, size=ns, replace=False)
                new = _draw_unselected(rng, sel, visible, ns, k)
                cur = cur.copy()
                sel[cur[slots]] = False
                cur[slots] = new
                sel[new] = True
        out[r] = cur
    return out


@dataclasses.dataclass
class AttnCase:
    """One sparse attention workload (host arrays, natural layouts).

    q      uint16 bf16 bits [T, Hq, Dqk]
    k      uint16 bf16 bits [kv_total, Hkv, Dqk], or uint8 FP8 MLA records
           [kv_total, Hkv, 656] (mla_fp8_rows)
    v      uint16 bf16 bits [kv_total, Hkv, Dv], or None when V is the first
           Dv columns of each K row (MLA latent rows)
    idx    int32 [T, topk], token indices local to the row's request, -1 pad
    cu_seqlens_q / cu_seqlens_kv   ragged request bounds (None: one request
           whose KV length is kv_len)
    """
    name: str
    q: np.ndarray
    k: np.ndarray
    v: Optional[np.ndarray]
    idx: np.ndarray
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    scale: float
    kv_len: int
    positions: np.ndarray
    cu_seqlens_q: Optional[np.ndarray] = None
    cu_seqlens_kv: Optional[np.ndarray] = None

    @property
    def num_rows(self) -> int:
        return int(self.idx.shape[0])

    @property
    def topk(self) -> int:
        return int(self.idx.shape[1])

    @property
    def num_q_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def v_in_k(self) -> bool:
        return self.v is None

    def arrays(self) -> Dict[str, np.ndarray]:
        d = {"q": self.q, "k": self.k, "idx": self.idx, "positions": self.positions}
        if self.v is not None:
            d["v"] = self.v
        if self.cu_seqlens_q is not None:
            d["cu_seqlens_q"] = self.cu_seqlens_q
            d["cu_seqlens_kv"] = self.cu_seqlens_kv
        return d


def shuffle_slots(idx: np.ndarray, seed: int) -> np.ndarray:
    """The same index sets with every row's slot order permuted at random.

    The walk keeps a surviving token at its slot position from one row to the
    next; this variant removes that alignment while keeping each row's set,
    its padding and the overlap between rows.
    """
    return np.random.default_rng(seed).permuted(idx, axis=1)


FP8_ROW_BYTES = 656


def mla_fp8_rows(rng: np.random.Generator, tokens: int) -> np.ndarray:
    """FP8 MLA latent records, uint8 [tokens, 656]: 512 E4M3 latent codes,
    four fp32 block scales, 64 bf16 rope values (the record layout the
    oracle decodes). The latent values are N(0,1) draws; each 128-value
    block gets scale amax / 448 (E4M3's largest finite value) and its codes
    come from torch's float8_e4m3fn cast, so the record looks like a
    quantised cache row."""
    import torch
    x = rng.standard_normal((tokens, 4, 128), dtype=np.float32)
    scale = (np.abs(x).max(axis=2) / np.float32(448.0)).astype(np.float32)
    scale[scale == 0] = np.float32(1.0)
    codes = torch.from_numpy(x / scale[..., None]).to(torch.float8_e4m3fn).view(torch.uint8)
    rope = normal_bf16(rng, (tokens, 64))
    out = np.empty((tokens, FP8_ROW_BYTES), dtype=np.uint8)
    out[:, :512] = codes.numpy().reshape(tokens, 512)
    out[:, 512:528] = scale.astype("<f4").view(np.uint8)
    out[:, 528:] = rope.astype("<u2").view(np.uint8)
    return out


def make_attn_case(name: str, *, seed: int, num_rows: int, kv_len: int,
                   first_pos: int, num_q_heads: int, num_kv_heads: int,
                   head_dim_qk: int, head_dim_v: int, topk: int,
                   v_in_k: bool = False, walk: bool = True,
                   scale: Optional[float] = None, kv_fp8: bool = False) -> AttnCase:
    """One request: query rows at positions first_pos .. first_pos+num_rows-1
    over a KV buffer of kv_len tokens (kv_fp8: FP8 MLA records as K)."""
    rq, rk, rv, ri, _, _ = _streams(seed)
    positions = np.arange(first_pos, first_pos + num_rows, dtype=np.int64)
    q = normal_bf16(rq, (num_rows, num_q_heads, head_dim_qk))
    if kv_fp8:
        k = mla_fp8_rows(rk, kv_len * num_kv_heads).reshape(kv_len, num_kv_heads, FP8_ROW_BYTES)
    else:
        k = normal_bf16(rk, (kv_len, num_kv_heads, head_dim_qk))
    v = None if v_in_k else normal_bf16(rv, (kv_len, num_kv_heads, head_dim_v))
    if walk:
        idx = random_walk_indices(ri, positions, topk)
    else:
        idx = uniform_distinct_indices(ri, positions, topk)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim_qk)
    return AttnCase(name, q, k, v, idx, num_kv_heads, head_dim_qk, head_dim_v,
                    float(scale), kv_len, positions)


def make_ragged_case(name: str, *, seed: int, num_reqs: int, qlen_range, ctx_range,
                     num_q_heads: int, num_kv_heads: int, head_dim: int,
                     topk: int) -> AttnCase:
    """Ragged chunk prefill: request r has qlen_r rows at the end of a ctx_r
    token context; both drawn log-uniform and rounded, KV packed per request."""
    rq, rk, rv, ri, rl, _ = _streams(seed)
    lo_q, hi_q = qlen_range
    lo_c, hi_c = ctx_range
    qlens = np.rint(np.exp(rl.uniform(math.log(lo_q), math.log(hi_q), num_reqs))).astype(np.int64)
    ctxs = np.rint(np.exp(rl.uniform(math.log(lo_c), math.log(hi_c), num_reqs))).astype(np.int64)
    ctxs = np.maximum(ctxs, qlens)
    cu_q = np.zeros(num_reqs + 1, dtype=np.int32)
    cu_q[1:] = np.cumsum(qlens)
    cu_kv = np.zeros(num_reqs + 1, dtype=np.int64)
    cu_kv[1:] = np.cumsum(ctxs)
    T, kv_total = int(cu_q[-1]), int(cu_kv[-1])
    q = normal_bf16(rq, (T, num_q_heads, head_dim))
    k = normal_bf16(rk, (kv_total, num_kv_heads, head_dim))
    v = normal_bf16(rv, (kv_total, num_kv_heads, head_dim))
    idx = np.empty((T, topk), dtype=np.int32)
    positions = np.empty(T, dtype=np.int64)
    for r in range(num_reqs):
        pos = np.arange(ctxs[r] - qlens[r], ctxs[r], dtype=np.int64)
        positions[cu_q[r]:cu_q[r + 1]] = pos
        idx[cu_q[r]:cu_q[r + 1]] = random_walk_indices(ri, pos, topk)
    return AttnCase(name, q, k, v, idx, num_kv_heads, head_dim, head_dim,
                    1.0 / math.sqrt(head_dim), int(ctxs.max()), positions, cu_q, cu_kv)


@dataclasses.dataclass
class PageCase:
    """Decode KV pool and the sparse indices of one decode step.

    src    uint8 [num_src_pages, src_page_bytes]; a page is src_page_tokens
           rows of row_bytes, then src_page_tokens scales of scale_bytes
    idx    int32 [batch, topk] pool token ids (page * src_page_tokens + slot),
           -1 padding
    q      bf16 bits [batch, num_q_heads, 576]: the decode step's MLA queries
           (None for a pool of bytes only)
    """
    name: str
    src: np.ndarray
    idx: np.ndarray
    src_page_tokens: int
    dst_page_tokens: int
    row_bytes: int
    scale_bytes: int
    q: Optional[np.ndarray] = None
    scale: float = 1.0 / 24.0

    @property
    def num_src_pages(self) -> int:
        return int(self.src.shape[0])

    @property
    def src_page_bytes(self) -> int:
        return self.src_page_tokens * (self.row_bytes + self.scale_bytes)

    @property
    def dst_page_bytes(self) -> int:
        return self.dst_page_tokens * (self.row_bytes + self.scale_bytes)

    @property
    def ratio(self) -> int:
        return self.src_page_tokens // self.dst_page_tokens

    def arrays(self) -> Dict[str, np.ndarray]:
        out = {"src": self.src, "idx": self.idx}
        if self.q is not None:
            out["q"] = self.q
        return out


def make_page_case(name: str, *, seed: int, num_src_pages: int = 4096,
                   src_page_tokens: int = 256, dst_page_tokens: int = 64,
                   row_bytes: int = 656, scale_bytes: int = 4, batch: int = 32,
                   topk: int = 2048, window: int = 256, spread: bool = False,
                   num_q_heads: int = 8) -> PageCase:
    """Pool of random bytes plus one decode step's indices and queries.

    Each request owns its own pool pages (a random page table, disjoint across
    requests). Default: its slots hold the pool ids of its last `window`
    tokens, then -1, so about two pages per request are touched. With
    spread=True its topk slots are distinct positions spread over its whole
    context (a stress case that touches many pages).

    With 656-byte rows the token rows that the indices reference are
    overwritten with FP8 MLA records (mla_fp8_rows), and q holds batch x
    num_q_heads bf16 N(0,1) queries of width 576, so the step can also be
    attended; every other byte of the pool, the per-token scale words
    included, stays random."""
    rq, rk, _, ri, rl, rp = _streams(seed)
    page_bytes = src_page_tokens * (row_bytes + scale_bytes)
    src = rp.integers(0, 256, size=(num_src_pages, page_bytes), dtype=np.uint8)
    pages_per_req = num_src_pages // batch
    perm = rl.permutation(num_src_pages).reshape(batch, pages_per_req)
    max_ctx = pages_per_req * src_page_tokens
    idx = np.full((batch, topk), -1, dtype=np.int32)
    for b in range(batch):
        ctx = int(rl.integers(window + 1, max_ctx + 1))
        if spread:
            n = min(topk, ctx)
            pos = np.sort(ri.choice(ctx, size=n, replace=False))
        else:
            n = min(window, topk)
            pos = np.arange(ctx - n, ctx)
        page = perm[b, pos // src_page_tokens]
        idx[b, :n] = (page * src_page_tokens + pos % src_page_tokens).astype(np.int32)
    q = None
    if row_bytes == FP8_ROW_BYTES:
        tok = np.unique(idx[idx >= 0]).astype(np.int64)
        rec = mla_fp8_rows(rk, len(tok))
        page, slot = tok // src_page_tokens, tok % src_page_tokens
        cols = slot[:, None] * row_bytes + np.arange(row_bytes)[None, :]
        src[page[:, None], cols] = rec
        q = normal_bf16(rq, (batch, num_q_heads, 576))
    return PageCase(name, src, idx, src_page_tokens, dst_page_tokens, row_bytes, scale_bytes, q)


@dataclasses.dataclass
class TopkCase:
    """Indexer scores of one chunk of query rows and the selection budget.

    scores   float32 [T, kv_len]: row t's scores for positions 0 .. kv_len-1
    row_len  int32 [T]: positions visible to row t (its position + 1)
    """
    name: str
    scores: np.ndarray
    row_len: np.ndarray
    k: int

    def arrays(self) -> Dict[str, np.ndarray]:
        return {"scores": self.scores, "row_len": self.row_len}


def drifting_scores(rng: np.random.Generator, T: int, kv: int, drift: float) -> np.ndarray:
    """float32 [T, kv]: an N(0,1) base score per position plus, per
    position, a random walk over the rows with N(0, drift^2) steps, so that
    neighbouring rows rank positions almost alike."""
    x = rng.standard_normal(kv, dtype=np.float32)
    s = rng.standard_normal((T, kv), dtype=np.float32)
    s *= np.float32(drift)
    np.cumsum(s, axis=0, out=s)
    s += x
    return s


def make_topk_case(name: str, *, seed: int, num_rows: int, kv_len: int, first_pos: int,
                   k: int, drift: float = 0.027) -> TopkCase:
    """Rows at positions first_pos .. first_pos+num_rows-1 of one request.
    drift 0.027 changes about 2 % of a 2051-slot selection per row over
    ~30k visible positions, the walk's rate."""
    rng = _streams(seed)[3]
    scores = drifting_scores(rng, num_rows, kv_len, drift)
    row_len = np.arange(first_pos + 1, first_pos + num_rows + 1, dtype=np.int32)
    return TopkCase(name, scores, row_len, k)


CONFIG_NAMES = ("C0a", "C0b", "C1", "C2", "C3", "C3tail", "C3fp8", "C4", "C4decode",
                "C4spread", "C0topk", "C1topk")


def make_config(name: str, seed: int = 0):
    """The workloads, by name.

    C0a  128 rows at positions 0..127 over a 512-token KV buffer, top-k 64
         uniform distinct visible positions, -1 padded; 6 q heads / 1 KV head,
         d 256
    C0b  the same but rows at positions 384..511 (no padding)
    C1   8192 rows at the end of a 32768-token context, top-k 2051 random
         walk, group 6 over one KV head, d 256
    C2   8192 rows at the end of a 131072-token context, top-k 2051 walk,
         2 KV heads x 12 q heads, d 256
    C3   MLA: 4096 tokens from position 0, 8 heads over one 576-wide latent
         row per token (V = first 512 columns), top-k 2048 walk
    C3tail  1023 MLA rows at positions 3073..4095 (a group-size tail for
         union mode)
    C3fp8  C3 with the latent rows held as 656-byte FP8 records
    C4   16 ragged requests, qlen and context log-uniform in [512, 4096] and
         [8192, 65536], group 6 / one KV head, d 256, top-k 2051 walk
    C4decode  4096-page pool of 256-token pages (656 B rows plus 4 B scales),
         batch 32 x 2048 indices over each request's last 256 tokens (the
         referenced rows are FP8 MLA records), 8 MLA query heads per request
    C4spread  the same pool with 2048 indices spread over each context
    C0topk  indexer scores for 128 rows at positions 0..127 over 512
         positions, top-k 64 (rows t < 63 select everything and pad)
    C1topk  indexer scores for C1's 8192 rows (positions 24576..32767) over
         32768 positions, top-k 2051
    """
    if name == "C0a":
        return make_attn_case(name, seed=seed, num_rows=128, kv_len=512, first_pos=0,
                              num_q_heads=6, num_kv_heads=1, head_dim_qk=256,
                              head_dim_v=256, topk=64, walk=False)
    if name == "C0b":
        return make_attn_case(name, seed=seed, num_rows=128, kv_len=512, first_pos=384,
                              num_q_heads=6, num_kv_heads=1, head_dim_qk=256,
                              head_dim_v=256, topk=64, walk=False)
    if name == "C1":
        return make_attn_case(name, seed=seed, num_rows=8192, kv_len=32768,
                              first_pos=32768 - 8192, num_q_heads=6, num_kv_heads=1,
                              head_dim_qk=256, head_dim_v=256, topk=2051)
    if name == "C2":
        return make_attn_case(name, seed=seed, num_rows=8192, kv_len=131072,
                              first_pos=131072 - 8192, num_q_heads=24, num_kv_heads=2,
                              head_dim_qk=256, head_dim_v=256, topk=2051)
    if name == "C3":
        return make_attn_case(name, seed=seed, num_rows=4096, kv_len=4096, first_pos=0,
                              num_q_heads=8, num_kv_heads=1, head_dim_qk=576,
                              head_dim_v=512, topk=2048, v_in_k=True)
    if name == "C3tail":
        return make_attn_case(name, seed=seed, num_rows=1023, kv_len=4096,
                              first_pos=4096 - 1023, num_q_heads=8, num_kv_heads=1,
                              head_dim_qk=576, head_dim_v=512, topk=2048, v_in_k=True)
    if name == "C3fp8":
        return make_attn_case(name, seed=seed, num_rows=4096, kv_len=4096, first_pos=0,
                              num_q_heads=8, num_kv_heads=1, head_dim_qk=576,
                              head_dim_v=512, topk=2048, v_in_k=True, kv_fp8=True)
    if name == "C4":
        return make_ragged_case(name, seed=seed, num_reqs=16, qlen_range=(512, 4096),
                                ctx_range=(8192, 65536), num_q_heads=6, num_kv_heads=1,
                                head_dim=256, topk=2051)
    if name == "C4decode":
        return make_page_case(name, seed=seed)
    if name == "C4spread":
        return make_page_case(name, seed=seed, spread=True)
    if name == "C0topk":
        return make_topk_case(name, seed=seed, num_rows=128, kv_len=512, first_pos=0, k=64)
    if name == "C1topk":
        return make_topk_case(name, seed=seed, num_rows=8192, kv_len=32768,
                              first_pos=32768 - 8192, k=2051)
    raise KeyError(f"unknown config {name!r}; known: {CONFIG_NAMES}")


def sha256_manifest(arrays: Dict[str, np.ndarray]) -> Dict[str, str]:
    """SHA-256 of every array's bytes (C order), with dtype and shape."""
    out = {}
    for key in sorted(arrays):
        a = np.ascontiguousarray(arrays[key])
        h = hashlib.sha256()
        h.update(f"{a.dtype.str}{a.shape}".encode())
        h.update(a.tobytes())
        out[key] = h.hexdigest()
    return out
