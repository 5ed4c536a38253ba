"""GPU parity: a seeded sweep of small random cases over the attention entry
points (per-token, ragged chunk prefill, union, union over ragged requests),
both head shapes and both K encodings, against the fp64 oracle. Each case
draws its own group size, row count (tails not a multiple of any team or
group), top-k, KV length, padded strides, top-k lengths, -1 and
out-of-range indices; odd cases also hold a duplicated index in every row
(even cases let two-row teams match their rows by membership)."""
import numpy as np
import pytest
import torch

import gen
import oracle
import top_index_sparse_amd as sa
from tests.gpu_util import bf16_dev, check_close, i32_dev, i64_dev, say

pytestmark = pytest.mark.gpu

N_CASES = 100


def _padded(t, extra):
    """The same rows at a row stride `extra` elements longer."""
    buf = torch.zeros((t.shape[0], t[0].numel() + extra), dtype=t.dtype, device=t.device)
    buf[:, :t[0].numel()] = t.reshape(t.shape[0], -1)
    return buf[:, :t[0].numel()].view(t.shape)


def _case(i):
    rng = np.random.default_rng(1000 + i)
    mla = bool(rng.integers(0, 3) == 0)
    fp8 = mla and bool(rng.integers(0, 2))
    if mla:
        hkv, hq = 1, int(rng.choice([1, 2, 3, 5, 8, 13, 16, 24, 32]))
        dqk, dv = 576, 512
    else:
        hkv = int(rng.choice([1, 2, 3]))
        hq = hkv * int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 16, 20, 27, 32]))
        dqk = dv = 256
    kv = int(rng.integers(1, 700))
    T = int(rng.integers(1, 70))
    topk = int(rng.integers(1, 300))
    c = gen.make_attn_case("sweep", seed=2000 + i, num_rows=T, kv_len=kv,
                           first_pos=int(rng.integers(0, kv)), num_q_heads=hq, num_kv_heads=hkv,
                           head_dim_qk=dqk, head_dim_v=dv, topk=topk, v_in_k=mla, walk=False,
                           kv_fp8=fp8)
    idx = c.idx.copy()
    # plant -1, out-of-range and duplicated slots
    m = rng.random(idx.shape)
    idx[m < 0.05] = -1
    idx[(m >= 0.05) & (m < 0.08)] = kv + rng.integers(0, 50)
    if topk > 3 and i % 2:
        idx[:, 1] = idx[:, 0]   # (odd cases: two-row teams then match by position)
    c.idx = idx.astype(np.int32)
    return rng, c, mla, fp8


def _kv_f64(c, fp8):
    return oracle.mla_fp8_rows_to_f64(c.k) if fp8 else c.k


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep(i):
    rng, c, mla, fp8 = _case(i)
    T, hq, topk, kv = c.num_rows, c.num_q_heads, c.topk, c.kv_len
    say(f"[sweep {i}] {'MLA' if mla else 'GQA'}{' fp8' if fp8 else ''} T={T} Hq={hq} "
        f"Hkv={c.num_kv_heads} k={topk} kv={kv}")
    q = _padded(bf16_dev(c.q), 8 * int(rng.integers(0, 3)))
    if fp8:
        k = torch.from_numpy(np.ascontiguousarray(c.k)).cuda()
    else:
        k = _padded(bf16_dev(c.k), 8 * int(rng.integers(0, 3)))
    v = None if mla else _padded(bf16_dev(c.v), 8 * int(rng.integers(0, 3)))
    idx = _padded(i32_dev(c.idx), int(rng.integers(0, 5)))
    tl = rng.integers(-2, topk + 3, T).astype(np.int32)
    kw = dict(sm_scale=c.scale, head_dim_v=c.head_dim_v if mla else None)
    kd = _kv_f64(c, fp8)
    vd = None if mla else c.v

    # per-token, with and without top-k lengths
    o, l = sa.sparse_attn_prefill(q, k, v, idx, topk_len=i32_dev(tl), **kw)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_attention(c.q, kd, vd, c.idx, num_kv_heads=c.num_kv_heads,
                                     scale=c.scale, head_dim_v=c.head_dim_v, topk_len=tl)
    check_close(o, l, ro, rl, f"sweep {i} per-token")

    # ragged: split the rows into 1-3 requests over a packed KV of their own
    R = int(rng.integers(1, 4))
    cuts = np.sort(rng.choice(np.arange(1, T), size=min(R - 1, T - 1), replace=False)) if T > 1 else []
    cu_q = np.concatenate([[0], cuts, [T]]).astype(np.int32)
    R = len(cu_q) - 1
    lens = rng.integers(1, kv + 1, R)
    cu_kv = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    src = np.concatenate([rng.integers(0, kv - ln + 1, 1) for ln in lens])   # each request's KV window
    rows = np.concatenate([np.arange(s, s + ln) for s, ln in zip(src, lens)])
    kp = c.k[rows]
    vp = None if mla else c.v[rows]
    kpd = oracle.mla_fp8_rows_to_f64(kp) if fp8 else kp
    kt = torch.from_numpy(np.ascontiguousarray(kp)).cuda() if fp8 else bf16_dev(kp)
    vt = None if mla else bf16_dev(vp)
    o, l = sa.sparse_attn_chunk_prefill(q, kt, vt, idx, i32_dev(cu_q), i64_dev(cu_kv), **kw)
    torch.cuda.synchronize()
    ro, rl = oracle.chunk_prefill(c.q, kpd, vp, c.idx, cu_q, cu_kv,
                                  num_kv_heads=c.num_kv_heads, scale=c.scale,
                                  head_dim_v=c.head_dim_v)
    check_close(o, l, ro, rl, f"sweep {i} ragged")

    # union over the whole request and over the ragged requests; when the
    # union tile is illegal (G * group > 32) the per-token path runs instead,
    # which counts duplicated indices with their multiplicity
    G = int(rng.integers(1, 9))
    o, l, st = sa.sparse_attn_prefill_union(q, k, v, idx, G, **kw)
    torch.cuda.synchronize()
    if st == sa.SA_OK:
        ro, rl = oracle.union_attention(c.q, kd, vd, *oracle.union_build(c.idx, kv, G), G,
                                        num_kv_heads=c.num_kv_heads, scale=c.scale,
                                        head_dim_v=c.head_dim_v)
    else:
        assert st == sa.SA_OK_FALLBACK and G * (hq // c.num_kv_heads) > 32
        ro, rl = oracle.sparse_attention(c.q, kd, vd, c.idx, num_kv_heads=c.num_kv_heads,
                                         scale=c.scale, head_dim_v=c.head_dim_v)
    check_close(o, l, ro, rl, f"sweep {i} union G={G} status {st}")
    o, l, st = sa.sparse_attn_chunk_prefill_union(q, kt, vt, idx, i32_dev(cu_q), i64_dev(cu_kv),
                                                  G, **kw)
    torch.cuda.synchronize()
    if st == sa.SA_OK:
        ui, ub, ul, grq = oracle.chunk_union_build(c.idx, cu_q, cu_kv, G)
        ro, rl = oracle.chunk_union_attention(c.q, kpd, vp, ui, ub, ul, grq, cu_q, cu_kv, G,
                                              num_kv_heads=c.num_kv_heads, scale=c.scale,
                                              head_dim_v=c.head_dim_v)
    else:
        ro, rl = oracle.chunk_prefill(c.q, kpd, vp, c.idx, cu_q, cu_kv,
                                      num_kv_heads=c.num_kv_heads, scale=c.scale,
                                      head_dim_v=c.head_dim_v)
    check_close(o, l, ro, rl, f"sweep {i} ragged union G={G} status {st}")
