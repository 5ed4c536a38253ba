"""CPU checks of the every-row comparison machinery (tests/oracle_pool.py):
each task kind, fed the oracle's own results, passes on every row, and a
single perturbed element, LSE or index is caught and located."""
import numpy as np
import pytest

import gen
import oracle
from tests import oracle_pool


def _case(seed=3, T=37, kv=900, Hq=6, Hkv=1, topk=100):
    return gen.make_attn_case("pool", seed=seed, num_rows=T, kv_len=kv, first_pos=kv - T,
                              num_q_heads=Hq, num_kv_heads=Hkv, head_dim_qk=256,
                              head_dim_v=256, topk=topk)


def _params(c, **kw):
    p = {"num_kv_heads": c.num_kv_heads, "scale": c.scale, "kv_len": c.kv_len,
         "head_dim_v": c.head_dim_v, "has_v": c.v is not None}
    p.update(kw)
    return p


def test_chunks_cover_rows_on_group_boundaries():
    for T, step in [(37, 1), (37, 4), (8192, 2), (5, 8), (1, 1)]:
        ch = oracle_pool.row_chunks(T, step, pieces=7)
        assert ch[0][0] == 0 and ch[-1][1] == T
        assert all(a[1] == b[0] for a, b in zip(ch, ch[1:]))
        assert all(lo % step == 0 for lo, _ in ch)
    cu_q = np.array([0, 5, 5, 12, 40], dtype=np.int32)
    cu_kv = np.array([0, 100, 150, 300, 700], dtype=np.int64)
    ch = oracle_pool.ragged_chunks(cu_q, cu_kv, 2, pieces=6)
    rows = np.concatenate([np.arange(lo, hi) for lo, hi, _, _ in ch])
    assert np.array_equal(rows, np.arange(40))
    for lo, hi, kv0, kv1 in ch:
        r = np.searchsorted(cu_q, lo, side="right") - 1
        assert (lo - cu_q[r]) % 2 == 0 and hi <= cu_q[r + 1]
        assert (kv0, kv1) == (cu_kv[r], cu_kv[r + 1])


def test_attn_task_passes_and_catches_one_element():
    c = _case()
    ro, rl = oracle.sparse_attention(c.q, c.k, c.v, c.idx, num_kv_heads=1, scale=c.scale,
                                     kv_len=c.kv_len)
    a = {"q": c.q, "k": c.k, "v": c.v, "idx": c.idx, "out": ro.astype(np.float32),
         "lse": rl.astype(np.float32)}
    chunks = oracle_pool.row_chunks(c.num_rows, pieces=5)
    m = oracle_pool.run("attn", a, _params(c), chunks)
    assert m["rows"] == c.num_rows
    oracle_pool.assert_ok(m, "exact")
    bad = ro.astype(np.float32).copy()
    bad[29, 4, 200] += 0.05
    a["out"] = bad
    m = oracle_pool.run("attn", a, _params(c), chunks)
    assert m["worst"] == (29, 4, 200)
    with pytest.raises(AssertionError):
        oracle_pool.assert_ok(m, "perturbed O")
    a["out"] = ro.astype(np.float32)
    badl = rl.astype(np.float32).copy()
    badl[3, 1] += 1e-4
    a["lse"] = badl
    with pytest.raises(AssertionError):
        oracle_pool.assert_ok(oracle_pool.run("attn", a, _params(c), chunks), "perturbed LSE")


@pytest.mark.parametrize("G", [2, 3])
def test_union_task(G):
    c = _case(seed=4, T=23)
    ui, ub, ul = oracle.union_build(c.idx, c.kv_len, G)
    ro, rl = oracle.union_attention(c.q, c.k, c.v, ui, ub, ul, G, num_kv_heads=1, scale=c.scale)
    a = {"q": c.q, "k": c.k, "v": c.v, "idx": c.idx, "out": ro.astype(np.float32),
         "lse": rl.astype(np.float32)}
    m = oracle_pool.run("union", a, _params(c, G=G), oracle_pool.row_chunks(c.num_rows, G, 4))
    oracle_pool.assert_ok(m, f"union G={G}")
    assert m["rows"] == c.num_rows


def test_chunk_and_chunk_union_tasks():
    c = gen.make_ragged_case("pool", seed=5, num_reqs=4, qlen_range=(3, 17),
                             ctx_range=(200, 600), num_q_heads=6, num_kv_heads=1, head_dim=256,
                             topk=64)
    ro, rl = oracle.chunk_prefill(c.q, c.k, c.v, c.idx, c.cu_seqlens_q, c.cu_seqlens_kv,
                                  num_kv_heads=1, scale=c.scale)
    a = {"q": c.q, "k": c.k, "v": c.v, "idx": c.idx, "cu_q": c.cu_seqlens_q,
         "cu_kv": c.cu_seqlens_kv, "out": ro.astype(np.float32), "lse": rl.astype(np.float32)}
    oracle_pool.assert_ok(oracle_pool.run("chunk", a, _params(c),
                                          oracle_pool.row_chunks(c.num_rows, 1, 3)), "chunk")
    ui, ub, ul, own = oracle.chunk_union_build(c.idx, c.cu_seqlens_q, c.cu_seqlens_kv, 2)
    uo, ulse = oracle.chunk_union_attention(c.q, c.k, c.v, ui, ub, ul, own, c.cu_seqlens_q,
                                            c.cu_seqlens_kv, 2, num_kv_heads=1, scale=c.scale)
    a.update(out=uo.astype(np.float32), lse=ulse.astype(np.float32))
    m = oracle_pool.run("chunk_union", a, _params(c, G=2),
                        oracle_pool.ragged_chunks(c.cu_seqlens_q, c.cu_seqlens_kv, 2, 5))
    oracle_pool.assert_ok(m, "chunk union")
    assert m["rows"] == c.num_rows


def test_topk_task_chain():
    tc = gen.make_topk_case("pool", seed=6, num_rows=20, kv_len=700, first_pos=680, k=64)
    c = _case(seed=7, T=20, kv=700, topk=64)
    sel = oracle.topk_select(tc.scores, tc.k, tc.row_len)
    ro, rl = oracle.sparse_attention(c.q, c.k, c.v, sel, num_kv_heads=1, scale=c.scale,
                                     kv_len=c.kv_len)
    a = {"q": c.q, "k": c.k, "v": c.v, "scores": tc.scores, "row_len": tc.row_len,
         "gpu_idx": sel, "out": ro.astype(np.float32), "lse": rl.astype(np.float32)}
    m = oracle_pool.run("topk", a, _params(c, k=tc.k, attn_G=0),
                        oracle_pool.row_chunks(20, 1, 3))
    oracle_pool.assert_ok(m, "topk chain")
    assert m["idx_mismatch_rows"] == 0
    bad = sel.copy()
    bad[11, 5] += 1
    a["gpu_idx"] = bad
    m = oracle_pool.run("topk", a, _params(c, k=tc.k, attn_G=0), oracle_pool.row_chunks(20, 1, 3))
    assert m["idx_mismatch_rows"] == 1
