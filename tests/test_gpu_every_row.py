"""GPU parity on every row of every full-size workload.

Each test runs one entry point (or one chain of them) through the C ABI on a
full-size seeded workload, then evaluates the fp64 oracle over all of its
rows in worker processes (tests/oracle_pool.py) and compares element by
element: |O_gpu - O_ref| <= 2e-2 + 1e-2 |O_ref| and |LSE_gpu - LSE_ref| <=
1e-5 for every (row, head), and bit-exact index rows where a top-k is part
of the chain. The indexer chain compares the GPU's top-k -> attention with
the oracle's top-k -> attention, so no GPU output feeds the oracle.
"""
import numpy as np
import pytest
import torch

import gen
import top_index_sparse_amd as sa
from tests import oracle_pool
from tests.gpu_util import bf16_dev, config, i32_dev, i64_dev, say

pytestmark = pytest.mark.gpu


def _host(out, lse):
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.float().cpu().numpy()


def _inputs(c, idx=None):
    a = {"q": c.q, "k": c.k, "idx": c.idx if idx is None else idx}
    if c.v is not None:
        a["v"] = c.v
    if c.cu_seqlens_q is not None:
        a["cu_q"] = c.cu_seqlens_q
        a["cu_kv"] = c.cu_seqlens_kv
    return a


def _params(c, **kw):
    p = {"num_kv_heads": c.num_kv_heads, "scale": c.scale, "kv_len": c.kv_len,
         "head_dim_v": c.head_dim_v, "has_v": c.v is not None}
    p.update(kw)
    return p


def _dev(c, idx=None):
    k = (torch.from_numpy(np.ascontiguousarray(c.k)).cuda() if c.k.dtype == np.uint8
         else bf16_dev(c.k))
    return (bf16_dev(c.q), k, None if c.v is None else bf16_dev(c.v),
            i32_dev(c.idx if idx is None else idx))


def _report(m, what):
    say(f"  {what}: {m['rows']} rows, max abs err O {m.get('max_abs', 0):.2e}, "
        f"LSE {m.get('lse_max', 0):.2e}"
        + (f", index rows differing {m['idx_mismatch_rows']}" if "idx_mismatch_rows" in m else ""))
    oracle_pool.assert_ok(m, what)


def _per_token(c, q, k, v, idx, chunk):
    if chunk:
        cu_q = torch.tensor([0, c.num_rows], dtype=torch.int32, device="cuda")
        cu_kv = torch.tensor([0, c.kv_len], dtype=torch.int64, device="cuda")
        return sa.sparse_attn_chunk_prefill(q, k, v, idx, cu_q, cu_kv, total_q=c.num_rows,
                                            sm_scale=c.scale, head_dim_v=c.head_dim_v)
    return sa.sparse_attn_prefill(q, k, v, idx, sm_scale=c.scale, kv_len=c.kv_len,
                                  head_dim_v=c.head_dim_v)


@pytest.mark.parametrize("name,chunk", [("C1", True), ("C1", False), ("C2", False),
                                        ("C3", False), ("C3fp8", False)])
def test_per_token_every_row(name, chunk):
    entry = "chunk_prefill" if chunk else "prefill"
    say(f"[every row] {name} per-token through sparse_attn_{entry}")
    c = config(name)
    q, k, v, idx = _dev(c)
    o, l = _host(*_per_token(c, q, k, v, idx, chunk))
    a = _inputs(c)
    a.update(out=o, lse=l)
    m = oracle_pool.run("attn", a, _params(c), oracle_pool.row_chunks(c.num_rows))
    _report(m, f"{name} per-token ({entry})")


@pytest.mark.parametrize("name,chunk", [("C1", True), ("C3", False), ("C3fp8", False)])
def test_shuffled_slots_every_row(name, chunk):
    say(f"[every row] {name} with every row's slot order shuffled (membership teams)")
    c = config(name)
    sidx = gen.shuffle_slots(c.idx, 1)
    q, k, v, idx = _dev(c, sidx)
    o, l = _host(*_per_token(c, q, k, v, idx, chunk))
    a = _inputs(c, sidx)
    a.update(out=o, lse=l)
    m = oracle_pool.run("attn", a, _params(c), oracle_pool.row_chunks(c.num_rows))
    _report(m, f"{name} shuffled per-token")


@pytest.mark.parametrize("name,G", [("C1", 2), ("C3", 2), ("C3", 4), ("C3fp8", 2), ("C3fp8", 4),
                                    ("C3tail", 4)])
def test_union_every_row(name, G):
    say(f"[every row] {name} union G={G} through sparse_attn_prefill_union")
    c = config(name)
    q, k, v, idx = _dev(c)
    o, l, st = sa.sparse_attn_prefill_union(q, k, v, idx, G, sm_scale=c.scale,
                                            kv_len=c.kv_len, head_dim_v=c.head_dim_v)
    assert st == sa.SA_OK
    o, l = _host(o, l)
    a = _inputs(c)
    a.update(out=o, lse=l)
    m = oracle_pool.run("union", a, _params(c, G=G), oracle_pool.row_chunks(c.num_rows, G))
    _report(m, f"{name} union G={G}")


def test_c4_ragged_every_row():
    say("[every row] C4 ragged chunk prefill, per-token and union G=2")
    c = config("C4")
    q, k, v, idx = _dev(c)
    cu_q, cu_kv = i32_dev(c.cu_seqlens_q), i64_dev(c.cu_seqlens_kv)
    o, l = _host(*sa.sparse_attn_chunk_prefill(q, k, v, idx, cu_q, cu_kv, total_q=c.num_rows,
                                               sm_scale=c.scale))
    a = _inputs(c)
    a.update(out=o, lse=l)
    m = oracle_pool.run("chunk", a, _params(c), oracle_pool.row_chunks(c.num_rows))
    _report(m, "C4 per-token")
    uo, ul, st = sa.sparse_attn_chunk_prefill_union(q, k, v, idx, cu_q, cu_kv, 2,
                                                    total_q=c.num_rows, sm_scale=c.scale)
    assert st == sa.SA_OK
    o, l = _host(uo, ul)
    a.update(out=o, lse=l)
    m = oracle_pool.run("chunk_union", a, _params(c, G=2),
                        oracle_pool.ragged_chunks(c.cu_seqlens_q, c.cu_seqlens_kv, 2))
    _report(m, "C4 union G=2")


@pytest.mark.parametrize("mode", ["per_token", "union2"])
def test_c1_indexer_chain_every_row(mode):
    say(f"[every row] C1topk scores -> indexer_topk -> attention ({mode}) on C1's Q/K/V")
    c = config("C1")
    tc = config("C1topk")
    q, k, v, _ = _dev(c)
    sc = torch.from_numpy(tc.scores).cuda()
    rl = torch.from_numpy(tc.row_len).cuda()
    tidx = sa.indexer_topk(sc, tc.k, row_len=rl)
    if mode == "per_token":
        o, l = _per_token(c, q, k, v, tidx, True)
        G = 0
    else:
        o, l, st = sa.sparse_attn_prefill_union(q, k, v, tidx, 2, sm_scale=c.scale,
                                                kv_len=c.kv_len)
        assert st == sa.SA_OK
        G = 2
    o, l = _host(o, l)
    gidx = tidx.cpu().numpy()
    del sc
    a = {"q": c.q, "k": c.k, "v": c.v, "scores": tc.scores, "row_len": tc.row_len,
         "gpu_idx": gidx, "out": o, "lse": l}
    m = oracle_pool.run("topk", a, _params(c, k=tc.k, attn_G=G),
                        oracle_pool.row_chunks(c.num_rows, max(G, 1)))
    _report(m, f"C1topk chain ({mode})")
