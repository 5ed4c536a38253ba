"""GPU: guard-banded outputs and workspaces for every entry point. Each
output and each workspace is a view of exactly its size inside one larger
allocation whose 64 KiB bands on both sides (and the bytes up to the next
256-byte boundary) hold a sentinel. After the call the bands must be
unchanged, and the outputs must equal those of the same call into plain
allocations (the kernels are deterministic). The shapes are small and
ragged: row counts that are not multiples of a team, a group or a block,
and workspaces at exactly the size the workspace query returns."""
import numpy as np
import pytest
import torch

import gen
import top_index_sparse_amd as sa
from tests.gpu_util import bf16_dev, i32_dev, i64_dev, say

pytestmark = pytest.mark.gpu

BAND = 1 << 16
FILL = 0x5A


class Banded:
    """nbytes of device memory between two sentinel bands."""

    def __init__(self, nbytes):
        self.n = int(nbytes)
        inner = (self.n + 255) // 256 * 256
        self.buf = torch.full((2 * BAND + inner,), FILL, dtype=torch.uint8, device="cuda")

    def bytes(self):
        return self.buf[BAND:BAND + self.n]

    def view(self, dtype, shape):
        return self.bytes().view(dtype).view(shape)

    def intact(self):
        lo = self.buf[:BAND]
        hi = self.buf[BAND + self.n:]
        return bool((lo == FILL).all()) and bool((hi == FILL).all())


def _banded_like(shape, dtype):
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    b = Banded(n)
    return b, b.view(dtype, shape)


def _check(bands, pairs, what):
    for i, b in enumerate(bands):
        assert b.intact(), f"{what}: a write past buffer {i}'s ends"
    for got, want in pairs:
        assert torch.equal(got, want), f"{what}: banded and plain outputs differ"


def _gqa(seed, T=37, topk=150, kv=400, hq=6, hkv=1):
    return gen.make_attn_case("guard", seed=seed, num_rows=T, kv_len=kv, first_pos=kv - T,
                              num_q_heads=hq, num_kv_heads=hkv, head_dim_qk=256, head_dim_v=256,
                              topk=topk, walk=False)


def _mla_fp8(seed, T=29, topk=130, kv=300, hq=8):
    return gen.make_attn_case("guard", seed=seed, num_rows=T, kv_len=kv, first_pos=kv - T,
                              num_q_heads=hq, num_kv_heads=1, head_dim_qk=576, head_dim_v=512,
                              topk=topk, v_in_k=True, walk=False, kv_fp8=True)


def _dev(c, fp8=False):
    k = torch.from_numpy(np.ascontiguousarray(c.k)).cuda() if fp8 else bf16_dev(c.k)
    v = None if c.v is None else bf16_dev(c.v)
    return bf16_dev(c.q), k, v, i32_dev(c.idx)


@pytest.mark.parametrize("mla", [False, True], ids=["gqa", "mla_fp8"])
def test_prefill_and_union_guarded(mla):
    c = _mla_fp8(11) if mla else _gqa(10, hq=12, hkv=2)
    q, k, v, idx = _dev(c, fp8=mla)
    T, hq, dv = c.num_rows, c.num_q_heads, c.head_dim_v
    kw = dict(sm_scale=c.scale, head_dim_v=dv if mla else None)
    say(f"[guard] prefill {'MLA FP8' if mla else 'GQA'} T={T} Hq={hq}")
    ob, out = _banded_like((T, hq, dv), torch.float32)
    lb, lse = _banded_like((T, hq), torch.float32)
    sa.sparse_attn_prefill(q, k, v, idx, out=out, lse=lse, **kw)
    po, pl = sa.sparse_attn_prefill(q, k, v, idx, **kw)
    torch.cuda.synchronize()
    _check([ob, lb], [(out, po), (lse, pl)], "prefill")
    for G in (2, 3):
        ws = Banded(sa.sparse_attn_union_workspace_bytes(T, c.topk, G))
        ob, out = _banded_like((T, hq, dv), torch.float32)
        lb, lse = _banded_like((T, hq), torch.float32)
        _, _, st = sa.sparse_attn_prefill_union(q, k, v, idx, G, ws=ws.bytes(), out=out, lse=lse,
                                                **kw)
        po, pl, st2 = sa.sparse_attn_prefill_union(q, k, v, idx, G, **kw)
        torch.cuda.synchronize()
        assert st == st2
        _check([ws, ob, lb], [(out, po), (lse, pl)], f"prefill union G={G} status {st}")


@pytest.mark.parametrize("kv", [700, 400_000], ids=["bit_planes", "sorted_lists"])
def test_union_build_guarded(kv):
    rng = np.random.default_rng(kv)
    T, topk, G = 45, 180, 2
    idx = rng.integers(-2, kv + 5, size=(T, topk)).astype(np.int32)
    idx[4, :90] = idx[4, 90:]
    say(f"[guard] union build T={T} topk={topk} G={G} kv={kv}")
    ng = (T + G - 1) // G
    ib, ui = _banded_like((ng, G * topk), torch.int32)
    bb, ubits = _banded_like((ng, G * topk), torch.uint8)
    nb, ulen = _banded_like((ng,), torch.int32)
    ws = Banded(sa.sparse_attn_union_workspace_bytes(T, topk, G))
    d = i32_dev(idx)
    sa.sparse_attn_union_build(d, kv, G, union_idx=ui, union_bits=ubits, union_len=ulen,
                               ws=ws.bytes())
    pi, pb, pn = sa.sparse_attn_union_build(d, kv, G)
    torch.cuda.synchronize()
    assert torch.equal(ulen, pn)
    for g in range(ng):   # entries past a group's length are not part of the output
        n = int(pn[g])
        assert torch.equal(ui[g, :n], pi[g, :n]) and torch.equal(ubits[g, :n], pb[g, :n])
    _check([ib, bb, nb, ws], [], "union build")


def test_chunk_prefill_and_union_guarded():
    c = gen.make_ragged_case("guard", seed=12, num_reqs=4, qlen_range=(3, 30),
                             ctx_range=(40, 300), num_q_heads=6, num_kv_heads=1, head_dim=256,
                             topk=96)
    q, k, v, idx = _dev(c)
    cq, ck = i32_dev(c.cu_seqlens_q), i64_dev(c.cu_seqlens_kv)
    T = c.num_rows
    say(f"[guard] chunk prefill T={T}, {len(c.cu_seqlens_q) - 1} requests")
    ob, out = _banded_like((T, 6, 256), torch.float32)
    lb, lse = _banded_like((T, 6), torch.float32)
    sa.sparse_attn_chunk_prefill(q, k, v, idx, cq, ck, sm_scale=c.scale, out=out, lse=lse)
    po, pl = sa.sparse_attn_chunk_prefill(q, k, v, idx, cq, ck, sm_scale=c.scale)
    torch.cuda.synchronize()
    _check([ob, lb], [(out, po), (lse, pl)], "chunk prefill")
    R = len(c.cu_seqlens_q) - 1
    ws = Banded(sa.sparse_attn_chunk_union_workspace_bytes(T, R, c.topk, 2))
    ob, out = _banded_like((T, 6, 256), torch.float32)
    lb, lse = _banded_like((T, 6), torch.float32)
    sa.sparse_attn_chunk_prefill_union(q, k, v, idx, cq, ck, 2, sm_scale=c.scale, ws=ws.bytes(),
                                       out=out, lse=lse)
    po, pl, _ = sa.sparse_attn_chunk_prefill_union(q, k, v, idx, cq, ck, 2, sm_scale=c.scale)
    torch.cuda.synchronize()
    _check([ws, ob, lb], [(out, po), (lse, pl)], "chunk prefill union")


def test_pages_and_decode_guarded():
    c = gen.make_page_case("guard", seed=13, num_src_pages=35, batch=5, topk=200, window=90,
                           num_q_heads=12)
    geom = dict(src_page_tokens=c.src_page_tokens, dst_page_tokens=c.dst_page_tokens,
                row_bytes=c.row_bytes, scale_bytes=c.scale_bytes)
    P, ratio = c.num_src_pages, c.ratio
    say(f"[guard] page mark / split / decode, {P} source pages")
    idx = i32_dev(c.idx)
    mb, mask = _banded_like((P,), torch.int8)
    sa.page_mark(idx, P, c.src_page_tokens, mask=mask)
    pm = sa.page_mark(idx, P, c.src_page_tokens)
    src = torch.from_numpy(c.src).cuda()
    results = []
    for m in (mask, None):
        db, dst = _banded_like((P * ratio, c.dst_page_bytes), torch.uint8)
        dst.fill_(0xA5)
        sa.page_split(src, dst, m, **geom)
        plain = torch.full((P * ratio, c.dst_page_bytes), 0xA5, dtype=torch.uint8, device="cuda")
        sa.page_split(src, plain, m, **geom)
        results.append((db, dst, plain))
    torch.cuda.synchronize()
    _check([mb], [(mask, pm)], "page mark")
    for db, dst, plain in results:
        _check([db], [(dst, plain)], "page split")

    pool = results[0][2]
    B, hq = c.idx.shape[0], 12
    q = bf16_dev(c.q)
    ws = Banded(sa.sparse_attn_decode_workspace_bytes(B, hq, c.idx.shape[1]))
    ob, out = _banded_like((B, hq, 512), torch.float32)
    lb, lse = _banded_like((B, hq), torch.float32)
    sa.sparse_attn_decode_paged(q, pool, idx, dst_page_tokens=c.dst_page_tokens, sm_scale=1 / 24,
                                ws=ws.bytes(), out=out, lse=lse)
    po, pl = sa.sparse_attn_decode_paged(q, pool, idx, dst_page_tokens=c.dst_page_tokens,
                                         sm_scale=1 / 24)
    torch.cuda.synchronize()
    _check([ws, ob, lb], [(out, po), (lse, pl)], "decode")


def test_indexer_topk_guarded():
    rng = np.random.default_rng(14)
    T, kv, k = 19, 3001, 257
    scores = torch.from_numpy(rng.standard_normal((T, kv)).astype(np.float32)).cuda()
    row_len = i32_dev(rng.integers(0, kv + 10, T).astype(np.int32))
    say(f"[guard] indexer top-k T={T} kv={kv} k={k}")
    ob, out = _banded_like((T, k), torch.int32)
    sa.indexer_topk(scores, k, row_len=row_len, out=out)
    plain = sa.indexer_topk(scores, k, row_len=row_len)
    torch.cuda.synchronize()
    _check([ob], [(out, plain)], "indexer top-k")
