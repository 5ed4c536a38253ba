"""GPU parity: sparse MLA decode over the split pool (656-byte FP8 records in
pages of dst_page_tokens) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import gen
import oracle
import top_index_sparse_amd as sa
from tests.gpu_util import bf16_dev, check_close, config, i32_dev, say

pytestmark = pytest.mark.gpu


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _pool(rng, pages, ptok, stride):
    """Pages of ptok FP8 records, then random per-token words and padding."""
    pool = rng.integers(0, 256, size=(pages, stride), dtype=np.uint8)
    pool[:, :ptok * 656] = gen.mla_fp8_rows(rng, pages * ptok).reshape(pages, ptok * 656)
    return pool


def _indices(rng, B, topk, tokens):
    idx = rng.integers(-3, tokens + 40, size=(B, topk)).astype(np.int32)   # -1s and past the pool
    h = topk // 2
    idx[0, :h] = idx[0, h:2 * h]                                           # duplicates
    if B > 2:
        idx[2] = -1                                                        # empty request
    return idx


@pytest.mark.parametrize("B,Hq,topk,ptok", [(1, 8, 2048, 64), (3, 16, 100, 64), (37, 3, 256, 64),
                                            (5, 1, 16, 16), (64, 8, 300, 128), (300, 8, 33, 64),
                                            (4, 32, 512, 64), (7, 17, 200, 64), (2, 24, 2048, 64)])
def test_decode_pool(B, Hq, topk, ptok):
    say(f"[decode] batch {B}, {Hq} heads, topk {topk}, {ptok}-token pages, padded stride")
    rng = np.random.default_rng(B * 1000 + Hq * 10 + topk)
    pages = max(4, 3000 // ptok)
    pool = _pool(rng, pages, ptok, ptok * 660 + 256)
    q = gen.normal_bf16(rng, (B, Hq, 576))
    idx = _indices(rng, B, topk, pages * ptok)
    scale = 1.0 / 24
    out, lse = sa.sparse_attn_decode_paged(bf16_dev(q), _u8(pool), i32_dev(idx),
                                           dst_page_tokens=ptok, sm_scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.paged_decode(q, pool, idx, page_tokens=ptok, scale=scale)
    e, el = check_close(out, lse, ro, rl, f"decode B={B} Hq={Hq} topk={topk}")
    say(f"  max abs err O {e:.2e} LSE {el:.2e}")


def test_decode_topk_len_and_stale_workspace():
    say("[decode] topk_len (0, negative, partial, past topk); a reused workspace")
    rng = np.random.default_rng(91)
    pages, ptok, B, topk = 40, 64, 9, 200
    pool = _pool(rng, pages, ptok, ptok * 660)
    q = gen.normal_bf16(rng, (B, 8, 576))
    tl = np.array([0, -5, 1, 16, 17, 100, 200, 250, 199], np.int32)
    scale = 0.05
    # first call: every slot valid, so every range writes its partial O
    full = rng.integers(0, pages * ptok, size=(B, topk)).astype(np.int32)
    ws = torch.empty(sa.sparse_attn_decode_workspace_bytes(B, 8, topk), dtype=torch.uint8,
                     device="cuda")
    qd, pd = bf16_dev(q), _u8(pool)
    sa.sparse_attn_decode_paged(qd, pd, i32_dev(full), sm_scale=scale, ws=ws)
    # second call on the same workspace: most ranges empty under topk_len
    out, lse = sa.sparse_attn_decode_paged(qd, pd, i32_dev(full), sm_scale=scale, ws=ws,
                                           topk_len=i32_dev(tl))
    torch.cuda.synchronize()
    ro, rl = oracle.paged_decode(q, pool, full, page_tokens=ptok, scale=scale, topk_len=tl)
    check_close(out, lse, ro, rl, "decode topk_len")
    assert np.all(np.isneginf(lse[:2].cpu().numpy())) and torch.all(out[:2] == 0)


@pytest.mark.parametrize("name", ["C4decode", "C4spread"])
def test_decode_after_mark_and_split(name):
    say(f"[decode] {name}: page mark, masked split, decode; oracle on its own split")
    c = config(name)
    geom = dict(src_page_tokens=c.src_page_tokens, dst_page_tokens=c.dst_page_tokens,
                row_bytes=c.row_bytes, scale_bytes=c.scale_bytes)
    P = c.num_src_pages
    src, idx = _u8(c.src), i32_dev(c.idx)
    dst = torch.full((P * c.ratio, c.dst_page_bytes), 0xA5, dtype=torch.uint8, device="cuda")
    mask = sa.page_mark(idx, P, c.src_page_tokens)
    sa.page_split(src, dst, mask, **geom)
    out, lse = sa.sparse_attn_decode_paged(bf16_dev(c.q), dst, idx,
                                           dst_page_tokens=c.dst_page_tokens,
                                           scale_bytes=c.scale_bytes, sm_scale=c.scale)
    torch.cuda.synchronize()
    m = oracle.page_mark(c.idx, P, c.src_page_tokens)
    dst_ref = oracle.page_split(c.src, np.full((P * c.ratio, c.dst_page_bytes), 0xA5, np.uint8),
                                m, **geom)
    ro, rl = oracle.paged_decode(c.q, dst_ref, c.idx, page_tokens=c.dst_page_tokens,
                                 scale=c.scale)
    e, el = check_close(out, lse, ro, rl, f"{name} decode")
    say(f"  {name}: {int(m.sum())} touched pages; max abs err O {e:.2e} LSE {el:.2e}")


@pytest.mark.parametrize("i", range(24))
def test_decode_sweep(i):
    """Seeded random decode cases: batch, 1-32 heads, top-k, page size, pool
    stride, top-k lengths, -1, out-of-range and duplicated slots."""
    rng = np.random.default_rng(5000 + i)
    B = int(rng.integers(1, 70))
    Hq = int(rng.integers(1, 33))
    topk = int(rng.integers(1, 1200))
    ptok = int(rng.choice([16, 32, 64, 128]))
    pages = int(rng.integers(1, 5000 // ptok + 2))
    stride = ptok * 660 + 16 * int(rng.integers(0, 9))
    say(f"[decode sweep {i}] B={B} Hq={Hq} topk={topk} ptok={ptok} pages={pages} stride={stride}")
    pool = _pool(rng, pages, ptok, stride)
    q = gen.normal_bf16(rng, (B, Hq, 576))
    idx = rng.integers(0, pages * ptok, size=(B, topk)).astype(np.int32)
    m = rng.random(idx.shape)
    idx[m < 0.2] = -1
    idx[(m >= 0.2) & (m < 0.23)] = pages * ptok + int(rng.integers(0, 99))
    if topk > 2:
        idx[:, 1] = idx[:, 0]
    tl = rng.integers(-3, topk + 5, B).astype(np.int32) if rng.random() < 0.5 else None
    scale = float(rng.uniform(0.02, 0.08))
    out, lse = sa.sparse_attn_decode_paged(bf16_dev(q), _u8(pool), i32_dev(idx),
                                           dst_page_tokens=ptok, sm_scale=scale,
                                           topk_len=None if tl is None else i32_dev(tl))
    torch.cuda.synchronize()
    ro, rl = oracle.paged_decode(q, pool, idx, page_tokens=ptok, scale=scale, topk_len=tl)
    check_close(out, lse, ro, rl, f"decode sweep {i}")
