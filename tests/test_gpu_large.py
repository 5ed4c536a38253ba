"""GPU parity with KV buffers and pools past 4 GiB: every gather address is
formed in 64 bits. The buffers are filled with NaN (bf16) or 0x7F bytes
(the E4M3 NaN code) except the rows the indices reference, which hold seeded
N(0, 1) values or FP8 records; a gather from any other address, such as one
whose byte offset was cut to 32 bits, turns the row's output into NaN and
fails the check. Indices lean to the top of the buffer (byte offsets above
2^32), with some near the bottom, -1 padding and out-of-range values.

The oracle sees only the referenced rows: the indices are renumbered onto a
compact copy of those rows (in the same order, so union lists keep their
order), which leaves every row's definition unchanged."""
import numpy as np
import pytest
import torch

import gen
import oracle
import top_index_sparse_amd as sa
from tests.gpu_util import bf16_dev, check_close, i32_dev, i64_dev, say

pytestmark = pytest.mark.gpu

FOUR_GIB = 1 << 32


@pytest.fixture(autouse=True)
def _enough_memory():
    if torch.cuda.get_device_properties(0).total_memory < (40 << 30):
        pytest.skip("needs 40 GiB of device memory")
    yield
    torch.cuda.empty_cache()


def _draw(rng, rows, topk, kv):
    """Indices over [0, kv): half in the top 2^20 tokens, a quarter in the
    bottom 2^20, a quarter anywhere; then -1 and out-of-range slots."""
    hi = rng.integers(max(0, kv - (1 << 20)), kv, size=(rows, topk))
    lo = rng.integers(0, min(kv, 1 << 20), size=(rows, topk))
    anyw = rng.integers(0, kv, size=(rows, topk))
    pick = rng.random((rows, topk))
    idx = np.where(pick < 0.5, hi, np.where(pick < 0.75, lo, anyw))
    idx[pick > 0.97] = -1
    idx[(pick > 0.95) & (pick <= 0.97)] = kv + 3
    return idx.astype(np.int32)


def _renumber(idx, kv, rows):
    """idx over [0, kv) -> idx over the sorted rows `rows` (which hold every
    valid index); invalid slots stay invalid for a KV of len(rows)."""
    valid = (idx >= 0) & (idx < kv)
    out = np.where(idx < 0, -1, len(rows) + 3).astype(np.int32)
    out[valid] = np.searchsorted(rows, idx[valid])
    return out


def _scatter(buf, rows, values):
    buf[torch.from_numpy(rows.astype(np.int64)).cuda()] = values


class GQABuffers:
    """K and V [kv, 2, 256] bf16 (1 KiB per token and tensor, 4.6 GB each)."""
    kv = 4_500_000
    hkv = 2

    def __init__(self, rng, referenced):
        self.rows = np.unique(referenced)
        shape = (self.kv, self.hkv, 256)
        self.k = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        self.v = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        self.kh = gen.normal_bf16(rng, (len(self.rows), self.hkv, 256))
        self.vh = gen.normal_bf16(rng, (len(self.rows), self.hkv, 256))
        _scatter(self.k, self.rows, bf16_dev(self.kh))
        _scatter(self.v, self.rows, bf16_dev(self.vh))
        assert self.k.numel() * 2 > FOUR_GIB


def test_gqa_prefill_and_union_past_4gib():
    rng = np.random.default_rng(4242)
    T, topk, group = 40, 320, 6
    kv = GQABuffers.kv
    idx = _draw(rng, T, topk, kv)
    idx[3, :topk // 2] = idx[3, topk // 2:2 * (topk // 2)]          # duplicates
    idx[7, :] = kv - 1 - np.arange(topk)                              # the last tokens
    b = GQABuffers(rng, idx[(idx >= 0) & (idx < kv)])
    hq = b.hkv * group
    say(f"[large] GQA K/V {b.k.numel() * 2 / 1e9:.1f} GB each, T={T} Hq={hq} topk={topk}")
    q = gen.normal_bf16(rng, (T, hq, 256))
    qd, idd = bf16_dev(q), i32_dev(idx)
    ic = _renumber(idx, kv, b.rows)
    scale = 1 / 16

    o, l = sa.sparse_attn_prefill(qd, b.k, b.v, idd, sm_scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_attention(q, b.kh, b.vh, ic, num_kv_heads=b.hkv, scale=scale)
    check_close(o, l, ro, rl, "GQA per-token past 4 GiB")

    for G in (2, 4):
        o, l, st = sa.sparse_attn_prefill_union(qd, b.k, b.v, idd, G, sm_scale=scale)
        torch.cuda.synchronize()
        assert st == sa.SA_OK
        ro, rl = oracle.union_attention(q, b.kh, b.vh, *oracle.union_build(ic, len(b.rows), G), G,
                                        num_kv_heads=b.hkv, scale=scale)
        check_close(o, l, ro, rl, f"GQA union G={G} past 4 GiB")


def test_gqa_ragged_requests_past_4gib():
    """Three requests whose KV ranges start at token 0, 1000 and 4.4 M
    (byte offset 4.5e9) of the packed buffers; indices local to each."""
    rng = np.random.default_rng(4343)
    kv = GQABuffers.kv
    cu_kv = np.array([0, 1000, 4_400_000, kv], np.int64)
    cu_q = np.array([0, 9, 30, 47], np.int32)
    topk, group, hkv = 200, 6, GQABuffers.hkv
    idx = np.empty((cu_q[-1], topk), np.int32)
    for r in range(3):
        n = int(cu_kv[r + 1] - cu_kv[r])
        idx[cu_q[r]:cu_q[r + 1]] = _draw(rng, int(cu_q[r + 1] - cu_q[r]), topk, n)
    glob = []
    for r in range(3):
        n = int(cu_kv[r + 1] - cu_kv[r])
        part = idx[cu_q[r]:cu_q[r + 1]]
        glob.append(part[(part >= 0) & (part < n)].astype(np.int64) + cu_kv[r])
    b = GQABuffers(rng, np.concatenate(glob))
    # the oracle's packed KV: each request's referenced rows, renumbered
    ic = np.empty_like(idx)
    cu_c = [0]
    kc, vc = [], []
    for r in range(3):
        n = int(cu_kv[r + 1] - cu_kv[r])
        rows = np.unique(glob[r]) - cu_kv[r]
        ic[cu_q[r]:cu_q[r + 1]] = _renumber(idx[cu_q[r]:cu_q[r + 1]], n, rows)
        at = np.searchsorted(b.rows, rows + cu_kv[r])
        kc.append(b.kh[at])
        vc.append(b.vh[at])
        cu_c.append(cu_c[-1] + len(rows))
    kc, vc, cu_c = np.concatenate(kc), np.concatenate(vc), np.array(cu_c, np.int64)
    hq = hkv * group
    q = gen.normal_bf16(rng, (int(cu_q[-1]), hq, 256))
    say(f"[large] ragged GQA, request KV starts {cu_kv[:-1].tolist()}")
    qd, idd, cqd, ckd = bf16_dev(q), i32_dev(idx), i32_dev(cu_q), i64_dev(cu_kv)
    scale = 1 / 16

    o, l = sa.sparse_attn_chunk_prefill(qd, b.k, b.v, idd, cqd, ckd, sm_scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.chunk_prefill(q, kc, vc, ic, cu_q, cu_c, num_kv_heads=hkv, scale=scale)
    check_close(o, l, ro, rl, "ragged per-token past 4 GiB")

    o, l, st = sa.sparse_attn_chunk_prefill_union(qd, b.k, b.v, idd, cqd, ckd, 2, sm_scale=scale)
    torch.cuda.synchronize()
    assert st == sa.SA_OK
    ui, ub, ul, grq = oracle.chunk_union_build(ic, cu_q, cu_c, 2)
    ro, rl = oracle.chunk_union_attention(q, kc, vc, ui, ub, ul, grq, cu_q, cu_c, 2,
                                          num_kv_heads=hkv, scale=scale)
    check_close(o, l, ro, rl, "ragged union G=2 past 4 GiB")


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_mla_prefill_and_union_past_4gib(fp8):
    rng = np.random.default_rng(4444 + fp8)
    row_bytes = 656 if fp8 else 1152
    kv = FOUR_GIB // row_bytes + 600_000
    T, topk, hq = 24, 256, 8
    idx = _draw(rng, T, topk, kv)
    idx[5, :] = kv - 1 - np.arange(topk)
    rows = np.unique(idx[(idx >= 0) & (idx < kv)])
    if fp8:
        k = torch.full((kv, 1, 656), 0x7F, dtype=torch.uint8, device="cuda")
        kh = gen.mla_fp8_rows(rng, len(rows)).reshape(len(rows), 1, 656)
        _scatter(k, rows, torch.from_numpy(kh).cuda())
        kd = oracle.mla_fp8_rows_to_f64(kh)
    else:
        k = torch.full((kv, 1, 576), float("nan"), dtype=torch.bfloat16, device="cuda")
        kh = gen.normal_bf16(rng, (len(rows), 1, 576))
        _scatter(k, rows, bf16_dev(kh))
        kd = kh
    assert k.numel() * k.element_size() > FOUR_GIB
    say(f"[large] MLA {'FP8' if fp8 else 'bf16'} rows, {k.numel() * k.element_size() / 1e9:.1f} GB")
    q = gen.normal_bf16(rng, (T, hq, 576))
    qd, idd = bf16_dev(q), i32_dev(idx)
    ic = _renumber(idx, kv, rows)
    scale = 1 / 24

    o, l = sa.sparse_attn_prefill(qd, k, None, idd, sm_scale=scale, head_dim_v=512)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_attention(q, kd, None, ic, num_kv_heads=1, scale=scale, head_dim_v=512)
    check_close(o, l, ro, rl, "MLA per-token past 4 GiB")

    o, l, st = sa.sparse_attn_prefill_union(qd, k, None, idd, 2, sm_scale=scale, head_dim_v=512)
    torch.cuda.synchronize()
    assert st == sa.SA_OK
    ro, rl = oracle.union_attention(q, kd, None, *oracle.union_build(ic, len(rows), 2), 2,
                                    num_kv_heads=1, scale=scale, head_dim_v=512)
    check_close(o, l, ro, rl, "MLA union G=2 past 4 GiB")


def test_decode_chain_past_4gib():
    """Page mark, masked split and decode over a 4.7 GB source pool and a
    4.7 GB split pool; the referenced pages sit mostly at the top."""
    rng = np.random.default_rng(4545)
    P, sp, dp, rb, sb = 28_000, 256, 64, 656, 4
    ratio = sp // dp
    src_stride, dst_stride = sp * (rb + sb), dp * (rb + sb)
    pages = np.unique(np.concatenate([rng.choice(np.arange(P - 1000, P), 24, replace=False),
                                      rng.choice(P, 16, replace=False), [P - 1]]))
    B, topk = 6, 384
    tok = pages[rng.integers(0, len(pages), (B, topk))] * sp + rng.integers(0, sp, (B, topk))
    idx = tok.astype(np.int32)
    idx[1, 300:] = -1
    idx[4, 10:20] = P * sp + 7                                        # past the pool
    idx[2, :] = -1                                                    # empty request
    # host copies of the referenced source pages: random bytes, with FP8
    # records in every referenced token row
    src_h = rng.integers(0, 256, (len(pages), src_stride), dtype=np.uint8)
    valid = (idx >= 0) & (idx < P * sp)
    ref = np.unique(idx[valid]).astype(np.int64)
    pi, slot = np.searchsorted(pages, ref // sp), ref % sp
    src_h[pi[:, None], slot[:, None] * rb + np.arange(rb)[None]] = gen.mla_fp8_rows(rng, len(ref))

    src = torch.full((P, src_stride), 0x7F, dtype=torch.uint8, device="cuda")
    _scatter(src, pages, torch.from_numpy(src_h).cuda())
    dst = torch.full((P * ratio, dst_stride), 0xA5, dtype=torch.uint8, device="cuda")
    assert src.numel() > FOUR_GIB and dst.numel() > FOUR_GIB
    say(f"[large] decode chain: {P} source pages ({src.numel() / 1e9:.1f} GB), {len(pages)} touched")
    q = gen.normal_bf16(rng, (B, 16, 576))
    idd = i32_dev(idx)
    geom = dict(src_page_tokens=sp, dst_page_tokens=dp, row_bytes=rb, scale_bytes=sb)

    mask = sa.page_mark(idd, P, sp)
    sa.page_split(src, dst, mask, **geom)
    o, l = sa.sparse_attn_decode_paged(bf16_dev(q), dst, idd, dst_page_tokens=dp, sm_scale=1 / 24)
    torch.cuda.synchronize()

    want_mask = oracle.page_mark(idx, P, sp)
    assert np.array_equal(mask.cpu().numpy(), want_mask)
    assert np.array_equal(np.flatnonzero(want_mask), pages)
    split_h = oracle.page_split(src_h, np.full((len(pages) * ratio, dst_stride), 0xA5, np.uint8),
                                None, **geom)
    drows = (pages[:, None] * ratio + np.arange(ratio)[None]).ravel()
    got = dst[torch.from_numpy(drows).cuda()].cpu().numpy()
    assert np.array_equal(got, split_h), "split pages differ"
    others = np.setdiff1d(np.concatenate([rng.choice(P * ratio, 200), [P * ratio - 5]]), drows)
    assert np.all(dst[torch.from_numpy(others).cuda()].cpu().numpy() == 0xA5)

    # decode against the oracle's split, renumbered onto the touched pages
    ic = np.where(idx < 0, -1, len(pages) * sp + 3).astype(np.int32)
    ic[valid] = np.searchsorted(pages, idx[valid] // sp) * sp + idx[valid] % sp
    ro, rl = oracle.paged_decode(q, split_h, ic, page_tokens=dp, scale=1 / 24)
    check_close(o, l, ro, rl, "decode past 4 GiB")
