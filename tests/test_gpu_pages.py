"""GPU parity: decode-pool page mark and masked page split, bit-exact
against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import gen
import oracle
import top_index_sparse_amd as sa
from tests.gpu_util import config, say

pytestmark = pytest.mark.gpu


def _geom(c):
    return dict(src_page_tokens=c.src_page_tokens, dst_page_tokens=c.dst_page_tokens,
                row_bytes=c.row_bytes, scale_bytes=c.scale_bytes)


@pytest.mark.parametrize("name", ["C4decode", "C4spread"])
def test_page_mark_exact(name):
    say(f"[pages] mark {name}")
    c = config(name)
    idx = torch.from_numpy(c.idx).cuda()
    mask = torch.full((c.num_src_pages,), 7, dtype=torch.int8, device="cuda")   # stale bytes
    sa.page_mark(idx, c.num_src_pages, c.src_page_tokens, mask=mask)
    torch.cuda.synchronize()
    want = oracle.page_mark(c.idx, c.num_src_pages, c.src_page_tokens)
    assert np.array_equal(mask.cpu().numpy(), want)
    say(f"  {name}: {int(want.sum())} touched pages")


@pytest.mark.parametrize("name", ["C4decode", "C4spread"])
def test_masked_split_exact(name):
    say(f"[pages] masked split {name}")
    c = config(name)
    src = torch.from_numpy(c.src).cuda()
    dst = torch.full((c.num_src_pages * c.ratio, c.dst_page_bytes), 0xA5, dtype=torch.uint8,
                     device="cuda")
    idx = torch.from_numpy(c.idx).cuda()
    mask = sa.page_mark(idx, c.num_src_pages, c.src_page_tokens)
    sa.page_split(src, dst, mask, **_geom(c))
    torch.cuda.synchronize()
    m = oracle.page_mark(c.idx, c.num_src_pages, c.src_page_tokens)
    touched = np.flatnonzero(m)
    got = dst.cpu().numpy()
    # touched destination pages: exactly the oracle's split of those pages
    sub = oracle.page_split(c.src[touched], np.full((len(touched) * c.ratio, c.dst_page_bytes),
                                                    0xA5, np.uint8), None, **_geom(c))
    rows = (touched[:, None] * c.ratio + np.arange(c.ratio)[None]).ravel()
    assert np.array_equal(got[rows], sub)
    untouched = np.ones(got.shape[0], bool)
    untouched[rows] = False
    assert np.all(got[untouched] == 0xA5), "untouched destination pages must stay stale"


def test_full_split_exact_and_equals_masked_on_touched():
    say("[pages] full split (NULL mask) == numpy reshape; masked == full on touched pages")
    c = config("C4decode")
    src = torch.from_numpy(c.src).cuda()
    full = torch.zeros((c.num_src_pages * c.ratio, c.dst_page_bytes), dtype=torch.uint8,
                       device="cuda")
    sa.page_split(src, full, None, **_geom(c))
    torch.cuda.synchronize()
    f = full.cpu().numpy()
    rb = c.dst_page_tokens * c.row_bytes
    assert np.array_equal(f[:, :rb], c.src[:, :c.src_page_tokens * c.row_bytes].reshape(-1, rb))
    sb = c.dst_page_tokens * c.scale_bytes
    assert np.array_equal(f[:, rb:rb + sb], c.src[:, c.src_page_tokens * c.row_bytes:].reshape(-1, sb))
    dst = torch.full_like(full, 0xA5)
    mask = sa.page_mark(torch.from_numpy(c.idx).cuda(), c.num_src_pages, c.src_page_tokens)
    sa.page_split(src, dst, mask, **_geom(c))
    torch.cuda.synchronize()
    m = mask.cpu().numpy().astype(bool)
    rows = (np.flatnonzero(m)[:, None] * c.ratio + np.arange(c.ratio)[None]).ravel()
    assert np.array_equal(dst.cpu().numpy()[rows], f[rows])


def test_odd_geometry_byte_path_and_padded_pages():
    say("[pages] odd geometry (byte copies), padded destination stride, invalid ids")
    rng = np.random.default_rng(4)
    P, stok, dtok, rb, sb = 37, 12, 4, 5, 3
    ratio = stok // dtok
    src_np = rng.integers(0, 256, size=(P, stok * (rb + sb) + 9), dtype=np.uint8)
    idx_np = rng.integers(-3, P * stok + 40, size=(3, 50)).astype(np.int32)
    src = torch.from_numpy(src_np).cuda()
    dstride = dtok * (rb + sb) + 7
    dst = torch.full((P * ratio, dstride), 0xA5, dtype=torch.uint8, device="cuda")
    mask = sa.page_mark(torch.from_numpy(idx_np).cuda(), P, stok)
    sa.page_split(src, dst, mask, src_page_tokens=stok, dst_page_tokens=dtok, row_bytes=rb,
                  scale_bytes=sb)
    torch.cuda.synchronize()
    m = oracle.page_mark(idx_np, P, stok)
    assert np.array_equal(mask.cpu().numpy(), m)
    want = oracle.page_split(src_np[:, :stok * (rb + sb)], np.full((P * ratio, dstride), 0xA5,
                                                                    np.uint8), m,
                             src_page_tokens=stok, dst_page_tokens=dtok, row_bytes=rb,
                             scale_bytes=sb)
    assert np.array_equal(dst.cpu().numpy(), want)


def test_mark_reuses_mask_and_empty_index_list():
    c = config("C4decode")
    mask = torch.ones((c.num_src_pages,), dtype=torch.int8, device="cuda")
    empty = torch.empty((0,), dtype=torch.int32, device="cuda")
    sa.page_mark(empty, c.num_src_pages, c.src_page_tokens, mask=mask)
    torch.cuda.synchronize()
    assert int(mask.abs().sum()) == 0
