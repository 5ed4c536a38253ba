"""Decode-pool page mark and page split (TEST INFRASTRUCTURE: oracle only).

sglang PR 32320 ("Only split touched SWA pages in FlashMLA page-split
kernel"), "Modifications": the decode pool keeps pages of src_pbs = 256
tokens; the decode kernel wants pages of 64 tokens. The mark pass sets
mask[t // src_pbs] = 1 for every valid token index t of the step (-1 is
skipped); the split pass copies source page p into destination pages
p*ratio .. p*ratio+ratio-1 (data rows and their scales), and with a mask it
skips every page whose mask byte is 0, leaving that destination stale.

Page layout (the pages name a padded destination page size without its
value; this is the reading taken): a source page is src_page_tokens token
rows of row_bytes, followed by src_page_tokens scales of scale_bytes; a
destination page is dst_page_tokens rows followed by their scales, at
dst_page_stride bytes per page. Token ids outside the pool are skipped like
-1 (the pages never write outside the mask).
"""
from __future__ import annotations

import numpy as np


def page_mark(idx: np.ndarray, num_src_pages: int, src_page_tokens: int) -> np.ndarray:
    """int8 mask [num_src_pages]: 1 iff some valid token index lies in the page."""
    mask = np.zeros(num_src_pages, dtype=np.int8)
    limit = num_src_pages * src_page_tokens
    for t in np.asarray(idx).ravel().tolist():
        if 0 <= t < limit:
            mask[t // src_page_tokens] = 1
    return mask


def page_split(src: np.ndarray, dst: np.ndarray, mask, *, src_page_tokens: int,
               dst_page_tokens: int, row_bytes: int, scale_bytes: int) -> np.ndarray:
    """Returns a copy of dst with every (masked-in) source page split.

    src uint8 [P, src_page_stride]; dst uint8 [P*ratio, dst_page_stride];
    mask int8 [P] or None (None = split every page).
    """
    ratio = src_page_tokens // dst_page_tokens
    out = dst.copy()
    src_scale0 = src_page_tokens * row_bytes
    dst_scale0 = dst_page_tokens * row_bytes
    for p in range(src.shape[0]):
        if mask is not None and mask[p] == 0:
            continue
        for s in range(ratio):
            d = p * ratio + s
            rows = slice(s * dst_page_tokens * row_bytes, (s + 1) * dst_page_tokens * row_bytes)
            out[d, :dst_scale0] = src[p, rows]
            sc = slice(src_scale0 + s * dst_page_tokens * scale_bytes,
                       src_scale0 + (s + 1) * dst_page_tokens * scale_bytes)
            out[d, dst_scale0:dst_scale0 + dst_page_tokens * scale_bytes] = src[p, sc]
    return out
