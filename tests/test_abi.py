"""The C-ABI library: loads without a GPU, exports every symbol the header
declares, and its host-side validation returns the documented status codes
(no device is touched by any call here)."""
import ctypes
import math
import os
import re

import pytest

import top_index_sparse_amd as sa

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "sparse_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("sparse_attn_prefill", "sparse_attn_chunk_prefill", "sparse_attn_prefill_union",
                 "sparse_attn_union_build", "sparse_attn_union_workspace_bytes", "page_mark",
                 "page_split", "sparse_attn_decode_paged", "sparse_attn_decode_workspace_bytes",
                 "sparse_attn_decode_paged_noalloc", "sparse_attn_fp8_records_to_bf16",
                 "indexer_topk",
                 "sa_validate_attn", "sa_last_error", "sa_call_count"):
        assert want in names


def test_library_exports_every_declared_symbol():
    handle = ctypes.CDLL(sa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(handle, name), name
    assert sa.lib() is not None


def _desc(**kw):
    d = dict(num_q_heads=6, num_kv_heads=1, head_dim_qk=256, head_dim_v=256, topk=2051,
             v_in_k=0, kv_dtype=sa.SA_DTYPE_BF16, sm_scale=1 / 16, q_row_stride=6 * 256,
             kv_row_stride=256, v_row_stride=256, idx_row_stride=2051, out_row_stride=6 * 256)
    d.update(kw)
    return sa.AttnDesc(**d)


def _mla(**kw):
    d = dict(num_q_heads=8, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, topk=2048,
             v_in_k=1, q_row_stride=8 * 576, kv_row_stride=576, v_row_stride=576,
             idx_row_stride=2048, out_row_stride=8 * 512)
    d.update(kw)
    return _desc(**d)


def test_validate_ok_shapes():
    assert sa.sa_validate_attn(_desc()) == sa.SA_OK
    assert sa.sa_validate_attn(_desc(num_q_heads=24, num_kv_heads=2, q_row_stride=24 * 256,
                                     kv_row_stride=512, v_row_stride=512,
                                     out_row_stride=24 * 256)) == sa.SA_OK
    assert sa.sa_validate_attn(_mla()) == sa.SA_OK
    assert sa.sa_validate_attn(_mla(), 2) == sa.SA_OK
    assert sa.sa_validate_attn(_mla(), 4) == sa.SA_OK


@pytest.mark.parametrize("kw,code", [
    (dict(kv_dtype=sa.SA_DTYPE_FP8_E4M3), -3),          # FP8 records are MLA-only
    (dict(num_q_heads=7), -2),
    (dict(num_q_heads=0), -2),
    (dict(topk=0), -2),
    (dict(sm_scale=math.inf), -2),
    (dict(head_dim_qk=128, head_dim_v=128, q_row_stride=768, kv_row_stride=128,
          v_row_stride=128, out_row_stride=768), -4),
    (dict(num_q_heads=33, q_row_stride=33 * 256, out_row_stride=33 * 256), -4),
    (dict(q_row_stride=6 * 256 - 8), -2),
    (dict(q_row_stride=6 * 256 + 4), -2),
    (dict(kv_row_stride=250), -2),
    (dict(v_row_stride=260), -2),
    (dict(kv_row_stride=1 << 31), -2),
    (dict(v_row_stride=1 << 31), -2),
    (dict(idx_row_stride=2050), -2),
    (dict(out_row_stride=6 * 256 + 2), -2),
])
def test_validate_rejects(kw, code):
    assert sa.sa_validate_attn(_desc(**kw)) == code
    assert sa.sa_last_error() != ""


def test_wide_head_groups():
    # up to 32 query heads per KV head; MLA above 16 heads needs one latent head
    assert sa.sa_validate_attn(_desc(num_q_heads=32, q_row_stride=32 * 256,
                                     out_row_stride=32 * 256)) == sa.SA_OK
    assert sa.sa_validate_attn(_mla(num_q_heads=32, q_row_stride=32 * 576,
                                    out_row_stride=32 * 512)) == sa.SA_OK
    assert sa.sa_validate_attn(_mla(num_q_heads=48, num_kv_heads=2, q_row_stride=48 * 576,
                                    kv_row_stride=2 * 576, out_row_stride=48 * 512)) == -4
    # a 32-head group only fits union tiles of one row
    d = _desc(num_q_heads=32, q_row_stride=32 * 256, out_row_stride=32 * 256)
    assert sa.sa_validate_attn(d, 1) == sa.SA_OK
    assert sa.sa_validate_attn(d, 2) == sa.SA_OK_FALLBACK


def test_union_fallback_and_g_range():
    # 16 heads with G = 4 needs a 64-row tile: per-token fallback
    d = _mla(num_q_heads=16, q_row_stride=16 * 576, out_row_stride=16 * 512)
    assert sa.sa_validate_attn(d, 4) == sa.SA_OK_FALLBACK
    assert sa.sa_validate_attn(d, 2) == sa.SA_OK
    assert sa.sa_validate_attn(_mla(), 9) == -2
    assert sa.sa_validate_attn(_mla(), 0) == -2


def test_entry_points_reject_without_touching_device():
    lib = sa.lib()
    d = _desc()
    # NULL pointers with rows > 0
    st = lib.sparse_attn_prefill(ctypes.byref(d), None, None, None, None, None, 4, 10, None,
                                 None, None)
    assert st == -1
    # misaligned q
    st = lib.sparse_attn_prefill(ctypes.byref(d), 0x1008, 0x2000, 0x3000, 0x4000, None, 4, 10,
                                 0x5000, 0x6000, None)
    assert st == -2
    # zero rows: nothing to launch
    before = sa.sa_call_count("sparse_attn_prefill")
    st = lib.sparse_attn_prefill(ctypes.byref(d), None, None, None, None, None, 0, 10, None,
                                 None, None)
    assert st == 0 and sa.sa_call_count("sparse_attn_prefill") == before + 1
    # negative sizes
    st = lib.sparse_attn_prefill(ctypes.byref(d), None, None, None, None, None, -1, 10, None,
                                 None, None)
    assert st == -2
    # chunk prefill: rows but no requests
    st = lib.sparse_attn_chunk_prefill(ctypes.byref(d), None, None, None, None, None, None, 0,
                                       5, None, None, None)
    assert st == -2
    st = lib.sparse_attn_chunk_prefill(ctypes.byref(d), 0x1000, 0x2000, 0x3000, 0x4000, None,
                                       None, 2, 5, 0x5000, 0x6000, None)
    assert st == -1
    # null desc
    assert lib.sparse_attn_prefill(None, None, None, None, None, None, 1, 1, None, None,
                                   None) == -1


def test_grid_beyond_one_launch_is_refused_on_the_host():
    # 2^31 - 1 rows over 16 KV heads (group 1, four rows per one-wave team)
    # need 2^33 teams: refused before any launch, not wrapped to a small grid
    lib = sa.lib()
    d = _desc(num_q_heads=16, num_kv_heads=16, q_row_stride=16 * 256, kv_row_stride=16 * 256,
              v_row_stride=16 * 256, out_row_stride=16 * 256)
    before = sa.sa_call_count("sparse_attn_prefill")
    st = lib.sparse_attn_prefill(ctypes.byref(d), 0x1000, 0x2000, 0x3000, 0x4000, None,
                                 (1 << 31) - 1, 10, 0x5000, 0x6000, None)
    assert st == -2 and "exceed one launch" in sa.sa_last_error()
    assert sa.sa_call_count("sparse_attn_prefill") == before


def test_bad_entry_count_is_zero():
    assert sa.sa_call_count(99) == 0
    assert sa.sa_call_count(-1) == 0


def test_union_workspace_bytes():
    n = sa.sparse_attn_union_workspace_bytes(4096, 2048, 4)
    # sorted keys + union rows (int32 + uint8) + lengths
    assert n >= 4096 * 2048 * 4 + 1024 * 8192 * 5 + 1024 * 4
    assert n % 256 == 0
    assert sa.sparse_attn_union_workspace_bytes(10, 2051, 2) >= 10 * 4096 * 4
    assert sa.sparse_attn_union_workspace_bytes(10, 0, 2) == 0
    assert sa.sparse_attn_union_workspace_bytes(10, 20, 9) == 0
    assert sa.sparse_attn_union_workspace_bytes(10, 9000, 2) == 0
    assert sa.sparse_attn_union_workspace_bytes(-1, 20, 2) == 0


def test_union_build_and_pages_reject_on_host():
    lib = sa.lib()
    # bad G, missing workspace, null outputs
    assert lib.sparse_attn_union_build(0x1000, 8, 4, 8, 100, 9, 0x2000, 0x3000, 0x4000, 0x5000,
                                       1 << 20, None) == -2
    assert lib.sparse_attn_union_build(0x1000, 8, 4, 8, 100, 2, 0x2000, 0x3000, 0x4000, None, 0,
                                       None) == -5
    assert lib.sparse_attn_union_build(0x1000, 8, 4, 8, 100, 2, None, 0x3000, 0x4000, 0x5000,
                                       1 << 20, None) == -1
    assert lib.sparse_attn_union_build(0x1000, 4, 4, 8, 100, 2, 0x2000, 0x3000, 0x4000, 0x5000,
                                       1 << 20, None) == -2
    d = sa.PageDesc(src_page_tokens=256, dst_page_tokens=96, row_bytes=656, scale_bytes=4,
                    src_page_stride=168960, dst_page_stride=42240)
    assert lib.page_split(ctypes.byref(d), 0x1000, 0x2000, None, 4, None) == -2
    d = sa.PageDesc(src_page_tokens=256, dst_page_tokens=64, row_bytes=656, scale_bytes=4,
                    src_page_stride=168960, dst_page_stride=42000)
    assert lib.page_split(ctypes.byref(d), 0x1000, 0x2000, None, 4, None) == -2
    d.dst_page_stride = 42240
    assert lib.page_split(ctypes.byref(d), None, 0x2000, None, 4, None) == -1
    assert lib.page_split(None, None, None, None, 4, None) == -1
    assert lib.page_mark(0x1000, 10, 4096, 0, 0x2000, None) == -2
    assert lib.page_mark(0x1000, 10, 4096, 256, None, None) == -1
    assert lib.page_mark(None, 10, 4096, 256, 0x2000, None) == -1


def test_prefill_union_rejects_on_host():
    lib = sa.lib()
    d = _mla()
    # workspace too small for a legal union
    st = lib.sparse_attn_prefill_union(ctypes.byref(d), 0x1000, 0x2000, None, 0x3000, 8, 100, 2,
                                       None, 0, 0x4000, 0x5000, None)
    assert st == -5
    assert "workspace" in sa.sa_last_error()


def test_chunk_union_workspace_and_host_rejections():
    # first group ids, then at most ceil(total_q / G) + num_reqs groups of
    # align16(G * topk) int32 + uint8 rows and their lengths
    groups = (28988 + 1) // 2 + 16
    stride = (2 * 2051 + 15) // 16 * 16
    n = sa.sparse_attn_chunk_union_workspace_bytes(28988, 16, 2051, 2)
    assert n >= 17 * 4 + groups * stride * 5 + groups * 4 and n % 256 == 0
    assert sa.sparse_attn_chunk_union_workspace_bytes(10, 0, 20, 2) == 0
    assert sa.sparse_attn_chunk_union_workspace_bytes(10, 2, 20, 9) == 0
    assert sa.sparse_attn_chunk_union_workspace_bytes(-1, 2, 20, 2) == 0
    lib = sa.lib()
    d = _desc()
    f = lib.sparse_attn_chunk_prefill_union
    # rows but no request; missing cu_seqlens; missing and short workspace;
    # misaligned workspace; bad G
    assert f(ctypes.byref(d), None, None, None, None, None, None, 0, 5, 2, None, 0, None, None,
             None) == -2
    assert f(ctypes.byref(d), 0x1000, 0x2000, 0x3000, 0x4000, None, None, 2, 5, 2, 0x7000, 1 << 20,
             0x5000, 0x6000, None) == -1
    assert f(ctypes.byref(d), 0x1000, 0x2000, 0x3000, 0x4000, 0x8000, 0x9000, 2, 5, 2, None, 0,
             0x5000, 0x6000, None) == -5
    assert f(ctypes.byref(d), 0x1000, 0x2000, 0x3000, 0x4000, 0x8000, 0x9000, 2, 5, 2, 0x7000, 64,
             0x5000, 0x6000, None) == -5
    assert f(ctypes.byref(d), 0x1000, 0x2000, 0x3000, 0x4000, 0x8000, 0x9000, 2, 5, 2, 0x7010,
             1 << 20, 0x5000, 0x6000, None) == -2
    assert f(ctypes.byref(d), 0x1000, 0x2000, 0x3000, 0x4000, 0x8000, 0x9000, 2, 5, 9, 0x7000,
             1 << 20, 0x5000, 0x6000, None) == -2
    # no rows: nothing to launch, counted
    before = sa.sa_call_count("sparse_attn_chunk_prefill_union")
    assert f(ctypes.byref(d), None, None, None, None, None, None, 0, 0, 2, None, 0, None, None,
             None) == 0
    assert sa.sa_call_count("sparse_attn_chunk_prefill_union") == before + 1


def test_fp8_records_validation():
    # 656-byte records for the MLA shape; stride in bytes, multiple of 16
    d = _mla(kv_dtype=sa.SA_DTYPE_FP8_E4M3, kv_row_stride=656)
    assert sa.sa_validate_attn(d) == sa.SA_OK
    assert sa.sa_validate_attn(_mla(kv_dtype=sa.SA_DTYPE_FP8_E4M3, kv_row_stride=672)) == sa.SA_OK
    assert sa.sa_validate_attn(_mla(kv_dtype=sa.SA_DTYPE_FP8_E4M3, kv_row_stride=648)) == -2
    assert sa.sa_validate_attn(_mla(kv_dtype=sa.SA_DTYPE_FP8_E4M3, kv_row_stride=664)) == -2
    assert sa.sa_validate_attn(_mla(kv_dtype=7)) == -3


def test_decode_workspace_bytes():
    # ~512 (request, range) teams, each range at most 8 of a request's 16-slot
    # tiles: batch 32 x 2048 slots -> 16 ranges; partial O [512][8][512]
    # fp32, then LSE
    assert sa.sparse_attn_decode_workspace_bytes(32, 8, 2048) == 32 * 16 * 8 * 2048 + 32 * 16 * 8 * 4
    # batch 1: one range per tile (128 ranges)
    assert sa.sparse_attn_decode_workspace_bytes(1, 8, 2048) == 128 * 8 * 2048 + 4096
    # batch 512: one range per request; 7 tiles of slots -> 1 range
    assert sa.sparse_attn_decode_workspace_bytes(512, 2, 100) == 512 * 2 * 2048 + 4096
    # batch 8: 64 ranges of 2 tiles each
    assert sa.sparse_attn_decode_workspace_bytes(8, 8, 2048) == 8 * 64 * 8 * 2048 + 8 * 64 * 8 * 4
    # batch 512 x 2048 slots: 128 tiles need 16 ranges of 8
    assert sa.sparse_attn_decode_workspace_bytes(512, 1, 2048) == 512 * 16 * 2048 + 32768
    assert sa.sparse_attn_decode_workspace_bytes(0, 8, 2048) == 0
    # 32 heads (two 16-head slices of one launch each): batch 4 -> 128 ranges
    assert sa.sparse_attn_decode_workspace_bytes(4, 32, 2048) == 4 * 128 * 32 * 2048 + 4 * 128 * 32 * 4
    assert sa.sparse_attn_decode_workspace_bytes(4, 33, 2048) == 0
    assert sa.sparse_attn_decode_workspace_bytes(4, 8, 0) == 0


def test_decode_rejects_on_host():
    lib = sa.lib()
    f = lib.sparse_attn_decode_paged

    def pg(**kw):
        g = dict(src_page_tokens=256, dst_page_tokens=64, row_bytes=656, scale_bytes=4,
                 src_page_stride=256 * 660, dst_page_stride=64 * 660)
        g.update(kw)
        return sa.PageDesc(**g)

    fp8 = _mla(kv_dtype=sa.SA_DTYPE_FP8_E4M3, kv_row_stride=656)
    ws = sa.sparse_attn_decode_workspace_bytes(32, 8, 2048)

    def call(d=fp8, p=pg(), batch=32, w=0x10000, wb=ws, pool=0x2000):
        return f(ctypes.byref(d), None if p is None else ctypes.byref(p), 0x1000, pool, 16384,
                 0x3000, None, batch, w, wb, 0x4000, 0x5000, None)

    assert call(d=_mla()) == -3                                     # bf16 rows
    assert call(d=_mla(kv_dtype=sa.SA_DTYPE_FP8_E4M3, kv_row_stride=656, num_kv_heads=2,
                       q_row_stride=8 * 576)) == -2                 # two latent heads
    assert call(p=None) == -1
    assert call(p=pg(dst_page_tokens=48)) == -2                     # not a power of two
    assert call(p=pg(row_bytes=660)) == -2
    assert call(d=_mla(kv_dtype=sa.SA_DTYPE_FP8_E4M3, kv_row_stride=672)) == -2
    assert call(p=pg(dst_page_stride=64 * 660 + 8)) == -2          # not a multiple of 16
    assert call(p=pg(dst_page_stride=64 * 600)) == -2               # shorter than a page
    assert call(pool=None) == -1
    assert call(w=None, wb=0) == -5
    assert call(wb=ws - 1) == -5
    assert call(w=0x10010) == -5                                    # misaligned workspace
    assert call(batch=-1) == -2
    before = sa.sa_call_count("sparse_attn_decode_paged")
    assert call(batch=0, w=None, wb=0) == 0                         # nothing to launch, counted
    assert sa.sa_call_count("sparse_attn_decode_paged") == before + 1


def test_decode_noalloc_rejects_on_host():
    # the same validation as the workspace entry point, then the size check
    # against the static scratch, all before the scratch is looked up
    f = sa.lib().sparse_attn_decode_paged_noalloc
    fp8 = _mla(kv_dtype=sa.SA_DTYPE_FP8_E4M3, kv_row_stride=656)
    pg = sa.PageDesc(src_page_tokens=256, dst_page_tokens=64, row_bytes=656, scale_bytes=4,
                     src_page_stride=256 * 660, dst_page_stride=64 * 660)

    def call(d=fp8, p=pg, batch=32, pool=0x2000):
        return f(None if d is None else ctypes.byref(d), None if p is None else ctypes.byref(p),
                 0x1000, pool, 16384, 0x3000, None, batch, 0x4000, 0x5000, None)

    assert call(d=None) == -1
    assert call(d=_mla()) == -3                                     # bf16 rows
    assert call(p=None) == -1
    assert call(pool=None) == -1
    assert call(batch=-1) == -2
    # batch x heads beyond the scratch (16 ranges x 2052 B per request head)
    assert sa.sparse_attn_decode_workspace_bytes(128, 8, 2048) > sa.SA_DECODE_SCRATCH_BYTES
    assert call(batch=128) == -5
    assert "static scratch" in sa.sa_last_error()
    before = sa.sa_call_count("sparse_attn_decode_paged_noalloc")
    assert call(batch=0) == 0                                       # nothing to launch, counted
    assert sa.sa_call_count("sparse_attn_decode_paged_noalloc") == before + 1


def test_indexer_topk_rejects_on_host():
    f = sa.lib().indexer_topk
    assert f(0x1000, 32768, None, 8, 32768, 0, 0x2000, 2051, None) == -2          # k = 0
    assert f(0x1000, 32766, None, 8, 32768, 2051, 0x2000, 2051, None) == -2      # stride < kv
    assert f(0x1000, 32768, None, 8, 32768, 2051, 0x2000, 2050, None) == -2      # idx stride < k
    assert f(None, 32768, None, 8, 32768, 2051, 0x2000, 2051, None) == -1
    assert f(0x1002, 32768, None, 8, 32768, 2051, 0x2000, 2051, None) == -2      # misaligned
    assert f(0x1000, 32768, 0x3002, 8, 32768, 2051, 0x2000, 2051, None) == -2    # row_len align
    assert f(0x1000, 32768, None, -1, 32768, 2051, 0x2000, 2051, None) == -2
    before = sa.sa_call_count("indexer_topk")
    assert f(None, 0, None, 0, 0, 5, None, 5, None) == 0                          # no rows
    assert sa.sa_call_count("indexer_topk") == before + 1


def test_fp8_records_to_bf16_rejects_on_host():
    f = sa.lib().sparse_attn_fp8_records_to_bf16

    def call(pool=0x1000, ps=656, n=8, h=1, out=0x2000, os_=576):
        return f(pool, ps, n, h, None, out, os_, None)

    assert call(ps=655) == -2                 # shorter than a record
    assert call(ps=664) == -2                 # not a multiple of 16
    assert call(h=2, ps=1296) == -2           # two records need 1312 bytes
    assert call(os_=570) == -2                # shorter than a row
    assert call(os_=580) == -2                # not a multiple of 8
    assert call(n=-1) == -2
    assert call(h=0) == -2
    assert call(pool=None) == -1
    assert call(out=None) == -1
    assert call(pool=0x1008) == -2            # misaligned
    before = sa.sa_call_count("sparse_attn_fp8_records_to_bf16")
    assert call(n=0, pool=None, out=None) == 0    # nothing to launch, counted
    assert sa.sa_call_count("sparse_attn_fp8_records_to_bf16") == before + 1


def test_probe_gather_rejects_on_host():
    h = sa.lib()
    null = ctypes.c_void_p(0)
    shape, null_ptr = -2, -1
    assert h.sa_probe_gather(null, null, 10, null, 4, 0, 1, null, null) == shape   # topk 0
    assert h.sa_probe_gather(null, null, 10, null, 4, 8, 2, null, null) == shape   # mode
    assert h.sa_probe_gather(null, null, 1 << 23, null, 4, 8, 1, null, null) == shape   # > 2 GiB
    assert h.sa_probe_gather(null, null, 10, null, 4, 8, 1, null, null) == null_ptr
    assert h.sa_probe_gather(null, null, 10, null, 0, 8, 1, null, null) == sa.SA_OK   # no rows
