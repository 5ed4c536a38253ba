"""Index-gathered sparse attention forward for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI in ``include/sparse_attn.h``: every
function here has the name of the C entry point it calls, checks and
marshals torch tensors (device pointers, strides, the current HIP stream),
allocates outputs when none are given, and raises on a non-OK status. All
computation runs in the library's HIP kernels; there is no other code path,
and a missing or unloadable library raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "SparseAttnError",
    "lib",
    "sparse_attn_prefill",
    "sparse_attn_chunk_prefill",
    "sparse_attn_union_workspace_bytes",
    "sparse_attn_union_build",
    "sparse_attn_prefill_union",
    "sparse_attn_chunk_union_workspace_bytes",
    "sparse_attn_chunk_prefill_union",
    "page_mark",
    "page_split",
    "sparse_attn_decode_workspace_bytes",
    "sparse_attn_decode_paged",
    "sparse_attn_decode_paged_noalloc",
    "indexer_topk",
    "sa_validate_attn",
    "sa_last_error",
    "sa_call_count",
    "AttnDesc",
    "PageDesc",
    "SA_OK",
    "SA_OK_FALLBACK",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsparse_attn.so")

SA_OK = 0
SA_OK_FALLBACK = 1
SA_DTYPE_BF16 = 1
SA_DTYPE_FP8_E4M3 = 2
STATUS_NAMES = {0: "SA_OK", 1: "SA_OK_FALLBACK", -1: "SA_ERR_NULL", -2: "SA_ERR_SHAPE",
                -3: "SA_ERR_DTYPE", -4: "SA_ERR_UNSUPPORTED", -5: "SA_ERR_WORKSPACE",
                -6: "SA_ERR_HIP"}
ENTRIES = {"sparse_attn_prefill": 0, "sparse_attn_chunk_prefill": 1,
           "sparse_attn_union_build": 2, "sparse_attn_prefill_union": 3,
           "page_mark": 4, "page_split": 5, "sparse_attn_chunk_prefill_union": 6,
           "sparse_attn_decode_paged": 7, "indexer_topk": 8,
           "sparse_attn_decode_paged_noalloc": 9, "sparse_attn_fp8_records_to_bf16": 10}
SA_DECODE_SCRATCH_BYTES = 32 << 20


class SparseAttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)}: {sa_last_error()}")


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim_qk", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("v_in_k", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("q_row_stride", ctypes.c_int64),
        ("kv_row_stride", ctypes.c_int64),
        ("v_row_stride", ctypes.c_int64),
        ("idx_row_stride", ctypes.c_int64),
        ("out_row_stride", ctypes.c_int64),
    ]


class PageDesc(ctypes.Structure):
    _fields_ = [
        ("src_page_tokens", ctypes.c_int32),
        ("dst_page_tokens", ctypes.c_int32),
        ("row_bytes", ctypes.c_int32),
        ("scale_bytes", ctypes.c_int32),
        ("src_page_stride", ctypes.c_int64),
        ("dst_page_stride", ctypes.c_int64),
    ]


_P = ctypes.c_void_p
_I32, _I64, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_SIGNATURES = {
    "sparse_attn_prefill": (_I32, [ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _P, _I32, _I32,
                                   _P, _P, _P]),
    "sparse_attn_chunk_prefill": (_I32, [ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _P, _P,
                                         _I32, _I32, _P, _P, _P]),
    "sparse_attn_union_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "sparse_attn_union_build": (_I32, [_P, _I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _SZ,
                                       _P]),
    "sparse_attn_prefill_union": (_I32, [ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _I32, _I32,
                                         _I32, _P, _SZ, _P, _P, _P]),
    "sparse_attn_chunk_union_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "sparse_attn_chunk_prefill_union": (_I32, [ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _P, _P,
                                               _I32, _I32, _I32, _P, _SZ, _P, _P, _P]),
    "page_mark": (_I32, [_P, _I64, _I32, _I32, _P, _P]),
    "page_split": (_I32, [ctypes.POINTER(PageDesc), _P, _P, _P, _I32, _P]),
    "sparse_attn_decode_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "indexer_topk": (_I32, [_P, _I64, _P, _I32, _I32, _I32, _P, _I64, _P]),
    "sparse_attn_decode_paged": (_I32, [ctypes.POINTER(AttnDesc), ctypes.POINTER(PageDesc), _P, _P,
                                        _I32, _P, _P, _I32, _P, _SZ, _P, _P, _P]),
    "sparse_attn_decode_paged_noalloc": (_I32, [ctypes.POINTER(AttnDesc), ctypes.POINTER(PageDesc),
                                                _P, _P, _I32, _P, _P, _I32, _P, _P, _P]),
    "sparse_attn_fp8_records_to_bf16": (_I32, [_P, _I64, _I32, _I32, _P, _P, _I64, _P]),
    "sa_probe_gather": (_I32, [_P, _P, _I32, _P, _I32, _I32, _I32, _P, _P]),
    "sa_validate_attn": (ctypes.c_int, [ctypes.POINTER(AttnDesc), _I32]),
    "sa_last_error": (ctypes.c_char_p, []),
    "sa_call_count": (ctypes.c_uint64, [_I32]),
}

_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it is missing: build it with
    ``python -m top_index_sparse_amd.build``)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m top_index_sparse_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def sa_last_error() -> str:
    return lib().sa_last_error().decode()


def sa_call_count(entry) -> int:
    if isinstance(entry, str):
        entry = ENTRIES[entry]
    return int(lib().sa_call_count(entry))


def sa_validate_attn(desc: AttnDesc, G: int = 1) -> int:
    return int(lib().sa_validate_attn(ctypes.byref(desc), G))


# ------------------------------------------------------------------ helpers

def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _check(status: int, what: str) -> int:
    if status not in (SA_OK, SA_OK_FALLBACK):
        raise SparseAttnError(status, what)
    return status


def _need(t: torch.Tensor, name: str, dtype, ndim: int, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _need_size(t: torch.Tensor, name: str, rows: int, inner: Tuple[int, ...]):
    """At least `rows` rows, and exactly the given inner dims: the kernels
    write rows 0 .. rows - 1 at the tensor's row stride."""
    if t.shape[0] < rows or tuple(t.shape[1:]) != tuple(inner):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, needs [>= {rows}, "
                         f"{', '.join(str(d) for d in inner)}]")


def _rows_dense(t: torch.Tensor, name: str):
    """Inner dims contiguous; the row stride is free."""
    if t.dim() >= 2 and t.numel() > 0:
        inner = t[0]
        if not inner.is_contiguous():
            raise ValueError(f"{name}: every row must be contiguous")


FP8_RECORD_BYTES = 656   # 512 E4M3 latent values, 4 fp32 block scales, 64 bf16 rope


def _kv_dtype_code(t: torch.Tensor) -> int:
    """bf16 K/V, or FP8 MLA records given as uint8 [tokens, Hkv, 656]."""
    if t.dtype == torch.bfloat16:
        return SA_DTYPE_BF16
    if t.dtype == torch.uint8 and t.dim() == 3 and t.shape[2] == FP8_RECORD_BYTES:
        return SA_DTYPE_FP8_E4M3
    raise TypeError(f"K dtype {t.dtype} / shape {tuple(t.shape)} is not supported "
                    "(bf16, or uint8 [tokens, Hkv, 656] FP8 MLA records)")


def make_desc(q: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor], idx: torch.Tensor,
              out: torch.Tensor, sm_scale: float, head_dim_v: int) -> AttnDesc:
    v_in_k = v is None
    return AttnDesc(
        num_q_heads=q.shape[1], num_kv_heads=k.shape[1], head_dim_qk=q.shape[2],
        head_dim_v=head_dim_v, topk=idx.shape[1], v_in_k=int(v_in_k),
        kv_dtype=_kv_dtype_code(k), sm_scale=float(sm_scale),
        q_row_stride=q.stride(0), kv_row_stride=k.stride(0),
        v_row_stride=(k.stride(0) if v_in_k else v.stride(0)),
        idx_row_stride=idx.stride(0), out_row_stride=out.stride(0))


def _prep_attn(q, k, v, idx, sm_scale, head_dim_v, out, lse, num_rows):
    if k.dtype != torch.bfloat16:
        _kv_dtype_code(k)
    _need(q, "q", torch.bfloat16, 3)
    _need(k, "k", k.dtype, 3, q.device)
    _need(idx, "idx", torch.int32, 2, q.device)
    if v is not None:
        _need(v, "v", k.dtype, 3, q.device)
        head_dim_v = v.shape[2]
    elif head_dim_v is None:
        raise ValueError("head_dim_v is required when V lives in K (v=None)")
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (idx, "idx")):
        if t is not None:
            _rows_dense(t, name)
    if idx.shape[0] != num_rows or q.shape[0] != num_rows:
        raise ValueError(f"q rows {q.shape[0]} / idx rows {idx.shape[0]} != {num_rows}")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[2])
    if out is None:
        out = torch.empty((num_rows, q.shape[1], head_dim_v), dtype=torch.float32,
                          device=q.device)
    if lse is None:
        lse = torch.empty((num_rows, q.shape[1]), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, 3, q.device)
    _need(lse, "lse", torch.float32, 2, q.device)
    _need_size(out, "out", num_rows, (q.shape[1], head_dim_v))
    _need_size(lse, "lse", num_rows, (q.shape[1],))
    _rows_dense(out, "out")
    if not lse.is_contiguous():
        raise ValueError("lse must be contiguous")
    desc = make_desc(q, k, v, idx, out, sm_scale, head_dim_v)
    return desc, out, lse


# ------------------------------------------------------------- entry points

def sparse_attn_prefill(q: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor],
                        idx: torch.Tensor, *, sm_scale: Optional[float] = None,
                        kv_len: Optional[int] = None, topk_len: Optional[torch.Tensor] = None,
                        head_dim_v: Optional[int] = None, out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None,
                        stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-token sparse prefill over one request (C: sparse_attn_prefill).

    q [T, Hq, Dqk] bf16; k [kv, Hkv, Dqk] bf16; v [kv, Hkv, Dv] bf16 or None
    (V = first head_dim_v columns of K); idx [T, topk] int32 (-1 = padding);
    topk_len optional [T] int32. Returns (out [T, Hq, Dv] fp32, lse [T, Hq]).
    """
    T = q.shape[0]
    desc, out, lse = _prep_attn(q, k, v, idx, sm_scale, head_dim_v, out, lse, T)
    if topk_len is not None:
        _need(topk_len, "topk_len", torch.int32, 1, q.device)
        if topk_len.shape[0] != T or not topk_len.is_contiguous():
            raise ValueError("topk_len must be a contiguous [T] tensor")
    kv_len = k.shape[0] if kv_len is None else int(kv_len)
    if kv_len > k.shape[0]:
        raise ValueError(f"kv_len {kv_len} > k rows {k.shape[0]}")
    st = lib().sparse_attn_prefill(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(idx),
                                   _ptr(topk_len), T, kv_len, _ptr(out), _ptr(lse),
                                   _stream(stream))
    _check(st, "sparse_attn_prefill")
    return out, lse


def sparse_attn_chunk_prefill(q: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor],
                              idx: torch.Tensor, cu_seqlens_q: torch.Tensor,
                              cu_seqlens_kv: torch.Tensor, *, total_q: Optional[int] = None,
                              sm_scale: Optional[float] = None,
                              head_dim_v: Optional[int] = None,
                              out: Optional[torch.Tensor] = None,
                              lse: Optional[torch.Tensor] = None,
                              stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Ragged chunk prefill (C: sparse_attn_chunk_prefill). cu_seqlens_q
    int32 [R+1] and cu_seqlens_kv int64 [R+1] are device tensors; indices are
    local to each request's KV range. total_q defaults to q.shape[0]."""
    T = q.shape[0] if total_q is None else int(total_q)
    desc, out, lse = _prep_attn(q, k, v, idx, sm_scale, head_dim_v, out, lse, T)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1, q.device)
    _need(cu_seqlens_kv, "cu_seqlens_kv", torch.int64, 1, q.device)
    R = cu_seqlens_q.shape[0] - 1
    if cu_seqlens_kv.shape[0] != R + 1 or not cu_seqlens_q.is_contiguous() \
            or not cu_seqlens_kv.is_contiguous():
        raise ValueError("cu_seqlens_q/kv must be contiguous [R+1]")
    st = lib().sparse_attn_chunk_prefill(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(idx), _ptr(cu_seqlens_q), _ptr(cu_seqlens_kv),
                                         R, T, _ptr(out), _ptr(lse), _stream(stream))
    _check(st, "sparse_attn_chunk_prefill")
    return out, lse


def sparse_attn_union_workspace_bytes(num_rows: int, topk: int, G: int) -> int:
    return int(lib().sparse_attn_union_workspace_bytes(num_rows, topk, G))


def _workspace(ws, nbytes, device):
    if ws is None:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} B, needs {nbytes}")
    return ws


def sparse_attn_union_build(idx: torch.Tensor, kv_len: int, G: int, *,
                            union_idx: Optional[torch.Tensor] = None,
                            union_bits: Optional[torch.Tensor] = None,
                            union_len: Optional[torch.Tensor] = None,
                            ws: Optional[torch.Tensor] = None, stream=None):
    """Union-of-G index sets (C: sparse_attn_union_build). Returns
    (union_idx int32 [ceil(T/G), G*topk], union_bits uint8 [same],
    union_len int32 [ceil(T/G)])."""
    _need(idx, "idx", torch.int32, 2)
    _rows_dense(idx, "idx")
    T, K = idx.shape
    ng = (T + G - 1) // G
    dev = idx.device
    if union_idx is None:
        union_idx = torch.empty((ng, G * K), dtype=torch.int32, device=dev)
    if union_bits is None:
        union_bits = torch.empty((ng, G * K), dtype=torch.uint8, device=dev)
    if union_len is None:
        union_len = torch.empty((ng,), dtype=torch.int32, device=dev)
    for t, name, dtype in ((union_idx, "union_idx", torch.int32), (union_bits, "union_bits", torch.uint8),
                           (union_len, "union_len", torch.int32)):
        if not t.is_contiguous() or t.device != dev or t.dtype != dtype:
            raise ValueError(f"{name} must be a contiguous {dtype} tensor on {dev}")
    if union_idx.dim() != 2 or union_bits.dim() != 2:
        raise ValueError("union_idx and union_bits are [groups, G * topk] tensors")
    _need_size(union_idx, "union_idx", ng, (G * K,))
    _need_size(union_bits, "union_bits", ng, (G * K,))
    if union_len.numel() < ng:
        raise ValueError(f"union_len holds {union_len.numel()} entries, needs {ng}")
    nbytes = sparse_attn_union_workspace_bytes(T, K, G)
    ws = _workspace(ws, nbytes, dev)
    st = lib().sparse_attn_union_build(_ptr(idx), idx.stride(0), T, K, int(kv_len), G,
                                       _ptr(union_idx), _ptr(union_bits), _ptr(union_len),
                                       _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "sparse_attn_union_build")
    return union_idx, union_bits, union_len


def sparse_attn_prefill_union(q: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor],
                              idx: torch.Tensor, G: int, *, sm_scale: Optional[float] = None,
                              kv_len: Optional[int] = None, head_dim_v: Optional[int] = None,
                              ws: Optional[torch.Tensor] = None,
                              out: Optional[torch.Tensor] = None,
                              lse: Optional[torch.Tensor] = None, stream=None):
    """Union-mode sparse prefill (C: sparse_attn_prefill_union). Returns
    (out, lse, status) where status is SA_OK or SA_OK_FALLBACK."""
    T = q.shape[0]
    desc, out, lse = _prep_attn(q, k, v, idx, sm_scale, head_dim_v, out, lse, T)
    kv_len = k.shape[0] if kv_len is None else int(kv_len)
    if kv_len > k.shape[0]:
        raise ValueError(f"kv_len {kv_len} > k rows {k.shape[0]}")
    nbytes = sparse_attn_union_workspace_bytes(T, idx.shape[1], G)
    ws = _workspace(ws, nbytes, q.device)
    st = lib().sparse_attn_prefill_union(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(idx), T, kv_len, G, _ptr(ws),
                                         ws.numel() * ws.element_size(), _ptr(out), _ptr(lse),
                                         _stream(stream))
    return out, lse, _check(st, "sparse_attn_prefill_union")


def sparse_attn_chunk_union_workspace_bytes(total_q: int, num_reqs: int, topk: int,
                                            G: int) -> int:
    return int(lib().sparse_attn_chunk_union_workspace_bytes(total_q, num_reqs, topk, G))


def sparse_attn_chunk_prefill_union(q: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor],
                                    idx: torch.Tensor, cu_seqlens_q: torch.Tensor,
                                    cu_seqlens_kv: torch.Tensor, G: int, *,
                                    total_q: Optional[int] = None,
                                    sm_scale: Optional[float] = None,
                                    head_dim_v: Optional[int] = None,
                                    ws: Optional[torch.Tensor] = None,
                                    out: Optional[torch.Tensor] = None,
                                    lse: Optional[torch.Tensor] = None, stream=None):
    """Union-mode ragged chunk prefill (C: sparse_attn_chunk_prefill_union).
    Groups of G rows never span requests. Returns (out, lse, status) where
    status is SA_OK or SA_OK_FALLBACK."""
    T = q.shape[0] if total_q is None else int(total_q)
    desc, out, lse = _prep_attn(q, k, v, idx, sm_scale, head_dim_v, out, lse, T)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1, q.device)
    _need(cu_seqlens_kv, "cu_seqlens_kv", torch.int64, 1, q.device)
    R = cu_seqlens_q.shape[0] - 1
    if cu_seqlens_kv.shape[0] != R + 1 or not cu_seqlens_q.is_contiguous() \
            or not cu_seqlens_kv.is_contiguous():
        raise ValueError("cu_seqlens_q/kv must be contiguous [R+1]")
    nbytes = sparse_attn_chunk_union_workspace_bytes(T, max(R, 1), idx.shape[1], G)
    ws = _workspace(ws, nbytes, q.device)
    st = lib().sparse_attn_chunk_prefill_union(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                               _ptr(idx), _ptr(cu_seqlens_q),
                                               _ptr(cu_seqlens_kv), R, T, G, _ptr(ws),
                                               ws.numel() * ws.element_size(), _ptr(out),
                                               _ptr(lse), _stream(stream))
    return out, lse, _check(st, "sparse_attn_chunk_prefill_union")


def fp8_records_to_bf16(pool: torch.Tensor, *, mask: Optional[torch.Tensor] = None,
                        out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """FP8 MLA records to bf16 rows (C: sparse_attn_fp8_records_to_bf16).

    pool uint8 [tokens, Hkv, 656] (row stride free, a multiple of 16 bytes);
    mask optional int8 [tokens] (rows with 0 are not written); out optional
    bf16 [tokens, Hkv, 576] (row stride free). Returns out.
    """
    _need(pool, "pool", torch.uint8, 3)
    if pool.shape[2] != 656:
        raise ValueError(f"pool records are 656 bytes, got {pool.shape[2]}")
    _rows_dense(pool, "pool")
    T, H = pool.shape[0], pool.shape[1]
    if out is None:
        out = torch.empty((T, H, 576), dtype=torch.bfloat16, device=pool.device)
    _need(out, "out", torch.bfloat16, 3, pool.device)
    _need_size(out, "out", T, (H, 576))
    _rows_dense(out, "out")
    if mask is not None:
        _need(mask, "mask", torch.int8, 1, pool.device)
        if mask.shape[0] < T or not mask.is_contiguous():
            raise ValueError("mask must be a contiguous int8 tensor of at least tokens entries")
    st = lib().sparse_attn_fp8_records_to_bf16(
        _ptr(pool), pool.stride(0) if T else H * 656, T, H, _ptr(mask), _ptr(out),
        out.stride(0) if T else H * 576, _stream(stream))
    _check(st, "sparse_attn_fp8_records_to_bf16")
    return out


def probe_gather(k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor, *, eight_waves: bool = True,
                 out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Measurement aid (C: sa_probe_gather): the head-dim-256 kernels' K/V
    row gathers alone. k, v bf16 [kv_len, 256] (contiguous); idx int32
    [rows, topk] (contiguous). Returns uint32 checksums [rows, 64] (as int32)."""
    for t, name in ((k, "k"), (v, "v")):
        _need(t, name, torch.bfloat16, 2)
        if t.shape[1] != 256 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [kv_len, 256] bf16 tensor")
    if v.shape[0] != k.shape[0]:
        raise ValueError("k and v must have the same rows")
    _need(idx, "idx", torch.int32, 2, k.device)
    if not idx.is_contiguous():
        raise ValueError("idx must be contiguous")
    rows, topk = idx.shape
    if out is None:
        out = torch.empty((rows, 64), dtype=torch.int32, device=k.device)
    _need(out, "out", torch.int32, 2, k.device)
    _need_size(out, "out", rows, (64,))
    st = lib().sa_probe_gather(_ptr(k), _ptr(v), k.shape[0], _ptr(idx), rows, topk,
                               1 if eight_waves else 0, _ptr(out), _stream(stream))
    _check(st, "sa_probe_gather")
    return out


def page_mark(idx: torch.Tensor, num_src_pages: int, src_page_tokens: int, *,
              mask: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Page mark (C: page_mark). Returns the int8 [num_src_pages] mask."""
    _need(idx, "idx", torch.int32, idx.dim())
    if not idx.is_contiguous():
        raise ValueError("idx must be contiguous")
    if mask is None:
        mask = torch.empty((num_src_pages,), dtype=torch.int8, device=idx.device)
    _need(mask, "mask", torch.int8, 1, idx.device)
    if mask.shape[0] < num_src_pages:
        raise ValueError("mask is shorter than num_src_pages")
    st = lib().page_mark(_ptr(idx), idx.numel(), num_src_pages, src_page_tokens, _ptr(mask),
                         _stream(stream))
    _check(st, "page_mark")
    return mask


def page_split(src: torch.Tensor, dst: torch.Tensor, mask: Optional[torch.Tensor], *,
               src_page_tokens: int, dst_page_tokens: int, row_bytes: int, scale_bytes: int,
               stream=None) -> torch.Tensor:
    """Page split (C: page_split); src uint8 [P, src_stride], dst uint8
    [P*ratio, dst_stride]; mask int8 [P] or None (split every page)."""
    _need(src, "src", torch.uint8, 2)
    _need(dst, "dst", torch.uint8, 2, src.device)
    if mask is not None:
        _need(mask, "mask", torch.int8, 1, src.device)
    _rows_dense(src, "src")
    _rows_dense(dst, "dst")
    desc = PageDesc(src_page_tokens=src_page_tokens, dst_page_tokens=dst_page_tokens,
                    row_bytes=row_bytes, scale_bytes=scale_bytes,
                    src_page_stride=src.stride(0), dst_page_stride=dst.stride(0))
    P = src.shape[0]
    if dst.shape[0] < P * (src_page_tokens // max(dst_page_tokens, 1)):
        raise ValueError("dst has fewer pages than the split produces")
    if mask is not None and mask.shape[0] < P:
        raise ValueError(f"mask holds {mask.shape[0]} pages, src has {P}")
    if src.shape[1] < src_page_tokens * (row_bytes + scale_bytes) or \
            dst.shape[1] < dst_page_tokens * (row_bytes + scale_bytes):
        raise ValueError("a src or dst row is narrower than one page")
    st = lib().page_split(ctypes.byref(desc), _ptr(src), _ptr(dst), _ptr(mask), P,
                          _stream(stream))
    _check(st, "page_split")
    return dst


def sparse_attn_decode_workspace_bytes(batch: int, num_q_heads: int, topk: int) -> int:
    return int(lib().sparse_attn_decode_workspace_bytes(batch, num_q_heads, topk))


def _decode_prep(q, pool, idx, dst_page_tokens, scale_bytes, sm_scale, topk_len, out, lse,
                 allocate):
    _need(q, "q", torch.bfloat16, 3)
    _need(pool, "pool", torch.uint8, 2, q.device)
    _need(idx, "idx", torch.int32, 2, q.device)
    _rows_dense(q, "q")
    _rows_dense(pool, "pool")
    _rows_dense(idx, "idx")
    B, Hq = q.shape[0], q.shape[1]
    if idx.shape[0] != B:
        raise ValueError(f"idx rows {idx.shape[0]} != batch {B}")
    if pool.shape[1] < dst_page_tokens * (FP8_RECORD_BYTES + scale_bytes):
        raise ValueError(f"pool rows of {pool.shape[1]} B are narrower than one page")
    if topk_len is not None:
        _need(topk_len, "topk_len", torch.int32, 1, q.device)
        if topk_len.shape[0] != B or not topk_len.is_contiguous():
            raise ValueError("topk_len must be a contiguous [B] tensor")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[2])
    if allocate and out is None:
        out = torch.empty((B, Hq, 512), dtype=torch.float32, device=q.device)
    if allocate and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if out is None or lse is None:
        raise ValueError("out and lse must be given")
    _need(out, "out", torch.float32, 3, q.device)
    _need(lse, "lse", torch.float32, 2, q.device)
    _need_size(out, "out", B, (Hq, 512))
    _need_size(lse, "lse", B, (Hq,))
    _rows_dense(out, "out")
    if not lse.is_contiguous():
        raise ValueError("lse must be contiguous")
    desc = AttnDesc(num_q_heads=Hq, num_kv_heads=1, head_dim_qk=q.shape[2], head_dim_v=512,
                    topk=idx.shape[1], v_in_k=1, kv_dtype=SA_DTYPE_FP8_E4M3,
                    sm_scale=float(sm_scale), q_row_stride=q.stride(0),
                    kv_row_stride=FP8_RECORD_BYTES, v_row_stride=FP8_RECORD_BYTES,
                    idx_row_stride=idx.stride(0), out_row_stride=out.stride(0))
    pages = PageDesc(src_page_tokens=0, dst_page_tokens=dst_page_tokens,
                     row_bytes=FP8_RECORD_BYTES, scale_bytes=scale_bytes, src_page_stride=0,
                     dst_page_stride=pool.stride(0))
    return desc, pages, out, lse, B


def sparse_attn_decode_paged(q: torch.Tensor, pool: torch.Tensor, idx: torch.Tensor, *,
                             dst_page_tokens: int = 64, scale_bytes: int = 4,
                             sm_scale: Optional[float] = None,
                             topk_len: Optional[torch.Tensor] = None,
                             ws: Optional[torch.Tensor] = None,
                             out: Optional[torch.Tensor] = None,
                             lse: Optional[torch.Tensor] = None,
                             stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Sparse MLA decode over the split pool (C: sparse_attn_decode_paged).

    q [B, Hq, 576] bf16 (one query row per request); pool uint8
    [num_dst_pages, dst_page_stride] (pages of dst_page_tokens 656-byte FP8
    records, then their per-token words); idx [B, topk] int32 pool token ids;
    topk_len optional [B] int32. Returns (out [B, Hq, 512] fp32, lse [B, Hq]).
    """
    desc, pages, out, lse, B = _decode_prep(q, pool, idx, dst_page_tokens, scale_bytes,
                                            sm_scale, topk_len, out, lse, True)
    nbytes = sparse_attn_decode_workspace_bytes(B, desc.num_q_heads, idx.shape[1])
    ws = _workspace(ws, nbytes, q.device) if B > 0 else ws
    st = lib().sparse_attn_decode_paged(ctypes.byref(desc), ctypes.byref(pages), _ptr(q),
                                        _ptr(pool), pool.shape[0], _ptr(idx), _ptr(topk_len), B,
                                        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                        _ptr(out), _ptr(lse), _stream(stream))
    _check(st, "sparse_attn_decode_paged")
    return out, lse


def sparse_attn_decode_paged_noalloc(q: torch.Tensor, pool: torch.Tensor, idx: torch.Tensor, *,
                                     out: torch.Tensor, lse: torch.Tensor,
                                     dst_page_tokens: int = 64, scale_bytes: int = 4,
                                     sm_scale: Optional[float] = None,
                                     topk_len: Optional[torch.Tensor] = None,
                                     stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Sparse MLA decode with the library's static scratch instead of a
    workspace (C: sparse_attn_decode_paged_noalloc); the caller passes out
    and lse, and nothing is allocated. Calls that overlap on one GPU race."""
    desc, pages, out, lse, B = _decode_prep(q, pool, idx, dst_page_tokens, scale_bytes,
                                            sm_scale, topk_len, out, lse, False)
    st = lib().sparse_attn_decode_paged_noalloc(ctypes.byref(desc), ctypes.byref(pages), _ptr(q),
                                                _ptr(pool), pool.shape[0], _ptr(idx),
                                                _ptr(topk_len), B, _ptr(out), _ptr(lse),
                                                _stream(stream))
    _check(st, "sparse_attn_decode_paged_noalloc")
    return out, lse


def indexer_topk(scores: torch.Tensor, k: int, *, row_len: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Indexer top-k selection (C: indexer_topk). scores [T, kv] fp32 (rows
    contiguous, any row stride); row_len optional [T] int32
    visible lengths. Returns idx [T, k] int32: ascending positions, -1 pad."""
    _need(scores, "scores", torch.float32, 2)
    _rows_dense(scores, "scores")
    T, kv = scores.shape
    if row_len is not None:
        _need(row_len, "row_len", torch.int32, 1, scores.device)
        if row_len.shape[0] != T or not row_len.is_contiguous():
            raise ValueError("row_len must be a contiguous [T] tensor")
    if out is None:
        out = torch.empty((T, k), dtype=torch.int32, device=scores.device)
    _need(out, "out", torch.int32, 2, scores.device)
    if out.shape[0] < T or out.shape[1] < k:
        raise ValueError(f"out has shape {tuple(out.shape)}, needs at least [{T}, {k}]")
    _rows_dense(out, "out")
    st = lib().indexer_topk(_ptr(scores), scores.stride(0) if T > 0 else kv, _ptr(row_len), T, kv,
                            int(k), _ptr(out), out.stride(0) if T > 0 else k, _stream(stream))
    _check(st, "indexer_topk")
    return out
