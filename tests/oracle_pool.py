"""Every-row parity at full size: the fp64 oracle evaluated over all rows of a
workload in worker processes and compared, element by element, with what the
GPU wrote.

Workers come from a forkserver that ``start()`` launches before anything
touches the GPU (``tests/conftest.py`` calls it at configure time), so no
process holding GPU state forks or execs. A worker imports numpy and
``oracle`` only: the inputs and the GPU's outputs reach it as ``.npy`` files
mapped read-only, and it sends back per-chunk error statistics, not arrays.
Its BLAS runs on one thread.

Tasks (``kind``), each following the oracle function it names:

* ``attn``        oracle.sparse_attention over a row range (one request);
* ``chunk``       oracle.chunk_prefill over a row range (ragged requests);
* ``union``       oracle.union_build + union_attention over whole groups;
* ``chunk_union`` oracle.chunk_union_build + chunk_union_attention over
                  whole groups of one request;
* ``topk``        oracle.topk_select, compared bit for bit with the GPU's
                  index rows; with ``attn_G`` set it then runs per-token
                  (0) or union (G) attention over the oracle's own selection
                  and compares that with the GPU chain's output.

FP8 MLA records (``k`` of dtype uint8) are decoded by oracle.fp8 first.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import shutil
import tempfile

import numpy as np

ATOL = 2e-2
RTOL = 1e-2
LSE_TOL = 1e-5
WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))

_started = False


def start():
    """Starts the forkserver (call before the GPU is first used)."""
    global _started
    if _started:
        return
    ctx = mp.get_context("forkserver")
    ctx.set_forkserver_preload(["numpy", "oracle", "tests.oracle_pool"])
    from multiprocessing import forkserver
    forkserver.ensure_running()
    _started = True


# ------------------------------------------------------------------ worker

def _compare(ref_o, ref_l, o, l):
    o = np.asarray(o, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    err = np.abs(o - ref_o)
    excess = err - (ATOL + RTOL * np.abs(ref_o))
    inf_ref = np.isneginf(ref_l)
    inf_bad = int(np.count_nonzero(np.isneginf(l) != inf_ref))
    dl = np.abs(l[~inf_ref] - ref_l[~inf_ref])
    w = np.unravel_index(int(np.argmax(excess)), excess.shape) if excess.size else ()
    return {
        "rows": int(ref_o.shape[0]),
        "finite": bool(np.isfinite(o).all()),
        "max_abs": float(err.max()) if err.size else 0.0,
        "max_excess": float(excess.max()) if excess.size else -1.0,
        "worst": tuple(int(x) for x in w),
        "lse_max": float(dl.max()) if dl.size else 0.0,
        "lse_inf_mismatch": inf_bad,
    }


def _shift(st, row0):
    if st.get("worst"):
        st["worst"] = (st["worst"][0] + row0,) + tuple(st["worst"][1:])
    return st


def _work(task):
    kind, d, p, lo, hi = task
    from threadpoolctl import threadpool_limits
    import oracle

    def A(name):
        return np.load(os.path.join(d, name + ".npy"), mmap_mode="r")

    def kv_rows(k):
        return oracle.mla_fp8_rows_to_f64(np.asarray(k)) if k.dtype == np.uint8 else k

    with threadpool_limits(1):
        out = A("out")
        lse = A("lse")
        q = A("q") if kind != "topk" or p.get("attn_G") is not None else None
        rows = np.arange(lo, hi)
        if kind == "attn":
            ro, rl = oracle.sparse_attention(q, kv_rows(A("k")), A("v") if p["has_v"] else None,
                                             A("idx"), num_kv_heads=p["num_kv_heads"],
                                             scale=p["scale"], kv_len=p["kv_len"],
                                             head_dim_v=p["head_dim_v"], rows=rows)
            return _shift(_compare(ro, rl, out[lo:hi], lse[lo:hi]), lo)
        if kind == "chunk":
            ro, rl = oracle.chunk_prefill(q, kv_rows(A("k")), A("v") if p["has_v"] else None,
                                          A("idx"), A("cu_q"), A("cu_kv"),
                                          num_kv_heads=p["num_kv_heads"], scale=p["scale"],
                                          head_dim_v=p["head_dim_v"], rows=rows)
            return _shift(_compare(ro, rl, out[lo:hi], lse[lo:hi]), lo)
        if kind == "union":
            G = p["G"]
            ui, ub, ul = oracle.union_build(np.asarray(A("idx")[lo:hi]), p["kv_len"], G)
            ro, rl = oracle.union_attention(np.asarray(q[lo:hi]), kv_rows(A("k")),
                                            A("v") if p["has_v"] else None, ui, ub, ul, G,
                                            num_kv_heads=p["num_kv_heads"], scale=p["scale"],
                                            head_dim_v=p["head_dim_v"])
            return _shift(_compare(ro, rl, out[lo:hi], lse[lo:hi]), lo)
        if kind == "chunk_union":
            G = p["G"]
            kv0, kv1 = p["kv0"], p["kv1"]
            k = kv_rows(A("k"))[kv0:kv1]
            v = A("v")[kv0:kv1] if p["has_v"] else None
            cu_q = np.array([0, hi - lo], dtype=np.int32)
            cu_kv = np.array([0, kv1 - kv0], dtype=np.int64)
            ui, ub, ul, owner = oracle.chunk_union_build(np.asarray(A("idx")[lo:hi]), cu_q, cu_kv, G)
            ro, rl = oracle.chunk_union_attention(np.asarray(q[lo:hi]), k, v, ui, ub, ul, owner,
                                                  cu_q, cu_kv, G, num_kv_heads=p["num_kv_heads"],
                                                  scale=p["scale"], head_dim_v=p["head_dim_v"])
            return _shift(_compare(ro, rl, out[lo:hi], lse[lo:hi]), lo)
        if kind == "topk":
            sel = oracle.topk_select(np.asarray(A("scores")[lo:hi]), p["k"],
                                     np.asarray(A("row_len")[lo:hi]))
            gidx = np.asarray(A("gpu_idx")[lo:hi])
            st = {"rows": hi - lo, "idx_mismatch_rows": int(np.count_nonzero(
                (sel != gidx).any(axis=1)))}
            G = p.get("attn_G")
            if G is None:
                return st
            kv = kv_rows(A("k"))
            v = A("v") if p["has_v"] else None
            if G == 0:
                ro, rl = oracle.sparse_attention(np.asarray(q[lo:hi]), kv, v, sel,
                                                 num_kv_heads=p["num_kv_heads"], scale=p["scale"],
                                                 kv_len=p["kv_len"], head_dim_v=p["head_dim_v"])
            else:
                ui, ub, ul = oracle.union_build(sel, p["kv_len"], G)
                ro, rl = oracle.union_attention(np.asarray(q[lo:hi]), kv, v, ui, ub, ul, G,
                                                num_kv_heads=p["num_kv_heads"],
                                                scale=p["scale"], head_dim_v=p["head_dim_v"])
            st.update(_compare(ro, rl, out[lo:hi], lse[lo:hi]))
            return _shift(st, lo)
    raise ValueError(kind)


# ------------------------------------------------------------------ driver

def row_chunks(T, step=1, pieces=None):
    """[lo, hi) ranges covering 0..T, boundaries at multiples of `step`."""
    pieces = pieces or 4 * WORKERS
    n = (T + step - 1) // step
    edges = np.linspace(0, n, min(pieces, max(n, 1)) + 1).round().astype(int) * step
    edges[-1] = T
    return [(int(a), int(b)) for a, b in zip(edges[:-1], edges[1:]) if b > a]


def ragged_chunks(cu_q, cu_kv, step=1, pieces=None):
    """Per-request ranges (lo, hi, kv0, kv1), split at multiples of `step`
    from each request's first row."""
    pieces = pieces or 4 * WORKERS
    T = int(cu_q[-1])
    out = []
    for r in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[r]), int(cu_q[r + 1])
        if q1 <= q0:
            continue
        share = max(1, round(pieces * (q1 - q0) / max(T, 1)))
        for a, b in row_chunks(q1 - q0, step, share):
            out.append((q0 + a, q0 + b, int(cu_kv[r]), int(cu_kv[r + 1])))
    return out


def run(kind, arrays, params, chunks):
    """Evaluates the oracle over every chunk and returns the merged statistics.
    chunks: (lo, hi) or (lo, hi, kv0, kv1) row ranges."""
    start()
    d = tempfile.mkdtemp(prefix="oracle_rows_")
    try:
        for name, a in arrays.items():
            np.save(os.path.join(d, name + ".npy"), np.ascontiguousarray(a))
        tasks = []
        for c in chunks:
            p = dict(params)
            if len(c) == 4:
                p["kv0"], p["kv1"] = c[2], c[3]
            tasks.append((kind, d, p, c[0], c[1]))
        ctx = mp.get_context("forkserver")
        with ctx.Pool(WORKERS) as pool:
            stats = pool.map(_work, tasks, chunksize=1)
    finally:
        shutil.rmtree(d, ignore_errors=True)
    return merge(stats)


def merge(stats):
    m = {"rows": sum(s["rows"] for s in stats), "chunks": len(stats)}
    if any("max_excess" in s for s in stats):
        att = [s for s in stats if "max_excess" in s]
        worst = max(att, key=lambda s: s["max_excess"])
        m.update({
            "finite": all(s["finite"] for s in att),
            "max_abs": max(s["max_abs"] for s in att),
            "max_excess": worst["max_excess"],
            "worst": worst["worst"],
            "lse_max": max(s["lse_max"] for s in att),
            "lse_inf_mismatch": sum(s["lse_inf_mismatch"] for s in att),
        })
    if any("idx_mismatch_rows" in s for s in stats):
        m["idx_mismatch_rows"] = sum(s.get("idx_mismatch_rows", 0) for s in stats)
    return m


def assert_ok(m, what):
    """Every row within tolerance (and bit-exact indices where compared)."""
    if "idx_mismatch_rows" in m:
        assert m["idx_mismatch_rows"] == 0, f"{what}: {m['idx_mismatch_rows']} index rows differ"
    if "max_excess" in m:
        assert m["finite"], f"{what}: non-finite output"
        assert m["max_excess"] <= 0.0, (
            f"{what}: O out of tolerance (worst at row/head/d {m['worst']}, max abs err "
            f"{m['max_abs']:.3e})")
        assert m["lse_inf_mismatch"] == 0, f"{what}: -inf LSE pattern differs"
        assert m["lse_max"] <= LSE_TOL, f"{what}: LSE max abs err {m['lse_max']:.3e}"
