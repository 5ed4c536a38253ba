"""Benchmark: sparse GQA chunk prefill, 8192 rows x 2051 slots, on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 100]

One step is one sparse_attn_chunk_prefill call over the 8192-row workload
(one request at the end of a 32768-token context, top-k 2051 random-walk
indices, 6 query heads over one KV head, head dim 256, bf16 inputs, fp32
output and log-sum-exp), with every input already resident in HBM.

Timing follows the pages' protocol: about 40 ms of untimed calls first (the
GPU's clocks ramp up after the host has left it idle), then the warm-up
calls, then the timed calls with a HIP event recorded after each one on the
launch stream; the line gives the mean and the median of the per-call times.

Prints one JSON line. `value` is the gathered-KV throughput: the K and V rows
of every valid slot (8192 * 2051 * (512 + 512) B = 17.205 GB per call)
divided by the measured time per call. Those bytes exceed HBM traffic many
times over (neighbouring rows select mostly the same tokens, which then come
from the caches), so `roofline` is taken on the vector L1 data path instead:
`achieved` is the bytes the kernel's vector loads request per call (the K/V
rows of every slot tile its teams issue, counted on the host from the index
rows and the team shapes), over the kernel's mean duration; `peak` is one
L1 tag access per clock per CU, 64 B each for these loads, x 256 CUs x
2.4 GHz. `traffic` is the HBM
bytes per call that rocprofv3 counters measured on the current kernel
source (null when the source has changed since).

`others` times every other workload the same way: C2 (group 12 over two KV
heads), MLA per-token and union G=2/4 (C3), MLA over FP8 records with the
dequant in the kernel and staged (records converted to bf16 rows once per
call), the ragged C4 chunk prefill and its union, the indexer top-k and the
chains over its rows, and the decode step (page mark, masked split, decode).

The CPU baseline runs the fp64 oracle on every row of the same workload
(`--cpu-stride N`: every N-th row), in worker processes forked before the
GPU is touched, and its results double as a parity gate on those rows.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import gen  # noqa: E402

METRIC = "sparse prefill ms/call + gathered-KV GB/s (% HBM roofline), 8192 rows × 2051 slots"
HBM_PEAK_GBS = 8000.0
# Vector L1 data cache: one tag access per clock per CU (the ceiling AMD's
# rocprofiler-compute sets for gfx950's vL1D). The gathers' 16-byte lanes
# take one access per 64 bytes (TCP_TOTAL_CACHE_ACCESSES counts 16 per
# 1 KB load instruction), so their ceiling is 64 B per clock per CU:
# 256 CUs x 64 B x 2.4 GHz.
VL1D_PEAK_GBS = 256 * 64 * 2.4
MFMA_BF16_PEAK_TFLOPS = 2500.0
FP8_RECORD_BYTES = 656          # one FP8 MLA record per gathered decode slot
KERNEL_SOURCE = os.path.join(ROOT, "top_index_sparse_amd", "csrc", "sa_gqa.hip")
COUNTER_FILE = os.path.join(ROOT, "profiles", "gqa_d256_c1_counters.txt")


def gathered_bytes(case: gen.AttnCase) -> int:
    """K and V bytes of every valid slot (one KV head per query group)."""
    if case.cu_seqlens_q is None:
        valid = int(((case.idx >= 0) & (case.idx < case.kv_len)).sum())
    else:
        valid = 0
        for r in range(len(case.cu_seqlens_q) - 1):
            rows = slice(case.cu_seqlens_q[r], case.cu_seqlens_q[r + 1])
            kv = case.cu_seqlens_kv[r + 1] - case.cu_seqlens_kv[r]
            blk = case.idx[rows]
            valid += int(((blk >= 0) & (blk < kv)).sum())
    if case.k.dtype == np.uint8:                     # FP8 MLA records
        per_slot = case.k.shape[2]
    else:
        per_slot = case.head_dim_qk * 2 + (0 if case.v_in_k else case.head_dim_v * 2)
    return valid * case.num_kv_heads * per_slot


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in ("sa_gqa.hip", "sa_attn_kernel.h", "sa_device.h", "sa_internal.h"):
        with open(os.path.join(ROOT, "top_index_sparse_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_counters():
    """The headline kernel's rocprofv3 counter summary (HBM bytes per call,
    vector L1 bytes, unit busy fractions), if it was taken on the current
    kernel source; else None."""
    try:
        with open(COUNTER_FILE) as f:
            kv = dict(l.split(":", 1) for l in f if ":" in l and not l.startswith("#"))
        if kv.get("kernel_source_sha256_16", "").strip() != kernel_source_hash():
            return None
        return {k.strip(): float(v) for k, v in kv.items() if k.strip() != "kernel_source_sha256_16"}
    except (OSError, ValueError):
        return None


def team_tiles(idx: np.ndarray, kv_len, rows_per_team: int, cu_q=None, cu_kv=None,
               every_tile: bool = False, member: bool = False):
    """Slot tiles the per-token team kernel issues, from the index rows.

    A team takes `rows_per_team` consecutive rows and walks their slots in
    tiles of 16 positions. A position is gathered once for every row whose
    token there equals the team's first row's; any other valid token is
    queued, once per run of consecutive rows holding it at that position, and
    the queue is gathered 16 tokens at a time. A tile with no valid token of
    the first row is skipped (`every_tile`: the three-tile shape issues all).
    Tokens are compared as global KV rows (request base + local index).
    `member` (two-row membership teams): a team whose two rows share one
    request of at most 32768 tokens and hold no token twice streams the
    union of its rows' sets instead, ceil(|union| / 16) tiles.

    Returns (tiles issued per KV head, valid K/V rows gathered per KV head).
    """
    T, k = idx.shape
    R = rows_per_team
    nt = (k + 15) // 16
    teams = (T + R - 1) // R
    X = np.full((teams * R, nt * 16), -1, dtype=np.int64)
    X[:T, :k] = idx
    if cu_q is None:
        ok = (X >= 0) & (X < kv_len)
        X = np.where(ok, X, -1)
    else:
        req = np.searchsorted(np.asarray(cu_q), np.arange(teams * R), side="right") - 1
        req = np.minimum(req, len(cu_q) - 2)
        base = np.asarray(cu_kv)[req][:, None]
        length = (np.asarray(cu_kv)[req + 1] - np.asarray(cu_kv)[req])[:, None]
        ok = (X >= 0) & (X < length)
        ok[T:] = False
        X = np.where(ok, X + base, -1)
    X = X.reshape(teams, R, nt * 16)
    row0 = X[:, 0, :]
    first = row0 >= 0
    primary = (np.full(teams, nt) if every_tile
               else first.reshape(teams, nt, 16).any(-1).sum(-1))
    queued = np.zeros(teams, dtype=np.int64)
    for r in range(1, R):
        x = X[:, r, :]
        start = (x >= 0) & (x != row0)
        if r >= 2:
            start &= x != X[:, r - 1, :]
        queued += start.sum(-1)
    tiles_t = primary + (queued + 15) // 16
    rows_t = first.sum(-1) + queued
    if member and R == 2:
        rows2 = np.arange(teams) * 2 + 1 < T
        if cu_q is None:
            same = np.full(teams, kv_len <= 32768)
        else:
            r2 = req.reshape(teams, 2)
            ln = np.asarray(length).reshape(teams, 2)
            same = (r2[:, 0] == r2[:, 1]) & (ln[:, 0] <= 32768)
        srt = np.sort(X, axis=-1)
        dup = ((srt[..., 1:] == srt[..., :-1]) & (srt[..., 1:] >= 0)).any(-1).any(-1)
        both = np.sort(X.reshape(teams, -1), axis=-1)
        inter = ((both[:, 1:] == both[:, :-1]) & (both[:, 1:] >= 0)).sum(-1)
        union = (both >= 0).sum(-1) - inter
        qual = rows2 & same & ~dup
        tiles_t = np.where(qual, (union + 15) // 16, tiles_t)
        rows_t = np.where(qual, union, rows_t)
    return int(tiles_t.sum()), int(rows_t.sum())


# ----------------------------------------------------------- CPU baseline

_CASE = None


def _cpu_worker(rows):
    from threadpoolctl import threadpool_limits
    import oracle
    with threadpool_limits(1):
        c = _CASE
        o, l = oracle.sparse_attention(c.q, c.k, c.v, c.idx, num_kv_heads=c.num_kv_heads,
                                       scale=c.scale, kv_len=c.kv_len, rows=rows)
    return rows, o.astype(np.float32), l


def cpu_baseline(case: gen.AttnCase, stride: int, workers: int):
    """The oracle over every `stride`-th row, split over `workers` processes."""
    import multiprocessing as mp
    global _CASE
    _CASE = case
    rows = np.arange(0, case.num_rows, stride)
    chunks = [c for c in np.array_split(rows, workers * 4) if len(c)]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(workers) as pool:
        parts = pool.map(_cpu_worker, chunks)
    wall = time.perf_counter() - t0
    sub = gen.AttnCase(case.name, case.q, case.k, case.v, case.idx[rows], case.num_kv_heads,
                       case.head_dim_qk, case.head_dim_v, case.scale, case.kv_len,
                       case.positions[rows])
    nbytes = gathered_bytes(sub)
    out_rows = np.concatenate([p[0] for p in parts])
    out_o = np.concatenate([p[1] for p in parts])
    out_l = np.concatenate([p[2] for p in parts])
    which = "every row" if stride == 1 else f"every {stride}-th row"
    return {"value": nbytes / wall / 1e9, "unit": "GB/s", "cores": workers, "kind": "oracle",
            "sample": f"{which} of the same workload ({len(rows)} of {case.num_rows} rows, "
                      f"{nbytes / 1e9:.3f} GB gathered), fp64 numpy, {workers} processes x 1 "
                      f"BLAS thread, {wall:.2f} s wall ({wall * workers:.0f} core-seconds)"}, \
        (out_rows, out_o, out_l)


# ------------------------------------------------------------------- GPU

SETTLE_MS = 40.0   # --settle-ms


def _settle(torch, stream, fn):
    """Runs fn until about SETTLE_MS of GPU time has passed. After the host
    has left the GPU idle (building the next workload's inputs), the first
    tens of milliseconds of work run at lower clocks: the headline kernel's
    duration falls from 0.49 to about 0.39 ms over its first 50 calls."""
    done, reps = 0.0, 1
    while done < SETTLE_MS:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        done += e0.elapsed_time(e1)
        reps *= 2


def _events_ms(torch, stream, fn, warmup, steps):
    _settle(torch, stream, fn)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _rate(nbytes, ms):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "GBps": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "bytes": int(nbytes)}


def _l1(r, nbytes):
    """Adds the vector L1 bytes the kernel's loads request and their rate
    against the vL1D ceiling to a result line."""
    gbs = nbytes / (r["ms"] * 1e-3) / 1e9
    r["vl1d_bytes"] = int(nbytes)
    r["vl1d_frac"] = round(gbs / VL1D_PEAK_GBS, 4)
    return r


def _union_tiles(ul, teams_per_group=1):
    return int(((ul.astype(np.int64) + 15) // 16).sum()) * teams_per_group


def measure_others(args, sa, torch, stream):
    """Times every other workload once (HIP events on the launch stream)."""
    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    res = {}
    w, n = 3, 10
    # union mode on the headline workload: two adjacent rows x 6 heads share
    # one 16-column tile and one gather of their union
    c = gen.make_config("C1", args.seed)
    q, k, v = bf16(c.q), bf16(c.k), bf16(c.v)
    idx = torch.from_numpy(c.idx).cuda()
    out = torch.empty((c.num_rows, c.num_q_heads, 256), dtype=torch.float32, device="cuda")
    lse = torch.empty((c.num_rows, c.num_q_heads), dtype=torch.float32, device="cuda")
    per_token_bytes = gathered_bytes(c)
    cu_q1 = torch.tensor([0, c.num_rows], dtype=torch.int32, device="cuda")
    cu_kv1 = torch.tensor([0, c.kv_len], dtype=torch.int64, device="cuda")

    # The headline with cold caches: every call reads the next of 10 copies
    # of K and V (335 MB in all, more than the 256 MB Infinity Cache), so each
    # call starts with its K/V rows in HBM only.
    copies = [(k.clone(), v.clone()) for _ in range(10)]
    turn = [0]

    def rotating():
        kk, vv = copies[turn[0] % len(copies)]
        turn[0] += 1
        sa.sparse_attn_chunk_prefill(q, kk, vv, idx, cu_q1, cu_kv1, sm_scale=c.scale, out=out,
                                     lse=lse, stream=stream)

    r = _rate(per_token_bytes, _events_ms(torch, stream, rotating, 10, 20))
    r["kv_copies"] = len(copies)
    res["headline_cold_kv"] = r
    del copies
    ws = torch.empty(sa.sparse_attn_union_workspace_bytes(c.num_rows, c.topk, 2),
                     dtype=torch.uint8, device="cuda")
    ui, ub, ul = sa.sparse_attn_union_build(idx, c.kv_len, 2, ws=ws, stream=stream)
    torch.cuda.synchronize()
    rows = int(ul.sum().item())
    ms_build = _events_ms(torch, stream, lambda: sa.sparse_attn_union_build(
        idx, c.kv_len, 2, union_idx=ui, union_bits=ub, union_len=ul, ws=ws, stream=stream), w, n)
    ms_all = _events_ms(torch, stream, lambda: sa.sparse_attn_prefill_union(
        q, k, v, idx, 2, sm_scale=c.scale, ws=ws, out=out, lse=lse, stream=stream), w, n)
    r = _rate(rows * 1024, ms_all)
    # (attention_ms = total - the public build, which also writes the lists'
    # -1 / 0 tails: a little low, as for the MLA union below)
    r.update({"union_rows": rows, "build_ms": round(ms_build, 4),
              "attention_ms": round(ms_all - ms_build, 4),
              "per_token_equivalent_GBps": round(per_token_bytes / (ms_all * 1e-3) / 1e9, 1)})
    res["gqa_union_G2_same_workload"] = r
    # The same sets with each row's slot order shuffled: the walk keeps
    # shared tokens at the same slot position in adjacent rows, which the
    # per-token path's row pairing uses; without that alignment the pairing
    # only queues, and the union path (which sorts) keeps its sharing.
    sidx = torch.from_numpy(gen.shuffle_slots(c.idx, args.seed + 1)).cuda()
    ms = _events_ms(torch, stream, lambda: sa.sparse_attn_chunk_prefill(
        q, k, v, sidx, cu_q1, cu_kv1, sm_scale=c.scale, out=out, lse=lse, stream=stream), w, n)
    r = _l1(_rate(per_token_bytes, ms),
            team_tiles(gen.shuffle_slots(c.idx, args.seed + 1), c.kv_len, 2, member=True)[0] * 16 * 1024)
    ms_u = _events_ms(torch, stream, lambda: sa.sparse_attn_prefill_union(
        q, k, v, sidx, 2, sm_scale=c.scale, ws=ws, out=out, lse=lse, stream=stream), w, n)
    r.update({"union_G2_ms": round(ms_u, 4)})
    res["shuffled_slots_same_sets"] = r

    # The indexer's top-k over the same rows (8192 x 32768 fp32 scores with
    # causal lengths, k 2051), then attention over what it selected. Its rows
    # come out in ascending position order, so shared tokens do not sit at
    # the same slot in adjacent rows; the union path, which sorts, shares
    # gathers anyway.
    tc = gen.make_config("C1topk", args.seed)
    sc = torch.from_numpy(tc.scores).cuda()
    rl = torch.from_numpy(tc.row_len).cuda()
    tidx = torch.empty((tc.scores.shape[0], tc.k), dtype=torch.int32, device="cuda")
    ms_t = _events_ms(torch, stream, lambda: sa.indexer_topk(sc, tc.k, row_len=rl, out=tidx,
                                                             stream=stream), w, n)
    score_bytes = int(np.minimum(tc.row_len, tc.scores.shape[1]).sum()) * 4
    r = _rate(score_bytes, ms_t)

    def select_then_union():
        sa.indexer_topk(sc, tc.k, row_len=rl, out=tidx, stream=stream)
        sa.sparse_attn_prefill_union(q, k, v, tidx, 2, sm_scale=c.scale, ws=ws, out=out,
                                     lse=lse, stream=stream)

    def select_then_per_token():
        sa.indexer_topk(sc, tc.k, row_len=rl, out=tidx, stream=stream)
        sa.sparse_attn_chunk_prefill(q, k, v, tidx, cu_q1, cu_kv1, sm_scale=c.scale, out=out,
                                     lse=lse, stream=stream)

    r.update({"score_bytes": score_bytes,
              "then_union_G2_ms": round(_events_ms(torch, stream, select_then_union, w, n), 4),
              "then_per_token_ms": round(_events_ms(torch, stream, select_then_per_token, w, n),
                                         4)})
    res["indexer_topk"] = r
    del q, k, v, idx, sidx, out, lse, ws, ui, ub, ul, sc, rl, tidx

    # group 12 over two KV heads, 131072-token context
    c = gen.make_config("C2", args.seed)
    q, k, v = bf16(c.q), bf16(c.k), bf16(c.v)
    idx = torch.from_numpy(c.idx).cuda()
    out = torch.empty((c.num_rows, c.num_q_heads, 256), dtype=torch.float32, device="cuda")
    lse = torch.empty((c.num_rows, c.num_q_heads), dtype=torch.float32, device="cuda")
    ms = _events_ms(torch, stream, lambda: sa.sparse_attn_prefill(
        q, k, v, idx, sm_scale=c.scale, out=out, lse=lse, stream=stream), w, n)
    res["group12_2kv_prefill"] = _l1(
        _rate(gathered_bytes(c), ms),
        team_tiles(c.idx, c.kv_len, 4, every_tile=True)[0] * 16 * 1024 * c.num_kv_heads)
    del q, k, v, idx, out, lse

    # MLA per-token and union
    c = gen.make_config("C3", args.seed)
    q, k = bf16(c.q), bf16(c.k)
    idx = torch.from_numpy(c.idx).cuda()
    out = torch.empty((c.num_rows, c.num_q_heads, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((c.num_rows, c.num_q_heads), dtype=torch.float32, device="cuda")
    per_token_bytes = gathered_bytes(c)
    ms = _events_ms(torch, stream, lambda: sa.sparse_attn_prefill(
        q, k, None, idx, sm_scale=c.scale, head_dim_v=512, out=out, lse=lse, stream=stream), w, n)
    res["mla_per_token"] = _l1(_rate(per_token_bytes, ms),
                               team_tiles(c.idx, c.kv_len, 2, member=True)[0] * 16 * 1152)
    # the same sets with every row's slots shuffled (membership teams)
    sidx = torch.from_numpy(gen.shuffle_slots(c.idx, args.seed + 1)).cuda()
    ms = _events_ms(torch, stream, lambda: sa.sparse_attn_prefill(
        q, k, None, sidx, sm_scale=c.scale, head_dim_v=512, out=out, lse=lse, stream=stream), w, n)
    res["mla_per_token_shuffled_slots"] = _rate(per_token_bytes, ms)
    del sidx
    for G in (2, 4):
        ws = torch.empty(sa.sparse_attn_union_workspace_bytes(c.num_rows, c.topk, G),
                         dtype=torch.uint8, device="cuda")
        ui, ub, ul = sa.sparse_attn_union_build(idx, c.kv_len, G, ws=ws, stream=stream)
        torch.cuda.synchronize()
        rows = int(ul.sum().item())
        ms_build = _events_ms(torch, stream, lambda: sa.sparse_attn_union_build(
            idx, c.kv_len, G, union_idx=ui, union_bits=ub, union_len=ul, ws=ws, stream=stream),
            w, n)
        ms_all = _events_ms(torch, stream, lambda: sa.sparse_attn_prefill_union(
            q, k, None, idx, G, sm_scale=c.scale, head_dim_v=512, ws=ws, out=out, lse=lse,
            stream=stream), w, n)
        r = _rate(rows * 1152, ms_all)
        # (build_ms times the public build, which also writes the -1 / 0 tail
        # of every list; the build inside the union call does not, so
        # attention_ms = total - build_ms reads about 2 % low: the kernel
        # trace gives the exact split)
        r.update({"union_rows": rows, "build_ms": round(ms_build, 4),
                  "attention_ms": round(ms_all - ms_build, 4),
                  "per_token_equivalent_GBps": round(per_token_bytes / (ms_all * 1e-3) / 1e9, 1),
                  "speedup_vs_per_token": round(res["mla_per_token"]["ms"] / ms_all, 3)})
        # (a team serves 16 / heads members of a group and streams the whole
        # list: G=4 over 8 heads has two teams per group)
        tpg = -(-G // (16 // c.num_q_heads))
        _l1(r, _union_tiles(ul.cpu().numpy(), tpg) * 16 * 1152)
        r["vl1d_bytes_per_row_gathered"] = round(r["vl1d_bytes"] / rows, 1)
        res[f"mla_union_G{G}"] = r
        del ws, ui, ub, ul
    del q, k, idx, out, lse

    # MLA over 656-byte FP8 records (dequantised to bf16 as they are staged)
    c = gen.make_config("C3fp8", args.seed)
    q = bf16(c.q)
    k = torch.from_numpy(np.ascontiguousarray(c.k)).cuda()
    idx = torch.from_numpy(c.idx).cuda()
    out = torch.empty((c.num_rows, c.num_q_heads, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((c.num_rows, c.num_q_heads), dtype=torch.float32, device="cuda")
    ms = _events_ms(torch, stream, lambda: sa.sparse_attn_prefill(
        q, k, None, idx, sm_scale=c.scale, head_dim_v=512, out=out, lse=lse, stream=stream), w, n)
    res["mla_fp8_per_token"] = _rate(gathered_bytes(c), ms)
    res["mla_fp8_per_token"]["speedup_vs_bf16"] = round(res["mla_per_token"]["ms"] / ms, 3)
    ws = torch.empty(sa.sparse_attn_union_workspace_bytes(c.num_rows, c.topk, 2),
                     dtype=torch.uint8, device="cuda")
    ms = _events_ms(torch, stream, lambda: sa.sparse_attn_prefill_union(
        q, k, None, idx, 2, sm_scale=c.scale, head_dim_v=512, ws=ws, out=out, lse=lse,
        stream=stream), w, n)
    res["mla_fp8_union_G2"] = {"ms": round(ms, 4),
                               "speedup_vs_bf16_union": round(res["mla_union_G2"]["ms"] / ms, 3)}
    # staged: convert the records to bf16 rows once per call, then the bf16
    # kernels (the same values, bit for bit). Every C3 token is touched, so
    # every row is converted; with long, sparsely touched contexts page_mark
    # over one-token pages first marks the rows to convert (timed beside).
    mask = torch.empty((c.kv_len,), dtype=torch.int8, device="cuda")
    rows = torch.empty((c.kv_len, 1, 576), dtype=torch.bfloat16, device="cuda")

    def staged(union):
        sa.fp8_records_to_bf16(k, out=rows, stream=stream)
        if union:
            sa.sparse_attn_prefill_union(q, rows, None, idx, 2, sm_scale=c.scale, head_dim_v=512,
                                         ws=ws, out=out, lse=lse, stream=stream)
        else:
            sa.sparse_attn_prefill(q, rows, None, idx, sm_scale=c.scale, head_dim_v=512,
                                   out=out, lse=lse, stream=stream)

    ms_conv = _events_ms(torch, stream, lambda: sa.fp8_records_to_bf16(k, out=rows, stream=stream),
                         w, n)
    ms_mark = _events_ms(torch, stream, lambda: (
        sa.page_mark(idx, c.kv_len, 1, mask=mask, stream=stream),
        sa.fp8_records_to_bf16(k, mask=mask, out=rows, stream=stream)), w, n)
    ms = _events_ms(torch, stream, lambda: staged(False), w, n)
    res["mla_fp8_staged_per_token"] = {
        "ms": round(ms, 4), "convert_ms": round(ms_conv, 4),
        "mark_and_masked_convert_ms": round(ms_mark, 4),
        "speedup_vs_bf16": round(res["mla_per_token"]["ms"] / ms, 3),
        "speedup_vs_in_kernel_fp8": round(res["mla_fp8_per_token"]["ms"] / ms, 3)}
    ms = _events_ms(torch, stream, lambda: staged(True), w, n)
    res["mla_fp8_staged_union_G2"] = {
        "ms": round(ms, 4), "speedup_vs_bf16_union": round(res["mla_union_G2"]["ms"] / ms, 3)}
    del mask, rows
    del q, k, idx, out, lse, ws

    # ragged chunk prefill, 16 requests
    c = gen.make_config("C4", args.seed)
    q, k, v = bf16(c.q), bf16(c.k), bf16(c.v)
    idx = torch.from_numpy(c.idx).cuda()
    cu_q = torch.from_numpy(c.cu_seqlens_q).cuda()
    cu_kv = torch.from_numpy(c.cu_seqlens_kv).cuda()
    out = torch.empty((c.num_rows, c.num_q_heads, 256), dtype=torch.float32, device="cuda")
    lse = torch.empty((c.num_rows, c.num_q_heads), dtype=torch.float32, device="cuda")
    ms = _events_ms(torch, stream, lambda: sa.sparse_attn_chunk_prefill(
        q, k, v, idx, cu_q, cu_kv, sm_scale=c.scale, out=out, lse=lse, stream=stream), w, n)
    res["ragged_chunk_prefill"] = _l1(
        _rate(gathered_bytes(c), ms),
        team_tiles(c.idx, None, 2, c.cu_seqlens_q, c.cu_seqlens_kv, member=True)[0] * 16 * 1024)
    res["ragged_chunk_prefill"]["rows"] = c.num_rows
    # union mode over the same ragged requests (groups of 2 rows per request)
    ws = torch.empty(sa.sparse_attn_chunk_union_workspace_bytes(c.num_rows, len(cu_q) - 1,
                                                                c.topk, 2),
                     dtype=torch.uint8, device="cuda")
    ms_u = _events_ms(torch, stream, lambda: sa.sparse_attn_chunk_prefill_union(
        q, k, v, idx, cu_q, cu_kv, 2, sm_scale=c.scale, ws=ws, out=out, lse=lse,
        stream=stream), w, n)
    r = _rate(gathered_bytes(c), ms_u)
    r = {"ms": r["ms"], "per_token_equivalent_GBps": r["GBps"],
         "speedup_vs_per_token": round(ms / ms_u, 3)}
    res["ragged_chunk_prefill_union_G2"] = r
    del q, k, v, idx, out, lse, ws

    # decode page mark + masked split vs full split
    c = gen.make_config("C4decode", args.seed)
    src = torch.from_numpy(c.src).cuda()
    dst = torch.full((c.num_src_pages * c.ratio, c.dst_page_bytes), 0xA5, dtype=torch.uint8,
                     device="cuda")
    didx = torch.from_numpy(c.idx).cuda()
    mask = torch.empty((c.num_src_pages,), dtype=torch.int8, device="cuda")
    geom = dict(src_page_tokens=c.src_page_tokens, dst_page_tokens=c.dst_page_tokens,
                row_bytes=c.row_bytes, scale_bytes=c.scale_bytes, stream=stream)
    sa.page_mark(didx, c.num_src_pages, c.src_page_tokens, mask=mask, stream=stream)
    torch.cuda.synchronize()
    touched = int(mask.sum().item())
    ms_mark = _events_ms(torch, stream, lambda: sa.page_mark(
        didx, c.num_src_pages, c.src_page_tokens, mask=mask, stream=stream), w, n)
    ms_split = _events_ms(torch, stream, lambda: sa.page_split(src, dst, mask, **geom), w, n)
    ms_full = _events_ms(torch, stream, lambda: sa.page_split(src, dst, None, **geom), w, n)
    page_bytes = c.src_page_bytes
    res["decode_page_split"] = {
        "touched_pages": touched, "mark_ms": round(ms_mark, 4),
        "masked_split_ms": round(ms_split, 4), "full_split_ms": round(ms_full, 4),
        "masked_GBps": round(2 * touched * page_bytes / (ms_split * 1e-3) / 1e9, 1),
        "full_GBps": round(2 * c.num_src_pages * page_bytes / (ms_full * 1e-3) / 1e9, 1),
        "full_frac_hbm_peak": round(2 * c.num_src_pages * page_bytes / (ms_full * 1e-3) / 1e9
                                    / HBM_PEAK_GBS, 4)}

    # sparse MLA decode over the split pages, and the whole decode step
    # (mark + masked split + decode); then the spread indices (2048 valid
    # slots per request, 1947 touched pages)
    def decode_lines(c, src, dst, didx, mask):
        geom = dict(src_page_tokens=c.src_page_tokens, dst_page_tokens=c.dst_page_tokens,
                    row_bytes=c.row_bytes, scale_bytes=c.scale_bytes, stream=stream)
        B, Hq, topk = c.q.shape[0], c.q.shape[1], c.idx.shape[1]
        dq = torch.from_numpy(c.q.view(np.int16)).view(torch.bfloat16).cuda()
        dws = torch.empty(sa.sparse_attn_decode_workspace_bytes(B, Hq, topk), dtype=torch.uint8,
                          device="cuda")
        dout = torch.empty((B, Hq, 512), dtype=torch.float32, device="cuda")
        dlse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")

        def decode(s=stream):
            sa.sparse_attn_decode_paged(dq, dst, didx, dst_page_tokens=c.dst_page_tokens,
                                        scale_bytes=c.scale_bytes, sm_scale=c.scale, ws=dws,
                                        out=dout, lse=dlse, stream=s)

        def step(s=stream):
            sa.page_mark(didx, c.num_src_pages, c.src_page_tokens, mask=mask, stream=s)
            sa.page_split(src, dst, mask, **{**geom, "stream": s})
            decode(s)

        step()
        ms_dec = _events_ms(torch, stream, decode, w, n)
        ms_step = _events_ms(torch, stream, step, w, n)
        # the same step (five kernel launches) captured once in a HIP graph
        # and replayed: what a serving loop pays per step without the host's
        # per-launch cost (the calls launch on the capture stream)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(None)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(None)
        ms_graph = _events_ms(torch, stream, graph.replay, w, n)
        valid = int(((c.idx >= 0) & (c.idx < c.num_src_pages * c.src_page_tokens)).sum())
        r = _rate(valid * FP8_RECORD_BYTES, ms_dec)
        r.update({"valid_slots": valid, "step_ms": round(ms_step, 4),
                  "step_graph_ms": round(ms_graph, 4)})
        return r

    res["decode_attention"] = decode_lines(c, src, dst, didx, mask)
    del src, dst
    c = gen.make_config("C4spread", args.seed)
    src = torch.from_numpy(c.src).cuda()
    dst = torch.full((c.num_src_pages * c.ratio, c.dst_page_bytes), 0xA5, dtype=torch.uint8,
                     device="cuda")
    didx = torch.from_numpy(c.idx).cuda()
    res["decode_attention_spread"] = decode_lines(c, src, dst, didx, mask)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # 100 calls (about 40 ms of the headline) bring the GPU to its steady
    # clocks before the timed calls (see _settle)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle-ms", type=float, default=40.0,
                    help="GPU time each of the other workloads runs untimed before its warm-up "
                         "calls (0: none, e.g. under counter collection)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on",
                    help="off for profiler runs (the profiler initialises the GPU before "
                         "the program, so no worker processes may be forked)")
    ap.add_argument("--cpu-stride", type=int, default=1)
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (to scale HBM counters)")
    ap.add_argument("--others", choices=["on", "off"], default="on",
                    help="also time the other workloads (group-12 prefill, MLA per-token "
                         "and union, ragged chunk prefill, decode page mark/split)")
    args = ap.parse_args()
    global SETTLE_MS
    SETTLE_MS = args.settle_ms

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(query rows and KV heads would shard across GPUs with no exchange). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        import torch
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n}))
        return

    case = gen.make_config("C1", args.seed)
    nbytes = gathered_bytes(case)

    cpu, cpu_out = None, None
    if args.cpu_baseline == "on":
        workers = max(1, min(16, len(os.sched_getaffinity(0))))
        cpu, cpu_out = cpu_baseline(case, args.cpu_stride, workers)

    import torch
    import top_index_sparse_amd as sa

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v = bf16(case.q), bf16(case.k), bf16(case.v)
    idx = torch.from_numpy(case.idx).cuda()
    cu_q = torch.tensor([0, case.num_rows], dtype=torch.int32, device="cuda")
    cu_kv = torch.tensor([0, case.kv_len], dtype=torch.int64, device="cuda")
    out = torch.empty((case.num_rows, case.num_q_heads, case.head_dim_v), dtype=torch.float32,
                      device="cuda")
    lse = torch.empty((case.num_rows, case.num_q_heads), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        sa.sparse_attn_chunk_prefill(q, k, v, idx, cu_q, cu_kv, total_q=case.num_rows,
                                     sm_scale=case.scale, out=out, lse=lse, stream=stream)

    # the pages' protocol: clocks settled, warm-up calls, then every timed
    # call bracketed by events on the launch stream (median and mean)
    _settle(torch, stream, step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    calls0 = sa.sa_call_count("sparse_attn_chunk_prefill")
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert sa.sa_call_count("sparse_attn_chunk_prefill") - calls0 == args.steps
    per_call = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    kernel_ms = evs[0].elapsed_time(evs[-1]) / args.steps
    kernel_ms_median = float(np.median(per_call))
    ms = wall * 1e3 / args.steps

    parity = None
    if cpu_out is not None:
        rows, ro, rl = cpu_out
        sel = torch.from_numpy(rows).cuda()
        go = out[sel].cpu().numpy().astype(np.float64)
        gl = lse[sel].cpu().numpy().astype(np.float64)
        err = np.abs(go - ro)
        ok = bool(np.all(err <= 2e-2 + 1e-2 * np.abs(ro)) and np.abs(gl - rl).max() <= 1e-5)
        parity = {"rows_checked": int(len(rows)), "max_abs_err_out": float(err.max()),
                  "max_abs_err_lse": float(np.abs(gl - rl).max()), "pass": ok}
        if not ok:
            print(json.dumps({"parity": parity}), file=sys.stderr)
            sys.exit(1)

    others = measure_others(args, sa, torch, stream) if args.others == "on" else None

    # A plain 1 GiB device copy on the same stream: the HBM rate this part
    # reaches in practice, beside the 8 TB/s of the data sheet.
    csrc = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    cdst = torch.empty_like(csrc)
    copy_ms = _events_ms(torch, stream, lambda: cdst.copy_(csrc), 3, 10)
    copy_gbs = 2.0 * (1 << 30) / (copy_ms * 1e-3) / 1e9
    del csrc, cdst

    # The gather stream alone (sa_probe_gather: the same 16-byte K/V row
    # reads through the same descriptors, one index row per wave, no
    # arithmetic) over the same index rows: the rate this access pattern
    # sustains on the device, at the kernel's eight waves per CU and at as
    # many waves as the probe's registers allow.
    probe_out = torch.empty((case.num_rows, 64), dtype=torch.int32, device="cuda")
    probe = {}
    ptiles = case.num_rows * ((case.topk + 15) // 16)
    k2, v2 = k.view(case.kv_len, case.head_dim_qk), v.view(case.kv_len, case.head_dim_v)   # one KV head
    for name, eight in (("eight_waves_per_cu", True), ("max_waves_per_cu", False)):
        pms = _events_ms(torch, stream, lambda e=eight: sa.probe_gather(
            k2, v2, idx, eight_waves=e, out=probe_out, stream=stream), 5, 20)
        probe[name] = round(ptiles * 16 * 1024 / (pms * 1e-3) / 1e9, 1)
    probe_gbs = max(probe.values())
    del probe_out

    # The vector L1 bytes the kernel's loads request: every slot tile a team
    # issues loads 16 K rows and 16 V rows (512 B each; invalid slots read a
    # cached row of zeros). Two rows x 6 heads share one 16-column tile.
    tiles, rows_gathered = team_tiles(case.idx, case.kv_len, 2, member=True)
    l1_bytes = tiles * 16 * 1024 * case.num_kv_heads
    l1_gbs = l1_bytes / (kernel_ms * 1e-3) / 1e9
    # Issued MFMA work per tile: S^T over 8 k-steps of 16x16x32 and O^T over
    # 16 d-blocks of 16x16x16, one 16-column tile.
    mfma_flops = tiles * (8 * 2 * 16 * 16 * 32 + 16 * 2 * 16 * 16 * 16)
    valid_slots = nbytes // 1024
    tflops = 2.0 * case.num_q_heads * valid_slots * (case.head_dim_qk + case.head_dim_v) \
        / (kernel_ms * 1e-3) / 1e12
    counters = load_counters()
    traffic = counters.get("hbm_bytes_per_call") if counters else None
    result = {
        "metric": METRIC,
        "value": round(nbytes / (ms * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "sparse GQA chunk prefill: 8192 query rows at the end of a "
                        "32768-token context, top-k 2051 random-walk indices, 6 query "
                        "heads over 1 KV head, head dim 256, bf16 in, fp32 out + LSE",
            "rows": case.num_rows, "topk": case.topk, "kv_len": case.kv_len,
            "num_q_heads": case.num_q_heads, "num_kv_heads": case.num_kv_heads,
            "head_dim": case.head_dim_qk, "seed": args.seed,
            "gathered_bytes_per_call": nbytes,
        },
        "roofline": {
            "bound": "vl1d", "achieved": round(l1_gbs, 1), "peak": round(VL1D_PEAK_GBS, 1),
            "unit": "GB/s", "frac": round(l1_gbs / VL1D_PEAK_GBS, 4), "traffic": traffic,
            "bytes_per_call": l1_bytes, "tiles_per_call": tiles,
            "valid_rows_gathered_per_call": rows_gathered,
            "hbm_frac": (round(traffic / (kernel_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                         if traffic else None),
            "mfma_issued_frac": round(mfma_flops / (kernel_ms * 1e-3) / 1e12
                                      / MFMA_BF16_PEAK_TFLOPS, 4),
            "gather_probe_GBps": probe,
            "frac_of_gather_probe": round(l1_gbs / probe_gbs, 4),
        },
        "cpu_baseline": cpu,
        "kernel_ms": round(kernel_ms, 4),
        "kernel_ms_median": round(kernel_ms_median, 4),
        "gathered_frac_hbm_peak": round(nbytes / (kernel_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "tflops_useful": round(tflops, 2),
        "copy_probe_GBps": round(copy_gbs, 1),
        "counters": counters,
        "parity": parity,
        "others": others,
    }
    print(json.dumps(result))


if __name__ == "__main__":
    main()
