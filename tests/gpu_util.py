"""Helpers for the GPU parity tests: host arrays to device tensors, the
tolerance check against the fp64 oracle, and cached workloads."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import gen

# Output tolerance, element-wise: |gpu - ref| <= ATOL + RTOL * |ref| (bf16 in,
# fp32 accumulate), and |lse_gpu - lse_ref| <= LSE_TOL absolute.
from tests.oracle_pool import ATOL, LSE_TOL, RTOL  # noqa: E402,F401


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def i32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def i64_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).cuda()


def check_close(out: torch.Tensor, lse: torch.Tensor, ref_o: np.ndarray, ref_l: np.ndarray,
                what: str = ""):
    o = out.detach().float().cpu().numpy().astype(np.float64)
    l = lse.detach().float().cpu().numpy().astype(np.float64)
    assert o.shape == ref_o.shape, (what, o.shape, ref_o.shape)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    err = np.abs(o - ref_o)
    bound = ATOL + RTOL * np.abs(ref_o)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), (
        f"{what}: O out of tolerance at {worst}: gpu {o[worst]} ref {ref_o[worst]}, "
        f"max abs err {err.max():.3e}")
    inf_ref = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(l), inf_ref), f"{what}: -inf LSE pattern differs"
    dl = np.abs(l[~inf_ref] - ref_l[~inf_ref])
    assert dl.size == 0 or dl.max() <= LSE_TOL, f"{what}: LSE max abs err {dl.max():.3e}"
    return float(err.max()), float(dl.max()) if dl.size else 0.0


@functools.lru_cache(maxsize=4)
def config(name: str, seed: int = 0):
    return gen.make_config(name, seed)


def attn_to_dev(case: gen.AttnCase):
    d = {
        "q": bf16_dev(case.q),
        "k": bf16_dev(case.k),
        "v": None if case.v is None else bf16_dev(case.v),
        "idx": i32_dev(case.idx),
    }
    if case.cu_seqlens_q is not None:
        d["cu_q"] = i32_dev(case.cu_seqlens_q)
        d["cu_kv"] = i64_dev(case.cu_seqlens_kv)
    return d


def sample_rows(T: int, n: int, seed: int = 0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    rows = set([0, 1, 2, 3, T - 1, T - 2, T // 2])
    rows.update(rng.choice(T, size=min(n, T), replace=False).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < T))
