"""GPU: the gather-rate probe (a measurement aid the benchmark uses) reads
exactly the K/V bytes the per-token kernels gather: its per-lane checksums
match the same XOR computed with numpy, in both occupancy modes."""
import numpy as np
import pytest
import torch

import top_index_sparse_amd as sa
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _expected(k_words, v_words, idx, kv_len):
    """k_words, v_words: uint32 [kv_len, 128] (a row's 512 bytes)."""
    rows, topk = idx.shape
    out = np.zeros((rows, 64), np.uint32)
    for r in range(rows):
        for lane in range(64):
            g, m = lane // 16, lane % 16
            acc = np.uint32(0)
            for j in range(topk):
                if (j % 16) // 4 != g:
                    continue
                t = idx[r, j]
                if not 0 <= t < kv_len:
                    continue
                for h in range(2):
                    w0 = (256 * h + 16 * m) // 4
                    for src in (k_words, v_words):
                        acc ^= np.bitwise_xor.reduce(src[t, w0:w0 + 4])
            out[r, lane] = acc
    return out


def test_gather_probe_checksums():
    say("[probe] gather checksums: 37 rows x 70 slots over 1000 rows, invalid slots included")
    rng = np.random.default_rng(4)
    kv_len, rows, topk = 1000, 37, 70
    kw = rng.integers(0, 2**32, (kv_len, 128), dtype=np.uint32)
    vw = rng.integers(0, 2**32, (kv_len, 128), dtype=np.uint32)
    idx = rng.integers(-3, kv_len + 5, (rows, topk)).astype(np.int32)
    k = torch.from_numpy(kw.view(np.int16).reshape(kv_len, 256).copy()).cuda().view(torch.bfloat16)
    v = torch.from_numpy(vw.view(np.int16).reshape(kv_len, 256).copy()).cuda().view(torch.bfloat16)
    di = torch.from_numpy(idx).cuda()
    want = _expected(kw, vw, idx, kv_len)
    for eight in (True, False):
        got = sa.probe_gather(k, v, di, eight_waves=eight)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy().view(np.uint32), want), f"eight_waves={eight}"
