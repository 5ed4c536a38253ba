"""GPU: sparse_attn_decode_paged_noalloc, the decode entry point that takes
no workspace (its partial results live in the library's static per-GPU
scratch), against sparse_attn_decode_paged with a caller workspace and the
fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import gen
import oracle
import top_index_sparse_amd as sa
from tests.gpu_util import bf16_dev, check_close, i32_dev, say

pytestmark = pytest.mark.gpu


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _case(seed, B, Hq, topk, pages=512, ptok=64):
    rng = np.random.default_rng(seed)
    stride = ptok * 660
    pool = rng.integers(0, 256, size=(pages, stride), dtype=np.uint8)
    pool[:, :ptok * 656] = gen.mla_fp8_rows(rng, pages * ptok).reshape(pages, ptok * 656)
    q = gen.normal_bf16(rng, (B, Hq, 576))
    idx = rng.integers(-2, pages * ptok + 20, size=(B, topk)).astype(np.int32)
    idx[0, 5:50] = idx[0, 4]                     # duplicates count with multiplicity
    if B > 3:
        idx[3] = -1                              # a request with no valid slot
    return q, pool, idx


def _both(q, pool, idx, scale):
    dq, dp, di = bf16_dev(q), _u8(pool), i32_dev(idx)
    ro, rl = sa.sparse_attn_decode_paged(dq, dp, di, sm_scale=scale)
    out = torch.full_like(ro, float("nan"))
    lse = torch.full_like(rl, float("nan"))
    calls = sa.sa_call_count("sparse_attn_decode_paged_noalloc")
    sa.sparse_attn_decode_paged_noalloc(dq, dp, di, out=out, lse=lse, sm_scale=scale)
    torch.cuda.synchronize()
    assert sa.sa_call_count("sparse_attn_decode_paged_noalloc") == calls + 1
    return out, lse, ro, rl


def test_noalloc_matches_workspace_entry_twice_then_smaller():
    scale = 1.0 / 24
    for step, (B, Hq, topk) in enumerate([(64, 8, 2048), (9, 16, 300)]):
        say(f"[noalloc] call {step + 1}: batch {B}, {Hq} heads, topk {topk}")
        q, pool, idx = _case(100 + step, B, Hq, topk)
        out, lse, ro, rl = _both(q, pool, idx, scale)
        # the same kernels over the same inputs: bit for bit
        assert torch.equal(out, ro) and torch.equal(lse, rl)
        oo, ol = oracle.paged_decode(q, pool, idx, page_tokens=64, scale=scale)
        e, el = check_close(out, lse, oo, ol, f"noalloc call {step + 1}")
        say(f"  equal to the workspace entry; vs oracle: O {e:.2e} LSE {el:.2e}")


def test_noalloc_rejects_sizes_beyond_the_scratch():
    B, Hq, topk = 128, 8, 2048                   # 16 ranges x 2052 B per (request, head)
    need = sa.sparse_attn_decode_workspace_bytes(B, Hq, topk)
    assert need > sa.SA_DECODE_SCRATCH_BYTES
    say(f"[noalloc] batch {B} x {Hq} heads needs {need} B > {sa.SA_DECODE_SCRATCH_BYTES} B")
    q = torch.zeros((B, Hq, 576), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((8, 64 * 660), dtype=torch.uint8, device="cuda")
    idx = torch.full((B, topk), -1, dtype=torch.int32, device="cuda")
    out = torch.full((B, Hq, 512), 7.0, device="cuda")
    lse = torch.full((B, Hq), 7.0, device="cuda")
    with pytest.raises(sa.SparseAttnError) as ei:
        sa.sparse_attn_decode_paged_noalloc(q, pool, idx, out=out, lse=lse)
    assert ei.value.status == -5                 # SA_ERR_WORKSPACE, before any launch
    assert "static scratch" in sa.sa_last_error()
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all())
    # the largest batch that fits still runs
    Bmax = B - 1
    assert sa.sparse_attn_decode_workspace_bytes(Bmax, Hq, topk) <= sa.SA_DECODE_SCRATCH_BYTES
    sa.sparse_attn_decode_paged_noalloc(q[:Bmax], pool, idx[:Bmax], out=out[:Bmax],
                                        lse=lse[:Bmax])
    torch.cuda.synchronize()
    assert bool((out[:Bmax] == 0).all()) and bool(torch.isneginf(lse[:Bmax]).all())


def test_noalloc_replayed_from_a_captured_graph():
    say("[noalloc] captured in a HIP graph, replayed with new inputs and eager work between")
    B, Hq, topk, scale = 32, 8, 2048, 1.0 / 24
    q, pool, idx = _case(200, B, Hq, topk)
    dq, dp, di = bf16_dev(q), _u8(pool), i32_dev(idx)
    out = torch.empty((B, Hq, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sa.sparse_attn_decode_paged_noalloc(dq, dp, di, out=out, lse=lse, sm_scale=scale)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sa.sparse_attn_decode_paged_noalloc(dq, dp, di, out=out, lse=lse, sm_scale=scale)
    for rep in range(3):
        q2, _, idx2 = _case(300 + rep, B, Hq, topk)
        dq.copy_(bf16_dev(q2))
        di.copy_(i32_dev(idx2))
        ro, rl = sa.sparse_attn_decode_paged(dq, dp, di, sm_scale=scale)   # eager, between
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ro) and torch.equal(lse, rl), f"replay {rep}"
