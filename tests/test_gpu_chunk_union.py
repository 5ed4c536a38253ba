"""GPU parity: union mode over ragged requests (sparse_attn_chunk_prefill_union)
against the fp64 oracle; the union lists it builds are compared bit for bit."""
import math

import numpy as np
import pytest
import torch

import gen
import oracle
import top_index_sparse_amd as sa
from tests.gpu_util import bf16_dev, check_close, config, i32_dev, i64_dev, sample_rows, say

pytestmark = pytest.mark.gpu


def _ragged(seed, qlens, ctxs, Hq, Dqk, Dv, topk, mla=False, swap=0.02):
    rng = np.random.default_rng(seed)
    cu_q = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    cu_kv = np.concatenate([[0], np.cumsum(ctxs)]).astype(np.int64)
    T, KV = int(cu_q[-1]), int(cu_kv[-1])
    q = gen.normal_bf16(rng, (T, Hq, Dqk))
    k = gen.normal_bf16(rng, (KV, 1, Dqk))
    v = None if mla else gen.normal_bf16(rng, (KV, 1, Dv))
    parts = [gen.random_walk_indices(rng, np.arange(c - n, c), topk, swap_frac=swap)
             for n, c in zip(qlens, ctxs)]
    idx = np.concatenate(parts).astype(np.int32) if T else np.zeros((0, topk), np.int32)
    return dict(q=q, k=k, v=v, idx=idx, cu_q=cu_q, cu_kv=cu_kv, scale=1 / math.sqrt(Dqk), dv=Dv)


def _workspace_lists(ws, T, R, topk, G):
    """The union lists inside the workspace (layout of the header)."""
    groups = (T + G - 1) // G + R
    stride = (G * topk + 15) // 16 * 16
    al = lambda x: (x + 255) // 256 * 256
    idx_off = al(4 * (R + 1))
    bits_off = idx_off + al(groups * stride * 4)
    len_off = bits_off + al(groups * stride)
    b = ws.cpu().numpy()
    gstart = b[:4 * (R + 1)].view(np.int32)
    ui = b[idx_off:idx_off + groups * stride * 4].view(np.int32).reshape(groups, stride)
    ub = b[bits_off:bits_off + groups * stride].reshape(groups, stride)
    ul = b[len_off:len_off + groups * 4].view(np.int32)
    return gstart, ui, ub, ul


def _run(c, G, check_lists=True):
    dev = dict(q=bf16_dev(c["q"]), k=bf16_dev(c["k"]),
               v=None if c["v"] is None else bf16_dev(c["v"]), idx=i32_dev(c["idx"]),
               cu_q=i32_dev(c["cu_q"]), cu_kv=i64_dev(c["cu_kv"]))
    T, R, topk = c["idx"].shape[0], len(c["cu_q"]) - 1, c["idx"].shape[1]
    ws = torch.full((sa.sparse_attn_chunk_union_workspace_bytes(T, R, topk, G),), 0x5A,
                    dtype=torch.uint8, device="cuda")
    out, lse, st = sa.sparse_attn_chunk_prefill_union(dev["q"], dev["k"], dev["v"], dev["idx"],
                                                      dev["cu_q"], dev["cu_kv"], G,
                                                      sm_scale=c["scale"], head_dim_v=c["dv"],
                                                      ws=ws)
    torch.cuda.synchronize()
    ui, ub, ul, gr = oracle.chunk_union_build(c["idx"], c["cu_q"], c["cu_kv"], G)
    if st == sa.SA_OK and check_lists:
        gstart, gi, gb, gl = _workspace_lists(ws, T, R, topk, G)
        n = len(ul)
        qlens = np.diff(c["cu_q"])
        want_start = np.concatenate([[0], np.cumsum((qlens + G - 1) // G)])
        assert np.array_equal(gstart, want_start), "first group ids"
        assert np.array_equal(gl[:n], ul), "union_len"
        for g in range(n):   # (entries past union_len are not written)
            assert np.array_equal(gi[g, :ul[g]], ui[g, :ul[g]]), f"union_idx of group {g}"
            assert np.array_equal(gb[g, :ul[g]], ub[g, :ul[g]]), f"union_bits of group {g}"
    return out, lse, st, (ui, ub, ul, gr), dev


@pytest.mark.parametrize("G", [2, 3, 4])
def test_chunk_union_small_ragged(G):
    say(f"[chunk union] group 6, G={G}: empty request, short groups, request-local indices")
    c = _ragged(40 + G, [7, 0, 5, 1, 12], [300, 50, 260, 90, 400], 6, 256, 256, 120, swap=0.1)
    c["idx"][3, 5] = -1
    c["idx"][6, 7] = 10 ** 6                  # beyond its request's KV range
    out, lse, st, (ui, ub, ul, gr), _ = _run(c, G)
    assert st == sa.SA_OK
    ro, rl = oracle.chunk_union_attention(c["q"], c["k"], c["v"], ui, ub, ul, gr, c["cu_q"],
                                          c["cu_kv"], G, num_kv_heads=1, scale=c["scale"])
    check_close(out, lse, ro, rl, f"chunk union G={G}")


@pytest.mark.parametrize("R", [256, 300])
def test_chunk_union_many_requests(R):
    # the build stages up to 256 requests' first group ids in LDS and
    # searches the rest in global memory: both sides of that limit
    say(f"[chunk union] {R} small requests, G=2")
    rng = np.random.default_rng(R)
    qlens = rng.integers(0, 5, R)
    ctxs = rng.integers(6, 40, R)
    c = _ragged(R, list(qlens), list(ctxs), 6, 256, 256, 8, swap=0.3)
    out, lse, st, (ui, ub, ul, gr), _ = _run(c, 2)
    assert st == sa.SA_OK
    ro, rl = oracle.chunk_union_attention(c["q"], c["k"], c["v"], ui, ub, ul, gr, c["cu_q"],
                                          c["cu_kv"], 2, num_kv_heads=1, scale=c["scale"])
    check_close(out, lse, ro, rl, f"chunk union {R} requests")


def test_chunk_union_long_context_chunked_planes():
    # ragged builds keep 16 KB of bit planes: 32768 tokens per chunk at G = 4,
    # so a 300000-token request takes ten chunks; indices spread over it all
    say("[chunk union] 300000-token request, ten bit-plane chunks")
    rng = np.random.default_rng(44)
    c = _ragged(44, [6, 9], [300000, 1000], 4, 256, 256, 64)
    for t in range(6):
        c["idx"][t] = rng.choice(300000, size=64, replace=False)
    c["idx"][1, :20] = c["idx"][0, :20]
    out, lse, st, (ui, ub, ul, gr), _ = _run(c, 4)
    assert st == sa.SA_OK
    ro, rl = oracle.chunk_union_attention(c["q"], c["k"], c["v"], ui, ub, ul, gr, c["cu_q"],
                                          c["cu_kv"], 4, num_kv_heads=1, scale=c["scale"])
    check_close(out, lse, ro, rl, "chunk union long")


@pytest.mark.parametrize("G", [2, 4])
def test_chunk_union_mla(G):
    say(f"[chunk union] MLA 576/512, 8 heads, G={G}")
    c = _ragged(50 + G, [9, 4, 13], [700, 300, 1200], 8, 576, 512, 256, mla=True)
    out, lse, st, (ui, ub, ul, gr), _ = _run(c, G)
    assert st == sa.SA_OK
    ro, rl = oracle.chunk_union_attention(c["q"], c["k"], None, ui, ub, ul, gr, c["cu_q"],
                                          c["cu_kv"], G, num_kv_heads=1, scale=c["scale"],
                                          head_dim_v=512)
    check_close(out, lse, ro, rl, f"chunk union MLA G={G}")


def test_chunk_union_fallback():
    say("[chunk union] group 12, G=4: illegal tile -> per-token result")
    c = _ragged(60, [5, 6], [200, 300], 12, 256, 256, 80)
    out, lse, st, _, dev = _run(c, 4, check_lists=False)
    assert st == sa.SA_OK_FALLBACK
    ro, rl = oracle.chunk_prefill(c["q"], c["k"], c["v"], c["idx"], c["cu_q"], c["cu_kv"],
                                  num_kv_heads=1, scale=c["scale"])
    check_close(out, lse, ro, rl, "chunk union fallback")


def test_chunk_union_c4_sampled_and_equal_to_per_token():
    say("[chunk union] C4 full size, G=2: sampled rows vs oracle, all rows vs per-token")
    c4 = config("C4")
    c = dict(q=c4.q, k=c4.k, v=c4.v, idx=c4.idx, cu_q=c4.cu_seqlens_q, cu_kv=c4.cu_seqlens_kv,
             scale=c4.scale, dv=256)
    out, lse, st, (ui, ub, ul, gr), dev = _run(c, 2)
    assert st == sa.SA_OK
    rows = sample_rows(c4.num_rows, 24)
    ro, rl = oracle.chunk_union_attention(c4.q, c4.k, c4.v, ui, ub, ul, gr, c4.cu_seqlens_q,
                                          c4.cu_seqlens_kv, 2, num_kv_heads=1, scale=c4.scale,
                                          rows=rows)
    sel = torch.from_numpy(rows).cuda()
    check_close(out[sel], lse[sel], ro, rl, "C4 chunk union")
    po, pl = sa.sparse_attn_chunk_prefill(dev["q"], dev["k"], dev["v"], dev["idx"], dev["cu_q"],
                                          dev["cu_kv"], sm_scale=c4.scale)
    torch.cuda.synchronize()
    dl = (lse - pl).abs().max().item()
    say(f"  C4 union vs per-token: max |dLSE| {dl:.2e}")
    assert dl < 2e-5
    assert ((out - po).abs() <= 2e-2 + 1e-2 * po.abs()).all()
