"""GPU: the entry points inside a captured HIP graph. Union prefill (build +
attention), the decode chain (page mark, masked split, decode), the indexer
top-k and ragged chunk prefill are captured once; the graph is replayed with
new inputs copied in between, with eager work and synchronisation between
the replays, and every replay must equal an eager run on the same inputs
bit for bit (the kernels are deterministic)."""
import numpy as np
import pytest
import torch

import gen
import top_index_sparse_amd as sa
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _bits_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def _inputs(seed):
    """Host arrays for one replay: an MLA union case, a decode pool step,
    top-k scores and a ragged GQA case."""
    rng = np.random.default_rng(seed)
    mla = gen.make_attn_case("g", seed=seed, num_rows=37, kv_len=300, first_pos=263,
                             num_q_heads=8, num_kv_heads=1, head_dim_qk=576, head_dim_v=512,
                             topk=128, v_in_k=True)
    pages = gen.make_page_case("g", seed=seed, num_src_pages=16, batch=4, topk=96, window=80)
    scores = rng.standard_normal((24, 5000)).astype(np.float32)
    row_len = rng.integers(0, 5200, 24).astype(np.int32)
    # ragged lengths come from a fixed seed (the graph's shapes are fixed);
    # each replay draws new values
    ragged = gen.make_ragged_case("g", seed=100, num_reqs=3, qlen_range=(5, 20),
                                  ctx_range=(40, 90), num_q_heads=6, num_kv_heads=1,
                                  head_dim=256, topk=48)
    ragged.q = gen.normal_bf16(rng, ragged.q.shape)
    ragged.k = gen.normal_bf16(rng, ragged.k.shape)
    ragged.v = gen.normal_bf16(rng, ragged.v.shape)
    return mla, pages, scores, row_len, ragged


class Bufs:
    """Static device tensors the graph reads and writes."""

    def __init__(self, host):
        mla, pages, scores, row_len, ragged = host
        dev = "cuda"
        self.mq = _bits_bf16(mla.q).to(dev)
        self.mk = _bits_bf16(mla.k).to(dev)
        self.midx = torch.from_numpy(mla.idx).to(dev)
        self.mws = torch.empty(sa.sparse_attn_union_workspace_bytes(37, 128, 2), dtype=torch.uint8,
                               device=dev)
        self.mo = torch.empty((37, 8, 512), dtype=torch.float32, device=dev)
        self.ml = torch.empty((37, 8), dtype=torch.float32, device=dev)
        self.src = torch.from_numpy(pages.src).to(dev)
        self.dst = torch.full((16 * 4, pages.dst_page_bytes), 0xA5, dtype=torch.uint8, device=dev)
        self.pidx = torch.from_numpy(pages.idx).to(dev)
        self.mask = torch.empty((16,), dtype=torch.int8, device=dev)
        self.dq = _bits_bf16(pages.q).to(dev)
        self.dws = torch.empty(sa.sparse_attn_decode_workspace_bytes(4, 8, 96), dtype=torch.uint8,
                               device=dev)
        self.do = torch.empty((4, 8, 512), dtype=torch.float32, device=dev)
        self.dl = torch.empty((4, 8), dtype=torch.float32, device=dev)
        self.sc = torch.from_numpy(scores).to(dev)
        self.rl = torch.from_numpy(row_len).to(dev)
        self.tk = torch.empty((24, 300), dtype=torch.int32, device=dev)
        self.rq = _bits_bf16(ragged.q).to(dev)
        self.rk = _bits_bf16(ragged.k).to(dev)
        self.rv = _bits_bf16(ragged.v).to(dev)
        self.ridx = torch.from_numpy(ragged.idx).to(dev)
        self.cuq = torch.from_numpy(ragged.cu_seqlens_q).to(dev)
        self.cukv = torch.from_numpy(ragged.cu_seqlens_kv).to(dev)
        self.ro = torch.empty((ragged.num_rows, 6, 256), dtype=torch.float32, device=dev)
        self.rlse = torch.empty((ragged.num_rows, 6), dtype=torch.float32, device=dev)
        self.geom = dict(src_page_tokens=256, dst_page_tokens=64, row_bytes=656, scale_bytes=4)

    def load(self, host):
        """Copies a new replay's inputs into the static tensors (same shapes)."""
        mla, pages, scores, row_len, ragged = host
        self.mq.copy_(_bits_bf16(mla.q))
        self.mk.copy_(_bits_bf16(mla.k))
        self.midx.copy_(torch.from_numpy(mla.idx))
        self.src.copy_(torch.from_numpy(pages.src))
        self.pidx.copy_(torch.from_numpy(pages.idx))
        self.dq.copy_(_bits_bf16(pages.q))
        self.sc.copy_(torch.from_numpy(scores))
        self.rl.copy_(torch.from_numpy(row_len))
        self.rq.copy_(_bits_bf16(ragged.q))
        self.rk.copy_(_bits_bf16(ragged.k))
        self.rv.copy_(_bits_bf16(ragged.v))
        self.ridx.copy_(torch.from_numpy(ragged.idx))

    def run(self):
        _, _, st = sa.sparse_attn_prefill_union(self.mq, self.mk, None, self.midx, 2,
                                                sm_scale=1 / 24, head_dim_v=512, ws=self.mws,
                                                out=self.mo, lse=self.ml)
        assert st == sa.SA_OK
        sa.page_mark(self.pidx, 16, 256, mask=self.mask)
        sa.page_split(self.src, self.dst, self.mask, **self.geom)
        sa.sparse_attn_decode_paged(self.dq, self.dst, self.pidx, sm_scale=1 / 24, ws=self.dws,
                                    out=self.do, lse=self.dl)
        sa.indexer_topk(self.sc, 300, row_len=self.rl, out=self.tk)
        sa.sparse_attn_chunk_prefill(self.rq, self.rk, self.rv, self.ridx, self.cuq, self.cukv,
                                     sm_scale=1 / 16, out=self.ro, lse=self.rlse)

    def outputs(self):
        return [t.clone() for t in (self.mo, self.ml, self.dst, self.do, self.dl, self.tk, self.ro,
                                    self.rlse)]


def test_graph_replays_equal_eager():
    say("[graph] capture union prefill, decode chain, top-k, ragged prefill; replay x3")
    b = Bufs(_inputs(100))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        b.run()                                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        b.run()
    names = ["union O", "union LSE", "split pages", "decode O", "decode LSE", "top-k",
             "ragged O", "ragged LSE"]
    for rep in range(3):
        b.load(_inputs(101 + rep))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = b.outputs()
        b.run()                                   # eager, same inputs, same buffers
        torch.cuda.synchronize()
        want = b.outputs()
        for name, x, y in zip(names, got, want):
            assert torch.equal(x, y), f"replay {rep}: {name} differs from eager"
        say(f"  replay {rep}: all outputs equal eager")
