"""GPU parity: per-token sparse prefill and ragged chunk prefill through the
C ABI against the fp64 oracle, element by element."""
import math

import numpy as np
import pytest
import torch

import gen
import oracle
import top_index_sparse_amd as sa
from tests.gpu_util import (attn_to_dev, bf16_dev, check_close, config, i32_dev, i64_dev,
                            sample_rows, say)

pytestmark = pytest.mark.gpu


def _run_prefill(case, dev, rows=None, **kw):
    out, lse = sa.sparse_attn_prefill(dev["q"], dev["k"], dev["v"], dev["idx"],
                                      sm_scale=case.scale, kv_len=case.kv_len,
                                      head_dim_v=case.head_dim_v, **kw)
    torch.cuda.synchronize()
    return out, lse


def _oracle(case, rows=None, idx=None, topk_len=None):
    return oracle.sparse_attention(case.q, case.k, case.v, case.idx if idx is None else idx,
                                   num_kv_heads=case.num_kv_heads, scale=case.scale,
                                   kv_len=case.kv_len, head_dim_v=case.head_dim_v,
                                   topk_len=topk_len, rows=rows)


@pytest.mark.parametrize("name", ["C0a", "C0b"])
def test_tiny_config_all_rows(name):
    say(f"[prefill] {name}")
    case = config(name)
    dev = attn_to_dev(case)
    out, lse = _run_prefill(case, dev)
    ro, rl = _oracle(case)
    e, el = check_close(out, lse, ro, rl, name)
    say(f"  max abs err O {e:.2e}  LSE {el:.2e}")


def _small(seed, T, kv, first, Hq, Hkv, topk, walk=True):
    return gen.make_attn_case("small", seed=seed, num_rows=T, kv_len=kv, first_pos=first,
                              num_q_heads=Hq, num_kv_heads=Hkv, head_dim_qk=256,
                              head_dim_v=256, topk=topk, walk=walk)


@pytest.mark.parametrize("Hq,Hkv", [(6, 1), (12, 1), (24, 2), (1, 1), (16, 1), (9, 3), (4, 2),
                                    (20, 1), (32, 1), (50, 2), (64, 2)])
def test_groups_and_ragged_tail_tile(Hq, Hkv):
    # 2051 = 128 * 16 + 3 slots: a 3-slot tail tile; 37 rows: 4-row groups with a tail
    say(f"[prefill] group {Hq // Hkv} x {Hkv} KV heads, topk 2051")
    case = _small(11, 37, 3000, 2900, Hq, Hkv, 2051)
    dev = attn_to_dev(case)
    out, lse = _run_prefill(case, dev)
    ro, rl = _oracle(case)
    check_close(out, lse, ro, rl, f"group {Hq}/{Hkv}")


def test_invalid_slots_anywhere():
    say("[prefill] -1, out-of-range, duplicates, all-invalid row, single slot")
    case = _small(12, 21, 700, 650, 6, 1, 100)
    idx = case.idx.copy()
    rng = np.random.default_rng(5)
    holes = rng.random(idx.shape) < 0.3
    idx[holes] = -1
    idx[1, ::3] = 700                      # == kv_len: out of range
    idx[2, ::5] = 10 ** 9
    idx[3, ::7] = -(10 ** 9)
    idx[4, :] = -1                         # empty support
    idx[5, :] = -1
    idx[5, 57] = 123                       # one valid slot
    idx[6, 10:40] = idx[6, 9]              # duplicates count with multiplicity
    idx[7, :95] = -1                       # only the tail tile is valid
    case.idx = idx
    dev = attn_to_dev(case)
    out, lse = _run_prefill(case, dev)
    ro, rl = _oracle(case)
    check_close(out, lse, ro, rl, "invalid slots")
    assert torch.all(out[4] == 0) and torch.all(torch.isneginf(lse[4]))


def test_topk_len_hint():
    say("[prefill] topk_len")
    case = _small(13, 17, 900, 880, 6, 1, 300)
    tl = np.random.default_rng(3).integers(-2, 320, size=17).astype(np.int32)
    dev = attn_to_dev(case)
    out, lse = _run_prefill(case, dev, topk_len=i32_dev(tl))
    ro, rl = _oracle(case, topk_len=tl)
    check_close(out, lse, ro, rl, "topk_len")


def test_kv_len_smaller_than_buffer():
    say("[prefill] kv_len < buffer rows")
    case = _small(14, 9, 500, 480, 6, 1, 64, walk=False)
    dev = attn_to_dev(case)
    case.kv_len = 300
    out, lse = _run_prefill(case, dev)
    ro, rl = _oracle(case)
    check_close(out, lse, ro, rl, "kv_len")


@pytest.mark.parametrize("mla", [False, True])
def test_row_stride_past_descriptor_field(mla):
    # K rows 16,400 bytes apart (past the 14-bit stride of a buffer
    # descriptor): the gathers take 64-bit addresses; same results
    say(f"[prefill] K row stride 8200 elements, {'MLA' if mla else 'GQA'}")
    if mla:
        case = gen.make_attn_case("small", seed=19, num_rows=21, kv_len=700, first_pos=680,
                                  num_q_heads=8, num_kv_heads=1, head_dim_qk=576,
                                  head_dim_v=512, topk=300, v_in_k=True, walk=True)
    else:
        case = _small(19, 21, 700, 680, 12, 1, 300)
    dqk = case.head_dim_qk
    dev = attn_to_dev(case)
    kp = torch.zeros((case.kv_len, 8200), dtype=torch.bfloat16, device="cuda")
    kp[:, :dqk] = dev["k"].reshape(case.kv_len, dqk)
    kw = kp[:, :dqk].view(case.kv_len, 1, dqk)
    if mla:
        out, lse = sa.sparse_attn_prefill(dev["q"], kw, None, dev["idx"], sm_scale=case.scale,
                                          head_dim_v=case.head_dim_v)
    else:
        vp = torch.zeros((case.kv_len, 8200), dtype=torch.bfloat16, device="cuda")
        vp[:, :256] = dev["v"].reshape(case.kv_len, 256)
        out, lse = sa.sparse_attn_prefill(dev["q"], kw, vp[:, :256].view(case.kv_len, 1, 256),
                                          dev["idx"], sm_scale=case.scale)
    torch.cuda.synchronize()
    ro, rl = _oracle(case)
    check_close(out, lse, ro, rl, "wide stride")
    # the descriptor gathers (contiguous K) feed the same operands in the same
    # order (MLA: V from the gathered registers there, read back from the
    # staged slice here), so the two paths agree bit for bit
    if mla:
        o2, l2 = sa.sparse_attn_prefill(dev["q"], dev["k"], None, dev["idx"], sm_scale=case.scale,
                                        head_dim_v=case.head_dim_v)
    else:
        o2, l2 = sa.sparse_attn_prefill(dev["q"], dev["k"], dev["v"], dev["idx"], sm_scale=case.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2), "64-bit and descriptor gathers differ"


def test_strided_rows_and_full_overwrite():
    say("[prefill] padded row strides, NaN-poisoned outputs, guard bands")
    case = _small(15, 13, 800, 780, 12, 1, 200)
    q = bf16_dev(case.q)
    k = bf16_dev(case.k)
    v = bf16_dev(case.v)
    qp = torch.zeros((13, 12 * 256 + 64), dtype=torch.bfloat16, device="cuda")
    qp[:, :12 * 256] = q.reshape(13, -1)
    qv = qp[:, :12 * 256].view(13, 12, 256)
    kp = torch.zeros((800, 256 + 8), dtype=torch.bfloat16, device="cuda")
    kp[:, :256] = k.reshape(800, 256)
    vp = torch.zeros((800, 256 + 24), dtype=torch.bfloat16, device="cuda")
    vp[:, :256] = v.reshape(800, 256)
    ip = torch.full((13, 256), -7, dtype=torch.int32, device="cuda")
    ip[:, :200] = i32_dev(case.idx)
    guard = 4096
    obuf = torch.full((guard * 2 + 13 * (12 * 256 + 4),), float("nan"), device="cuda")
    out = obuf[guard:guard + 13 * (12 * 256 + 4)].view(13, 12 * 256 + 4)[:, :12 * 256].view(13, 12, 256)
    lbuf = torch.full((guard * 2 + 13 * 12,), float("nan"), device="cuda")
    lse = lbuf[guard:guard + 13 * 12].view(13, 12)
    sa.sparse_attn_prefill(qv, kp[:, :256].view(800, 1, 256), vp[:, :256].view(800, 1, 256),
                           ip[:, :200], sm_scale=case.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    ro, rl = _oracle(case)
    check_close(out, lse, ro, rl, "strided")
    assert torch.isnan(obuf[:guard]).all() and torch.isnan(obuf[-guard:]).all()
    pad = obuf[guard:guard + 13 * (12 * 256 + 4)].view(13, -1)[:, 12 * 256:]
    assert torch.isnan(pad).all(), "row padding of out must not be written"
    assert torch.isnan(lbuf[:guard]).all() and torch.isnan(lbuf[-guard:]).all()


def test_side_stream_and_bitwise_replay():
    say("[prefill] side stream + replay")
    case = config("C0b")
    dev = attn_to_dev(case)
    o1, l1 = _run_prefill(case, dev)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o2, l2 = sa.sparse_attn_prefill(dev["q"], dev["k"], dev["v"], dev["idx"],
                                        sm_scale=case.scale, stream=s)
    s.synchronize()
    o3, l3 = _run_prefill(case, dev)
    assert torch.equal(o1, o2) and torch.equal(o1, o3)
    assert torch.equal(l1, l2) and torch.equal(l1, l3)


def test_call_counter_counts():
    case = config("C0a")
    dev = attn_to_dev(case)
    before = sa.sa_call_count("sparse_attn_prefill")
    _run_prefill(case, dev)
    assert sa.sa_call_count("sparse_attn_prefill") == before + 1


@pytest.mark.parametrize("name,nrows", [("C1", 48), ("C2", 24)])
def test_full_size_sampled(name, nrows):
    say(f"[prefill] {name} full size, sampled rows")
    case = config(name)
    dev = attn_to_dev(case)
    out, lse = _run_prefill(case, dev)
    rows = sample_rows(case.num_rows, nrows)
    ro, rl = _oracle(case, rows=rows)
    e, el = check_close(out[torch.from_numpy(rows).cuda()], lse[torch.from_numpy(rows).cuda()],
                        ro, rl, name)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    say(f"  {name}: max abs err O {e:.2e}  LSE {el:.2e} over {len(rows)} rows")


def test_c1_through_chunk_prefill_equals_prefill():
    say("[chunk] C1 as one request == prefill, bitwise")
    case = config("C1")
    dev = attn_to_dev(case)
    o1, l1 = _run_prefill(case, dev)
    cu_q = i32_dev(np.array([0, case.num_rows]))
    cu_kv = i64_dev(np.array([0, case.kv_len]))
    o2, l2 = sa.sparse_attn_chunk_prefill(dev["q"], dev["k"], dev["v"], dev["idx"], cu_q, cu_kv,
                                          sm_scale=case.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _chunk(case, dev):
    out, lse = sa.sparse_attn_chunk_prefill(dev["q"], dev["k"], dev["v"], dev["idx"],
                                            dev["cu_q"], dev["cu_kv"], sm_scale=case.scale)
    torch.cuda.synchronize()
    return out, lse


def test_chunk_prefill_small_ragged():
    say("[chunk] small ragged batch with empty requests")
    case = gen.make_ragged_case("r", seed=21, num_reqs=6, qlen_range=(1, 40),
                                ctx_range=(100, 600), num_q_heads=6, num_kv_heads=1,
                                head_dim=256, topk=130)
    # make requests 1 and 4 empty
    qlens = np.diff(case.cu_seqlens_q)
    keep = np.ones(case.num_rows, bool)
    keep[case.cu_seqlens_q[1]:case.cu_seqlens_q[2]] = False
    keep[case.cu_seqlens_q[4]:case.cu_seqlens_q[5]] = False
    qlens[[1, 4]] = 0
    case.q, case.idx, case.positions = case.q[keep], case.idx[keep], case.positions[keep]
    case.cu_seqlens_q = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    dev = attn_to_dev(case)
    out, lse = _chunk(case, dev)
    ro, rl = oracle.chunk_prefill(case.q, case.k, case.v, case.idx, case.cu_seqlens_q,
                                  case.cu_seqlens_kv, num_kv_heads=1, scale=case.scale)
    check_close(out, lse, ro, rl, "ragged small")


def test_chunk_prefill_ragged_group_32():
    say("[chunk] ragged batch, 32 query heads over one KV head (one row per team)")
    case = gen.make_ragged_case("r32", seed=23, num_reqs=4, qlen_range=(3, 30),
                                ctx_range=(200, 700), num_q_heads=32, num_kv_heads=1,
                                head_dim=256, topk=150)
    dev = attn_to_dev(case)
    out, lse = _chunk(case, dev)
    ro, rl = oracle.chunk_prefill(case.q, case.k, case.v, case.idx, case.cu_seqlens_q,
                                  case.cu_seqlens_kv, num_kv_heads=1, scale=case.scale)
    check_close(out, lse, ro, rl, "ragged group 32")


def test_chunk_prefill_c4_sampled():
    say("[chunk] C4 full size, sampled rows")
    case = config("C4")
    dev = attn_to_dev(case)
    out, lse = _chunk(case, dev)
    rows = sample_rows(case.num_rows, 48)
    # include each request's first and last row
    rows = np.unique(np.concatenate([rows, case.cu_seqlens_q[:-1], case.cu_seqlens_q[1:] - 1]))
    ro, rl = oracle.chunk_prefill(case.q, case.k, case.v, case.idx, case.cu_seqlens_q,
                                  case.cu_seqlens_kv, num_kv_heads=1, scale=case.scale, rows=rows)
    sel = torch.from_numpy(rows).cuda()
    e, el = check_close(out[sel], lse[sel], ro, rl, "C4")
    assert torch.isfinite(out).all()
    say(f"  C4: max abs err O {e:.2e}  LSE {el:.2e} over {len(rows)} rows")


def test_paired_rows_with_disjoint_positions():
    say("[prefill] row pairs: same sets at shifted positions, cross-position duplicates")
    case = _small(16, 24, 1500, 1400, 6, 1, 200)
    idx = case.idx.copy()
    for t in range(1, 24, 2):
        idx[t] = np.roll(idx[t - 1], 7)            # same set, no position matches
    idx[3, :50] = idx[2, 100:150]                  # matches at other positions only
    idx[5, ::2] = idx[4, ::2]                      # half the positions match
    idx[5, 1::2] = -1
    idx[7, :] = idx[6, :]                          # identical rows
    idx[9, 10:30] = idx[9, 9]                      # duplicates inside the second row
    idx[11] = -1                                   # empty second row
    case.idx = idx
    dev = attn_to_dev(case)
    out, lse = _run_prefill(case, dev)
    ro, rl = _oracle(case)
    check_close(out, lse, ro, rl, "paired positions")
    cu_q = i32_dev(np.array([0, 5, 5, 24]))        # pairs that straddle requests
    cu_kv = i64_dev(np.array([0, 1500, 1500, 3000]))
    k2 = torch.cat([dev["k"], dev["k"]])
    v2 = torch.cat([dev["v"], dev["v"]])
    o2, l2 = sa.sparse_attn_chunk_prefill(dev["q"], k2, v2, dev["idx"], cu_q, cu_kv,
                                          sm_scale=case.scale)
    torch.cuda.synchronize()
    check_close(o2, l2, ro, rl, "paired ragged")


@pytest.mark.parametrize("Hq", [6, 3, 12, 16])
def test_team_rows_position_sharing(Hq):
    # Teams of consecutive rows share slot positions: 16 / group rows for
    # group <= 8, up to four rows over three 16-column tiles above that.
    say(f"[prefill] team rows, group {Hq}: runs, gaps, realignments, straddled requests")
    case = _small(17, 24, 1500, 1400, Hq, 1, 160)
    idx = case.idx.copy()
    rng = np.random.default_rng(8)
    fresh = lambda k: rng.choice(np.arange(1400), size=k, replace=False).astype(np.int32)
    idx[1] = idx[0]
    idx[1, 5:35] = fresh(30)                       # a run of new tokens over rows 1-2
    idx[2] = idx[1]
    idx[3] = idx[0]                                # back to row 0
    idx[5] = np.roll(idx[4], 3)                    # no position matches
    idx[6] = idx[5]
    idx[6, :20] = idx[4, :20]                      # partial realignment with row 4
    idx[7] = idx[4]
    idx[7, 40:60] = idx[4, 40]                     # duplicates of a shared token
    idx[8] = -1                                    # empty first row
    idx[9] = idx[10] = idx[11] = fresh(160)        # a run that row 0 does not share
    idx[13] = idx[15] = idx[12]
    idx[14] = fresh(160)                           # alternating sets A B A
    idx[17, 80:] = -1                              # short rows inside a team
    idx[18, ::3] = -1
    case.idx = idx
    dev = attn_to_dev(case)
    out, lse = _run_prefill(case, dev)
    ro, rl = _oracle(case)
    check_close(out, lse, ro, rl, f"team rows group {Hq}")
    cu_q = i32_dev(np.array([0, 5, 5, 13, 24]))    # teams that straddle requests
    cu_kv = i64_dev(np.array([0, 1500, 1500, 3000, 4500]))
    k3 = torch.cat([dev["k"]] * 3)
    v3 = torch.cat([dev["v"]] * 3)
    o2, l2 = sa.sparse_attn_chunk_prefill(dev["q"], k3, v3, dev["idx"], cu_q, cu_kv,
                                          sm_scale=case.scale)
    torch.cuda.synchronize()
    check_close(o2, l2, ro, rl, f"team rows ragged group {Hq}")


def test_binding_rejects_undersized_outputs():
    say("[binding] caller outputs too small: ValueError before any launch")
    case = _small(41, 8, 500, 400, 6, 1, 64)
    dev = attn_to_dev(case)
    before = sa.sa_call_count("sparse_attn_prefill")
    with pytest.raises(ValueError):
        sa.sparse_attn_prefill(dev["q"], dev["k"], dev["v"], dev["idx"],
                               out=torch.empty((7, 6, 256), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        sa.sparse_attn_prefill(dev["q"], dev["k"], dev["v"], dev["idx"],
                               lse=torch.empty((8, 5), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        sa.sparse_attn_union_build(dev["idx"], 500, 2,
                                   union_len=torch.empty((3,), dtype=torch.int32, device="cuda"))
    with pytest.raises(ValueError):
        sa.indexer_topk(torch.zeros((4, 100), dtype=torch.float32, device="cuda"), 10,
                        out=torch.empty((4, 9), dtype=torch.int32, device="cuda"))
    with pytest.raises(ValueError):
        sa.sparse_attn_prefill_union(dev["q"], dev["k"], dev["v"], dev["idx"], 2, kv_len=501)
    assert sa.sa_call_count("sparse_attn_prefill") == before


def _shuffled_ragged(seed, qlens, ctxs, topk, Hq=6):
    """Ragged requests (group Hq over one KV head) with walk indices whose
    slot order is shuffled in every row."""
    rng = np.random.default_rng(seed)
    cu_q = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    cu_kv = np.concatenate([[0], np.cumsum(ctxs)]).astype(np.int64)
    T, KV = int(cu_q[-1]), int(cu_kv[-1])
    q = gen.normal_bf16(rng, (T, Hq, 256))
    k = gen.normal_bf16(rng, (KV, 1, 256))
    v = gen.normal_bf16(rng, (KV, 1, 256))
    idx = np.concatenate([gen.random_walk_indices(rng, np.arange(c - n, c), topk)
                          for n, c in zip(qlens, ctxs) if n > 0]).astype(np.int32)
    idx = gen.shuffle_slots(idx, seed + 1)
    return gen.AttnCase("shuffled", q, k, v, idx, 1, 256, 256, 1 / 16, int(max(ctxs)),
                        np.zeros(T, np.int64), cu_q, cu_kv)


def test_membership_teams_edge_cases():
    # Two-row teams (group 6) match their rows by membership: shuffled slot
    # order, odd request lengths (teams straddling two requests), a request
    # longer than the 32768-token bitmaps, a row holding a token twice and a
    # row of padding fall back to matching by position.
    say("[chunk] membership teams: shuffled rows, straddling teams, long request, duplicates")
    qlens, ctxs = [7, 0, 12, 5, 9], [3000, 500, 33000, 900, 40000]
    case = _shuffled_ragged(31, qlens, ctxs, 300)
    idx = case.idx.copy()
    idx[2, 10:20] = idx[2, 5]          # duplicates (row 2 and its team mate fall back)
    idx[4, :] = -1                     # an empty row
    idx[9, ::7] = 10 ** 6              # out-of-range slots
    case.idx = idx
    dev = attn_to_dev(case)
    out, lse = _chunk(case, dev)
    ro, rl = oracle.chunk_prefill(case.q, case.k, case.v, case.idx, case.cu_seqlens_q,
                                  case.cu_seqlens_kv, num_kv_heads=1, scale=case.scale)
    e, el = check_close(out, lse, ro, rl, "membership edge cases")
    say(f"  max abs err O {e:.2e}  LSE {el:.2e}")


@pytest.mark.parametrize("group", [5, 6, 7, 8])
def test_membership_groups_and_topk_len(group):
    say(f"[prefill] membership teams, group {group}, shuffled rows, per-row topk_len")
    case = _small(40 + group, 33, 5000, 4900, group, 1, 700)
    case.idx = gen.shuffle_slots(case.idx, 7)
    tl = np.random.default_rng(group).integers(-3, 760, size=case.num_rows).astype(np.int32)
    dev = attn_to_dev(case)
    out, lse = _run_prefill(case, dev, topk_len=i32_dev(tl))
    ro, rl = _oracle(case, topk_len=tl)
    check_close(out, lse, ro, rl, f"membership group {group} with topk_len")


@pytest.mark.parametrize("scale", [1 / 16, 0.25, 0.5])
@pytest.mark.parametrize("group,mla", [(6, False), (12, False), (8, True)])
def test_large_score_ranges(scale, group, mla):
    # Large sm_scale spreads the scores over hundreds of log2 units, so the
    # running max moves (and the accumulators rescale) many times per row,
    # and most probabilities underflow to 0; shuffled slots make the max
    # arrive in any order.
    say(f"[prefill] sm_scale {scale}, group {group}{' MLA' if mla else ''}, shuffled slots")
    if mla:
        case = gen.make_attn_case("small", seed=61, num_rows=29, kv_len=900, first_pos=880,
                                  num_q_heads=group, num_kv_heads=1, head_dim_qk=576,
                                  head_dim_v=512, topk=400, v_in_k=True, walk=True)
    else:
        case = _small(61, 29, 900, 880, group, 1, 400)
    case.idx = gen.shuffle_slots(case.idx, 3)
    case.scale = scale
    dev = attn_to_dev(case)
    out, lse = _run_prefill(case, dev)
    ro, rl = _oracle(case)
    e, el = check_close(out, lse, ro, rl, f"scale {scale}")
    say(f"  max abs err O {e:.2e}  LSE {el:.2e}")
