"""GPU parity: sparse MLA prefill (576-wide latent rows, V inside K), the
union-of-G index build (bit-exact) and union attention, against the fp64
oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import gen
import oracle
import top_index_sparse_amd as sa
from tests.gpu_util import attn_to_dev, check_close, config, i32_dev, sample_rows, say

pytestmark = pytest.mark.gpu


def _mla_small(seed, T, kv, first, topk, Hq=8):
    return gen.make_attn_case("mla", seed=seed, num_rows=T, kv_len=kv, first_pos=first,
                              num_q_heads=Hq, num_kv_heads=1, head_dim_qk=576, head_dim_v=512,
                              topk=topk, v_in_k=True, scale=1 / 24)


def _prefill(case, dev):
    out, lse = sa.sparse_attn_prefill(dev["q"], dev["k"], None, dev["idx"], sm_scale=case.scale,
                                      kv_len=case.kv_len, head_dim_v=case.head_dim_v)
    torch.cuda.synchronize()
    return out, lse


def _oracle(case, rows=None, idx=None):
    return oracle.sparse_attention(case.q, case.k, case.v, case.idx if idx is None else idx,
                                   num_kv_heads=case.num_kv_heads, scale=case.scale,
                                   kv_len=case.kv_len, head_dim_v=case.head_dim_v, rows=rows)


def test_mla_per_token_small_with_padding():
    say("[mla] per-token, rows with -1 padding and a ragged tail tile")
    case = _mla_small(31, 70, 300, 0, 130)           # rows 0..69 are padded
    dev = attn_to_dev(case)
    out, lse = _prefill(case, dev)
    ro, rl = _oracle(case)
    check_close(out, lse, ro, rl, "mla small")


@pytest.mark.parametrize("Hq", [8, 16, 3, 24, 32, 17])
def test_mla_head_counts(Hq):
    say(f"[mla] {Hq} heads")
    case = _mla_small(32, 9, 3000, 2500, 2048, Hq=Hq)
    dev = attn_to_dev(case)
    out, lse = _prefill(case, dev)
    ro, rl = _oracle(case)
    check_close(out, lse, ro, rl, f"mla {Hq} heads")


def test_mla_c3_sampled():
    say("[mla] C3 full size per-token, sampled rows")
    case = config("C3")
    dev = attn_to_dev(case)
    out, lse = _prefill(case, dev)
    rows = sample_rows(case.num_rows, 40)
    ro, rl = _oracle(case, rows=rows)
    sel = torch.from_numpy(rows).cuda()
    e, el = check_close(out[sel], lse[sel], ro, rl, "C3")
    assert torch.isfinite(out).all()
    say(f"  C3 per-token: max abs err O {e:.2e} LSE {el:.2e}")


# ------------------------------------------------------------- union build

def _check_union_exact(idx_np, kv_len, G, groups=None):
    idx = i32_dev(idx_np)
    ui, ub, ul = sa.sparse_attn_union_build(idx, kv_len, G)
    torch.cuda.synchronize()
    ri, rb, rl = oracle.union_build(idx_np, kv_len, G)
    assert np.array_equal(ul.cpu().numpy(), rl), "union_len"
    assert np.array_equal(ui.cpu().numpy(), ri), "union_idx"
    assert np.array_equal(ub.cpu().numpy(), rb), "union_bits"
    return ri, rb, rl


# Bit planes in LDS while G x kv_len <= 2^19 (64 KB), sort and merge above:
# (6, 500, 262144, 2) is the largest bitmap case, the next kv_len and the
# last three rows take the sort path.
@pytest.mark.parametrize("T,k,kv,G", [(9, 8, 20, 2), (10, 6, 12, 4), (7, 5, 9, 3), (5, 7, 30, 1),
                                      (33, 100, 500, 8), (17, 2051, 40000, 2), (1, 1, 3, 4),
                                      (6, 500, 262144, 2), (6, 500, 262145, 2),
                                      (9, 300, 600000, 2), (12, 40, 70000, 8),
                                      (20, 2051, 300000, 2)])
def test_union_build_random_exact(T, k, kv, G):
    say(f"[union build] random T={T} k={k} kv={kv} G={G}")
    rng = np.random.default_rng(T * 1000 + k)
    idx = rng.integers(-2, kv + 3, size=(T, k)).astype(np.int32)
    if T > 1 and k > 3:
        idx[1, :3] = idx[1, 0]
    _check_union_exact(idx, kv, G)


@pytest.mark.parametrize("i", range(40))
def test_union_build_sweep(i):
    """Seeded random T, top-k, kv_len (both build paths, up to 3M tokens) and
    G in 1..8; half the cases give neighbouring rows mostly the same slots."""
    rng = np.random.default_rng(70000 + i)
    T = int(rng.integers(1, 80))
    k = int(rng.integers(1, 2600))
    kv = int(rng.choice([rng.integers(1, 3000), rng.integers(3000, 300000),
                         rng.integers(300000, 3000000)]))
    G = int(rng.integers(1, 9))
    idx = rng.integers(-3, kv + 4, size=(T, k)).astype(np.int32)
    if rng.random() < 0.5:
        base = np.sort(rng.choice(kv, size=min(k, kv), replace=False)) if kv >= k \
            else rng.integers(0, kv, k)
        for t in range(T):
            row = np.array(base[:k], dtype=np.int64)
            m = rng.random(len(row)) < 0.05
            row[m] = rng.integers(-1, kv, m.sum())
            idx[t, :len(row)] = row
    if k > 4:
        idx[0, :2] = idx[0, 2]
    say(f"[union build sweep {i}] T={T} k={k} kv={kv} G={G}")
    _check_union_exact(idx, kv, G)


@pytest.mark.parametrize("G", [2, 4])
def test_union_build_c3_exact(G):
    say(f"[union build] C3 full size G={G}, bit-exact")
    case = config("C3")
    ri, rb, rl = _check_union_exact(case.idx, case.kv_len, G)
    say(f"  C3 G={G}: {int(rl.sum())} union rows")


def test_union_build_tail_and_strided_idx():
    say("[union build] T % G tail, strided index rows")
    case = config("C3tail")
    idx = torch.full((case.num_rows, case.topk + 16), -5, dtype=torch.int32, device="cuda")
    idx[:, :case.topk] = i32_dev(case.idx)
    ui, ub, ul = sa.sparse_attn_union_build(idx[:, :case.topk], case.kv_len, 4)
    torch.cuda.synchronize()
    ri, rb, rl = oracle.union_build(case.idx, case.kv_len, 4)
    assert np.array_equal(ul.cpu().numpy(), rl)
    assert np.array_equal(ui.cpu().numpy(), ri)
    assert np.array_equal(ub.cpu().numpy(), rb)


def test_union_build_deterministic():
    case = config("C3")
    idx = i32_dev(case.idx[:512])
    a = sa.sparse_attn_union_build(idx, case.kv_len, 4)
    b = sa.sparse_attn_union_build(idx, case.kv_len, 4)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# --------------------------------------------------------- union attention

def _union(case, dev, G):
    out, lse, st = sa.sparse_attn_prefill_union(dev["q"], dev["k"], dev["v"], dev["idx"], G,
                                                sm_scale=case.scale, kv_len=case.kv_len,
                                                head_dim_v=case.head_dim_v)
    torch.cuda.synchronize()
    return out, lse, st


@pytest.mark.parametrize("G", [2, 4])
def test_union_mla_c3_sampled(G):
    say(f"[union] C3 G={G}, sampled rows vs oracle union attention")
    case = config("C3")
    dev = attn_to_dev(case)
    out, lse, st = _union(case, dev, G)
    assert st == sa.SA_OK
    rows = sample_rows(case.num_rows, 32)
    ui, ub, ul = oracle.union_build(case.idx[: (rows.max() // G + 1) * G], case.kv_len, G)
    ro, rl = oracle.union_attention(case.q, case.k, None, ui, ub, ul, G, num_kv_heads=1,
                                    scale=case.scale, head_dim_v=512, rows=rows)
    sel = torch.from_numpy(rows).cuda()
    e, el = check_close(out[sel], lse[sel], ro, rl, f"union G={G}")
    assert torch.isfinite(out).all()
    # The per-token path on every row: duplicate-free rows give the same
    # result up to summation order. LSE is the sensitive check (one slot
    # more or less moves it by ~1/topk); O differs by the bf16 rounding of
    # P taken against different running maxima.
    po, pl = _prefill(case, dev)
    dl = (lse - pl).abs()
    do = (out.float() - po.float()).abs()
    say(f"  union vs per-token: max |dLSE| {dl.max().item():.2e} at row "
        f"{int(dl.amax(1).argmax())}, max |dO| {do.max().item():.2e}")
    assert dl.max().item() < 2e-5
    assert (do <= 2e-2 + 1e-2 * po.float().abs()).all()
    say(f"  C3 G={G}: max abs err O {e:.2e} LSE {el:.2e}")


def test_union_tail_rows():
    say("[union] T=1023, G=4: tail group of 3 rows")
    case = config("C3tail")
    dev = attn_to_dev(case)
    out, lse, st = _union(case, dev, 4)
    rows = np.concatenate([np.arange(0, 8), np.arange(case.num_rows - 7, case.num_rows)])
    ro, rl = _oracle(case, rows=rows)
    sel = torch.from_numpy(rows).cuda()
    check_close(out[sel], lse[sel], ro, rl, "union tail")


def test_union_duplicates_count_once():
    say("[union] duplicated indices: union counts each index once")
    case = _mla_small(33, 12, 400, 300, 64)
    idx = case.idx.copy()
    idx[3, 5:20] = idx[3, 4]
    idx[6, :] = -1
    idx[7, 1:] = -1
    case.idx = idx
    dev = attn_to_dev(case)
    out, lse, st = _union(case, dev, 2)
    dedup = np.full_like(idx, -1)
    for t in range(idx.shape[0]):
        u = np.unique(idx[t][(idx[t] >= 0) & (idx[t] < case.kv_len)])
        dedup[t, :len(u)] = u
    ro, rl = _oracle(case, idx=dedup)
    check_close(out, lse, ro, rl, "union dedup")


def test_union_fallback_when_tile_illegal():
    say("[union] group 16 x G=4 > 32 rows: per-token fallback")
    case = _mla_small(34, 10, 500, 400, 96, Hq=16)
    dev = attn_to_dev(case)
    out, lse, st = _union(case, dev, 4)
    assert st == sa.SA_OK_FALLBACK
    ro, rl = _oracle(case)
    check_close(out, lse, ro, rl, "fallback")
    po, pl = _prefill(case, dev)
    assert torch.equal(out, po) and torch.equal(lse, pl)


@pytest.mark.parametrize("Hq,Hkv,G", [(6, 1, 2), (12, 2, 2), (4, 1, 4), (2, 1, 8), (6, 1, 5), (12, 1, 4),
                                     (8, 1, 4), (12, 1, 2), (32, 1, 1), (40, 2, 1), (20, 1, 2)])
def test_union_gqa(Hq, Hkv, G):
    say(f"[union] GQA d=256 group {Hq // Hkv} x {Hkv} KV heads, G={G}")
    case = gen.make_attn_case("u", seed=35 + G, num_rows=23, kv_len=3000, first_pos=2977,
                              num_q_heads=Hq, num_kv_heads=Hkv, head_dim_qk=256, head_dim_v=256,
                              topk=300)
    dev = attn_to_dev(case)
    out, lse, st = _union(case, dev, G)
    assert st == (sa.SA_OK if G * Hq // Hkv <= 32 else sa.SA_OK_FALLBACK)
    ro, rl = _oracle(case)
    check_close(out, lse, ro, rl, f"union gqa {Hq}/{Hkv} G={G}")


@pytest.mark.parametrize("name,G", [("C2", 2), ("C1", 5)])
def test_union_gqa_two_tile_full_size(name, G):
    # the two-tile union team (G x group in 17..32 columns): C2 (2 KV heads x
    # group 12) at G=2, C1 (group 6) at G=5, full size, sampled rows
    say(f"[union] {name} G={G} full size, sampled rows vs oracle union attention")
    case = config(name)
    dev = attn_to_dev(case)
    out, lse, st = _union(case, dev, G)
    assert st == sa.SA_OK
    rows = sample_rows(case.num_rows, 16)
    ui, ub, ul = oracle.union_build(case.idx[: (rows.max() // G + 1) * G], case.kv_len, G)
    ro, rl = oracle.union_attention(case.q, case.k, case.v, ui, ub, ul, G,
                                    num_kv_heads=case.num_kv_heads, scale=case.scale, rows=rows)
    sel = torch.from_numpy(rows).cuda()
    e, el = check_close(out[sel], lse[sel], ro, rl, f"{name} union G={G}")
    assert torch.isfinite(out).all()
    say(f"  {name} G={G}: max abs err O {e:.2e} LSE {el:.2e}")


@pytest.mark.parametrize("Hq,G", [(24, 1), (32, 1), (32, 2)])
def test_mla_wide_head_rows_union(Hq, G):
    # more than 16 heads: two 16-head slices; G=2 is illegal (64 rows) and
    # falls back to the per-token path
    say(f"[union] MLA {Hq} heads, G={G}")
    case = _mla_small(36, 11, 2000, 1900, 300, Hq=Hq)
    dev = attn_to_dev(case)
    out, lse, st = _union(case, dev, G)
    assert st == (sa.SA_OK if G * Hq <= 32 else sa.SA_OK_FALLBACK)
    ro, rl = _oracle(case)
    check_close(out, lse, ro, rl, f"mla {Hq} heads G={G}")
