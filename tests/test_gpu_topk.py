"""GPU parity: the indexer's top-k selection, bit-exact against the oracle,
through the C ABI (rows in registers up to 32768 positions, re-read
beyond)."""
import numpy as np
import pytest
import torch

import gen
import oracle
import top_index_sparse_amd as sa
from tests.gpu_util import config, i32_dev, sample_rows, say

pytestmark = pytest.mark.gpu


def _f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _check(scores, k, row_len=None, what=""):
    got = sa.indexer_topk(_f32_dev(scores), k,
                          row_len=None if row_len is None else i32_dev(row_len))
    torch.cuda.synchronize()
    want = oracle.topk_select(scores, k, row_len)
    g = got.cpu().numpy()
    bad = np.nonzero((g != want).any(axis=1))[0]
    assert bad.size == 0, f"{what}: rows {bad[:8].tolist()} differ"


def test_topk_small_config():
    say("[topk] C0topk: 128 rows over 512 positions, k 64, short rows padded")
    c = config("C0topk")
    _check(c.scores, c.k, c.row_len, "C0topk")


@pytest.mark.parametrize("kv", [100, 4096, 4097, 16384, 16385, 32768, 32769, 70000])
@pytest.mark.parametrize("k", [1, 64, 2051])
def test_topk_ties_and_lengths(kv, k):
    say(f"[topk] kv {kv}, k {k}: ties, signed zeros, infinities, lengths")
    rng = np.random.default_rng(kv * 7 + k)
    T = 8
    s = (np.round(rng.standard_normal((T, kv)) * 8) / 8).astype(np.float32)   # heavy ties
    s[0, ::3] = -0.0
    s[0, 1::3] = 0.0
    s[1, rng.integers(0, kv, 5)] = np.inf
    s[2, rng.integers(0, kv, 50)] = -np.inf
    s[3] = 1.25                                                               # one value
    row_len = np.array([kv, kv - 1, kv // 2, kv, 0, min(k, kv), k + 1, kv + 9], np.int32)
    _check(s, k, row_len, f"kv={kv} k={k}")
    _check(s, k, None, f"kv={kv} k={k} whole rows")


def test_topk_padded_stride():
    say("[topk] scores with a padded row stride")
    rng = np.random.default_rng(5)
    T, kv, k = 6, 5000, 300
    buf = rng.standard_normal((T, kv + 12)).astype(np.float32)
    sc = torch.from_numpy(buf).cuda()[:, :kv]
    got = sa.indexer_topk(sc, k)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), oracle.topk_select(buf[:, :kv], k))


def test_topk_c1_full_size():
    say("[topk] C1topk: 8192 rows x 32768 positions, k 2051 (sampled rows)")
    c = config("C1topk")
    got = sa.indexer_topk(_f32_dev(c.scores), c.k, row_len=i32_dev(c.row_len))
    torch.cuda.synchronize()
    rows = sample_rows(c.scores.shape[0], 24)
    want = oracle.topk_select(c.scores[rows], c.k, c.row_len[rows])
    assert np.array_equal(got.cpu().numpy()[rows], want)
    # adjacent rows share about 98 % of their selection (the walk's rate)
    g = got.cpu().numpy()
    same = np.mean([len(np.intersect1d(g[t], g[t + 1])) / c.k for t in range(0, 8000, 97)])
    say(f"  mean overlap of adjacent rows {same:.4f}")
    assert 0.95 < same < 0.995


def test_topk_counts_past_16_bits():
    say("[topk] k 66000 of 70000 positions; 70000 equal scores")
    rng = np.random.default_rng(77)
    kv, k = 70000, 66000
    s = (np.round(rng.standard_normal((3, kv)) * 4) / 4).astype(np.float32)
    s[1] = -2.5
    _check(s, k, np.array([kv, kv, 69999], np.int32), "k=66000")
    _check(s[:2], 2051, None, "70000 ties")


@pytest.mark.parametrize("i", range(40))
def test_topk_sweep(i):
    """Seeded random shapes and score kinds: N(0,1), heavy ties, one value,
    fp32 subnormals, and a mix of +-inf, +-0 and +-1."""
    rng = np.random.default_rng(90000 + i)
    T = int(rng.integers(1, 9))
    kv = int(rng.choice([rng.integers(1, 600), rng.integers(600, 40000), rng.integers(40000, 90000)]))
    k = int(rng.integers(1, min(kv + 100, 9000)))
    kind = int(rng.integers(0, 5))
    if kind == 0:
        s = rng.standard_normal((T, kv))
    elif kind == 1:
        s = np.round(rng.standard_normal((T, kv)) * 2) / 2
    elif kind == 2:
        s = np.full((T, kv), float(rng.standard_normal()))
    elif kind == 3:
        s = rng.standard_normal((T, kv)) * 1e-40
    else:
        s = rng.choice([-np.inf, np.inf, 0.0, -0.0, 1.0, -1.0], size=(T, kv))
    s = s.astype(np.float32)
    rl = rng.integers(-5, kv + 20, T).astype(np.int32) if rng.random() < 0.6 else None
    say(f"[topk sweep {i}] T={T} kv={kv} k={k} kind={kind} row_len={rl is not None}")
    _check(s, k, rl, f"sweep {i}")


def _sample_positions(kv):
    """Positions the sampled selection reads for its threshold (rows of
    4097 .. 32768 positions): thread j of the row's 1024 reads position
    4 (c 1024 + j) with c = j mod (chunks of 4096 positions)."""
    nch = 8 if kv > 16384 else 4
    j = np.arange(1024)
    return 4 * ((j % nch) * 1024 + j)


@pytest.mark.parametrize("kv", [16384, 32768])
def test_topk_sample_misleads(kv):
    """The sample sees only planted large scores, so its threshold keeps
    fewer than k elements; the row must fall back to the full selection."""
    say(f"[topk] kv {kv}: large scores planted where the threshold sample reads")
    rng = np.random.default_rng(kv + 3)
    s = rng.standard_normal((4, kv)).astype(np.float32)
    pos = _sample_positions(kv)
    s[0, pos] = 100.0
    s[1, pos] = np.float32(5.0) + rng.random(pos.size).astype(np.float32)
    s[2, pos[::2]] = 7.0                       # half the sample
    s[3, pos] = -100.0                         # the sample sees only small scores
    for k in (1, 600, 1024, 1025, 2051, 4096):
        _check(s, k, None, f"kv={kv} k={k} planted")
        _check(s, k, np.array([kv, kv - 5, kv // 2 + 3, 4 * k // 3 + 1], np.int32),
               f"kv={kv} k={k} planted, lengths")


@pytest.mark.parametrize("kv", [8192, 20000, 32764])
def test_topk_sampled_row_ends(kv):
    """Rows of N(0,1) scores over storage of a multiple of four scores (the
    16-byte read of every chunk, lanes past the row reading the quad that
    holds its last position): lengths that end inside a quad, inside a
    chunk and chunks before the storage ends, with large scores stored past
    every row's end, where a missed mask would select them."""
    say(f"[topk] kv {kv}: sampled selection, row ends inside quads and chunks")
    rng = np.random.default_rng(kv + 11)
    lengths = [kv, kv - 1, kv - 3, 4097, 4099, kv // 2 + 1, kv // 2 + 2, 5 * kv // 8 + 3]
    s = rng.standard_normal((len(lengths), kv)).astype(np.float32)
    rl = np.array(lengths, np.int32)
    for t, n in enumerate(lengths):
        s[t, n:] = 50.0
    for k in (1, 777, 2051, 4096, 4097):   # (4097: past the sampled selection's k)
        _check(s, k, rl, f"kv={kv} k={k} row ends")


def test_topk_odd_row_stride():
    """A row stride of an odd number of floats leaves most rows unaligned
    for 16-byte loads: the selection must not depend on it."""
    say("[topk] scores with an odd row stride")
    rng = np.random.default_rng(6)
    T, kv, k = 6, 20000, 2051
    buf = rng.standard_normal((T, kv + 3)).astype(np.float32)
    sc = torch.from_numpy(buf).cuda()[:, :kv]
    rl = np.array([kv, kv - 1, 9001, 4097, 2052, 19999], np.int32)
    got = sa.indexer_topk(sc, k, row_len=i32_dev(rl))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), oracle.topk_select(buf[:, :kv], k, rl))


@pytest.mark.parametrize("kv", [16384, 32768])
def test_topk_sample_outliers(kv):
    """A few huge scores at sampled positions put the sample's largest key
    far above the bin its threshold lies in, beyond the 64 bins the short
    search scans below it, so the threshold comes from the search over all
    bins; the selection must not change."""
    say(f"[topk] kv {kv}: outliers at sampled positions")
    rng = np.random.default_rng(kv + 17)
    s = rng.standard_normal((4, kv)).astype(np.float32)
    pos = _sample_positions(kv)
    s[0, pos[:3]] = 1e30
    s[1, pos[::97]] = np.float32(3e38)
    s[2, pos[:1]] = 1e10
    s[3, pos[:40]] = 1e20 * rng.random(40).astype(np.float32)
    for k in (1, 64, 2051, 4096, 4097):
        _check(s, k, None, f"kv={kv} k={k} outliers")
        _check(s, k, np.array([kv, kv - 7, kv // 2 + 5, 3 * k // 2 + 1], np.int32),
               f"kv={kv} k={k} outliers, lengths")
