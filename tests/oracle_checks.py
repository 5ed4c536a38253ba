"""Checks that pin the fp64 oracle to definitions outside itself.

Each check takes the oracle entry point it examines as an argument, so the
same check runs on the real oracle (it must pass) and on deliberately broken
copies of it (at least one check must fail for every planted mistake).
A check returns None when it passes and raises AssertionError otherwise.

Independent references used here:
* torch's float64 scaled_dot_product_attention and its CPU flash kernel
  (which also returns the log-sum-exp), on dense masked inputs;
* mpmath at 50 digits, by brute force, on tiny inputs;
* closed forms (one slot, identical keys, constant values);
* Python-set semantics for the union contract;
* numpy unique / reshape for the page mark and split.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import gen

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def f64(bits):
    # Widening via torch (independent of the oracle's own widening).
    t = torch.from_numpy(np.ascontiguousarray(bits).astype(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64)


def _dense_reference(q, k, v, mask_add, scale, num_kv_heads, dv=None):
    """Dense float64 attention with an additive mask [T, kv] shared by all
    heads, through torch. Returns O [T, Hq, Dv], LSE [T, Hq] as numpy."""
    Q = f64(q).permute(1, 0, 2).unsqueeze(0)                # [1, Hq, T, D]
    K = f64(k).permute(1, 0, 2).unsqueeze(0)                # [1, Hkv, kv, D]
    V = (K[..., :dv] if v is None else f64(v).permute(1, 0, 2).unsqueeze(0))
    group = Q.shape[1] // num_kv_heads
    Kr = K.repeat_interleave(group, dim=1).contiguous()
    Vr = V.repeat_interleave(group, dim=1).contiguous()
    M = torch.from_numpy(mask_add).to(torch.float64)[None, None]
    O = torch.nn.functional.scaled_dot_product_attention(Q, Kr, Vr, attn_mask=M, scale=scale)
    _, L = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        Q, Kr, Kr, 0.0, False, attn_mask=M, scale=scale)[:2]
    return O[0].permute(1, 0, 2).numpy(), L[0].permute(1, 0).numpy()


def _case(seed, T, kv, Hq, Hkv, D, Dv, first_pos=0, v_in_k=False):
    rng = np.random.default_rng(seed)
    q = gen.normal_bf16(rng, (T, Hq, D))
    k = gen.normal_bf16(rng, (kv, Hkv, D))
    v = None if v_in_k else gen.normal_bf16(rng, (kv, Hkv, Dv))
    return rng, q, k, v


# --------------------------------------------------------------------------
# per-token attention

def check_dense_causal(sparse_attention, seed=1):
    """Indices that cover exactly the visible prefix [0, t] (in any order,
    with -1 padding anywhere) reproduce dense causal attention."""
    for (Hq, Hkv, D, Dv, v_in_k) in [(6, 2, 32, 32, False), (4, 1, 24, 16, True),
                                     (12, 1, 16, 16, False)]:
        T, kv, width = 9, 12, 16
        first = kv - T
        rng, q, k, v = _case(seed, T, kv, Hq, Hkv, D, Dv, v_in_k=v_in_k)
        idx = np.full((T, width), -1, np.int32)
        mask = np.full((T, kv), -np.inf)
        for t in range(T):
            p = first + t
            vis = rng.permutation(p + 1)
            slots = np.sort(rng.choice(width, size=p + 1, replace=False))
            idx[t, slots] = vis
            mask[t, :p + 1] = 0.0
        scale = 0.7 / math.sqrt(D)
        o, lse = sparse_attention(q, k, v, idx, num_kv_heads=Hkv, scale=scale,
                                  kv_len=kv, head_dim_v=Dv)
        ro, rl = _dense_reference(q, k, v, mask, scale, Hkv, Dv)
        assert np.abs(o - ro).max() <= 1e-12, ("dense O", np.abs(o - ro).max())
        assert np.abs(lse - rl).max() <= 1e-12, ("dense LSE", np.abs(lse - rl).max())


def check_multiplicity(sparse_attention, seed=2):
    """Arbitrary indices, with duplicates, -1 and out-of-range entries, equal
    dense attention with additive mask log(count)."""
    T, kv, Hq, Hkv, D, width = 7, 10, 4, 2, 16, 12
    rng, q, k, v = _case(seed, T, kv, Hq, Hkv, D, D)
    idx = rng.integers(-2, kv + 3, size=(T, width)).astype(np.int32)
    idx[:, 0] = rng.integers(0, kv, size=T)           # no empty rows
    idx[0, 1:4] = idx[0, 0]                           # a tripled entry
    mask = np.full((T, kv), -np.inf)
    for t in range(T):
        cnt = np.bincount(idx[t][(idx[t] >= 0) & (idx[t] < kv)], minlength=kv)
        with np.errstate(divide="ignore"):
            mask[t] = np.log(cnt.astype(np.float64))
    o, lse = sparse_attention(q, k, v, idx, num_kv_heads=Hkv, scale=0.25, kv_len=kv)
    ro, rl = _dense_reference(q, k, v, mask, 0.25, Hkv)
    assert np.abs(o - ro).max() <= 1e-12, ("multiplicity O", np.abs(o - ro).max())
    assert np.abs(lse - rl).max() <= 1e-12, ("multiplicity LSE", np.abs(lse - rl).max())


def check_mpmath(sparse_attention, seed=3):
    """Brute force at 50 significant digits on a tiny case."""
    import mpmath
    mpmath.mp.dps = 50
    T, kv, Hq, Hkv, D, width = 3, 6, 2, 1, 5, 6
    rng, q, k, v = _case(seed, T, kv, Hq, Hkv, D, 3)
    idx = rng.integers(-1, kv, size=(T, width)).astype(np.int32)
    idx[:, 0] = [5, 0, 2]
    scale = 0.37
    o, lse = sparse_attention(q, k, v, idx, num_kv_heads=Hkv, scale=scale, kv_len=kv)
    Q, K, V = (f64(x).numpy() for x in (q, k, v))
    for t in range(T):
        for h in range(Hq):
            sel = [int(x) for x in idx[t] if 0 <= x < kv]
            s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(Q[t, h, d]) * mpmath.mpf(K[x, 0, d])
                                                  for d in range(D)) for x in sel]
            z = mpmath.fsum(mpmath.exp(si) for si in s)
            for d in range(V.shape[2]):
                ref = mpmath.fsum(mpmath.exp(si) * mpmath.mpf(V[x, 0, d])
                                  for si, x in zip(s, sel)) / z
                assert abs(float(ref) - o[t, h, d]) <= 1e-13, ("mpmath O", t, h, d)
            assert abs(float(mpmath.log(z)) - lse[t, h]) <= 1e-13, ("mpmath LSE", t, h)


def check_closed_forms(sparse_attention, seed=4):
    T, kv, Hq, D = 4, 8, 3, 16
    rng, q, k, v = _case(seed, T, kv, Hq, 1, D, D)
    Q, K, V = (f64(x).numpy() for x in (q, k, v))
    # one valid slot: O = V[x], LSE = s
    idx = np.full((T, 5), -1, np.int32)
    idx[:, 2] = [3, 0, 7, 5]
    o, lse = sparse_attention(q, k, v, idx, num_kv_heads=1, scale=0.5, kv_len=kv)
    for t in range(T):
        x = idx[t, 2]
        assert np.allclose(o[t], V[x, 0][None], rtol=0, atol=1e-15), "one slot O"
        assert np.allclose(lse[t], 0.5 * (Q[t] @ K[x, 0]), rtol=0, atol=1e-13), "one slot LSE"
    # identical keys: O = mean of V over the support, LSE = s + ln n
    k_same = np.repeat(k[:1], kv, axis=0)
    idx2 = np.tile(np.array([[1, 4, 6, -1, 2]], np.int32), (T, 1))
    o, lse = sparse_attention(q, k_same, v, idx2, num_kv_heads=1, scale=0.5, kv_len=kv)
    for t in range(T):
        sup = [1, 4, 6, 2]
        assert np.allclose(o[t], V[sup, 0].mean(0)[None], rtol=0, atol=1e-13), "same keys O"
        s = 0.5 * (Q[t] @ K[0, 0])
        assert np.allclose(lse[t], s + math.log(4), rtol=0, atol=1e-13), "same keys LSE"
    # constant V = c: O = c
    v_const = np.full_like(v, gen.bf16_bits_rne(np.float32([1.5]))[0])
    o, _ = sparse_attention(q, k, v_const, idx2, num_kv_heads=1, scale=0.5, kv_len=kv)
    assert np.abs(o - 1.5).max() <= 1e-14, "constant V"
    # empty support: O = 0, LSE = -inf
    idx3 = np.full((T, 5), -1, np.int32)
    idx3[0, 0] = kv          # out of range is masked too
    o, lse = sparse_attention(q, k, v, idx3, num_kv_heads=1, scale=0.5, kv_len=kv)
    assert np.all(o == 0) and np.all(np.isneginf(lse)), "empty support"


def check_invariants(sparse_attention, seed=5):
    """Permuting slots, inserting -1 and replacing -1 by an out-of-range
    index change nothing (exactly, up to summation order)."""
    T, kv, Hq, Hkv, D = 6, 40, 6, 1, 32
    rng, q, k, v = _case(seed, T, kv, Hq, Hkv, D, D)
    idx = np.stack([rng.choice(kv, size=10, replace=False) for _ in range(T)]).astype(np.int32)
    base = sparse_attention(q, k, v, idx, num_kv_heads=Hkv, scale=0.2, kv_len=kv)
    perm = idx[:, rng.permutation(10)]
    padded = np.full((T, 17), -1, np.int32)
    padded[:, ::2][:, :9] = idx[:, :9]
    padded[:, 1] = idx[:, 9]
    oor = padded.copy()
    oor[oor == -1] = kv + 5
    for variant in (perm, padded, oor):
        o, lse = sparse_attention(q, k, v, variant, num_kv_heads=Hkv, scale=0.2, kv_len=kv)
        assert np.abs(o - base[0]).max() <= 1e-13, "invariant O"
        assert np.abs(lse - base[1]).max() <= 1e-13, "invariant LSE"


def check_chunk_dense(chunk_prefill, seed=6):
    """Ragged requests whose indices cover each row's visible prefix equal
    dense causal attention computed per request."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D = 4, 2, 16
    qlens, ctxs = [3, 1, 4], [5, 9, 4]
    cu_q = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    cu_kv = np.concatenate([[0], np.cumsum(ctxs)]).astype(np.int64)
    T, KV, width = cu_q[-1], cu_kv[-1], 10
    q = gen.normal_bf16(rng, (T, Hq, D))
    k = gen.normal_bf16(rng, (KV, Hkv, D))
    v = gen.normal_bf16(rng, (KV, Hkv, D))
    idx = np.full((T, width), -1, np.int32)
    ro = np.zeros((T, Hq, D))
    rl = np.zeros((T, Hq))
    for r in range(3):
        mask = np.full((qlens[r], ctxs[r]), -np.inf)
        for i in range(qlens[r]):
            p = ctxs[r] - qlens[r] + i
            idx[cu_q[r] + i, :p + 1] = rng.permutation(p + 1)
            mask[i, :p + 1] = 0
        rows = slice(cu_q[r], cu_q[r + 1])
        kvs = slice(cu_kv[r], cu_kv[r + 1])
        o, l = _dense_reference(q[rows], k[kvs], v[kvs], mask, 0.3, Hkv)
        ro[rows], rl[rows] = o, l
    o, lse = chunk_prefill(q, k, v, idx, cu_q, cu_kv, num_kv_heads=Hkv, scale=0.3)
    assert np.abs(o - ro).max() <= 1e-12, ("chunk O", np.abs(o - ro).max())
    assert np.abs(lse - rl).max() <= 1e-12, ("chunk LSE", np.abs(lse - rl).max())


ATTN_CHECKS = [check_dense_causal, check_multiplicity, check_mpmath, check_closed_forms,
               check_invariants]


# --------------------------------------------------------------------------
# union build and union attention

def check_union_golden(union_build):
    """Hand-derived examples of the pages' union rule (tests/golden)."""
    with open(os.path.join(GOLDEN, "union_small.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        idx = np.array(c["idx"], np.int32)
        ui, ub, ul = union_build(idx, c["kv_len"], c["G"])
        assert ul.tolist() == c["union_len"], (c["name"], "len", ul.tolist())
        for g, (ei, eb) in enumerate(zip(c["union_idx"], c["union_bits"])):
            n = len(ei)
            assert ui[g, :n].tolist() == ei, (c["name"], "idx", g, ui[g, :n].tolist())
            assert ub[g, :n].tolist() == eb, (c["name"], "bits", g, ub[g, :n].tolist())
            assert np.all(ui[g, n:] == -1) and np.all(ub[g, n:] == 0), (c["name"], "fill")


def check_union_contract(union_build, seed=7):
    """Set semantics: each valid index of a token appears once in its group,
    bits = OR of owners, -1/out-of-range dropped, token-major ascending."""
    rng = np.random.default_rng(seed)
    for (T, width, kv, G) in [(9, 8, 20, 2), (10, 6, 12, 4), (7, 5, 9, 3), (5, 7, 30, 1)]:
        idx = rng.integers(-1, kv + 2, size=(T, width)).astype(np.int32)
        idx[1, :3] = idx[1, 0]                          # in-row duplicates
        ui, ub, ul = union_build(idx, kv, G)
        assert ui.shape == ((T + G - 1) // G, G * width)
        for g in range(ui.shape[0]):
            members = list(range(g * G, min(g * G + G, T)))
            sets = [set(int(x) for x in idx[t] if 0 <= x < kv) for t in members]
            n = int(ul[g])
            rows = ui[g, :n].tolist()
            assert len(rows) == len(set(rows)), "rows distinct"
            assert set(rows) == set().union(*sets), "rows = union of sets"
            assert sum(bin(b).count("1") for b in ub[g, :n]) == sum(len(s) for s in sets)
            first = []
            for r, x in enumerate(rows):
                bits = int(ub[g, r])
                want = sum(1 << j for j, s in enumerate(sets) if x in s)
                assert bits == want, ("bits", g, x, bits, want)
                first.append((bits & -bits).bit_length() - 1)
            keyed = list(zip(first, rows))
            assert keyed == sorted(keyed), "token-major, ascending"
            assert np.all(ui[g, n:] == -1) and np.all(ub[g, n:] == 0)


def check_union_equals_per_token(union_attention, sparse_attention, union_build, seed=8):
    """With duplicate-free rows, union attention equals per-token attention
    (PR 32779: union mode must reproduce the per-token output)."""
    for (T, G, Hq) in [(12, 2, 4), (11, 4, 8), (5, 3, 2)]:
        kv, width, D = 30, 9, 16
        rng, q, k, _ = _case(seed + T, T, kv, Hq, 1, D, 8, v_in_k=True)
        pos = np.arange(kv - T, kv)
        idx = gen.random_walk_indices(rng, pos, width, swap_frac=0.25)
        idx[2, 3] = -1
        ui, ub, ul = union_build(idx, kv, G)
        a = union_attention(q, k, None, ui, ub, ul, G, num_kv_heads=1, scale=0.3, head_dim_v=8)
        b = sparse_attention(q, k, None, idx, num_kv_heads=1, scale=0.3, kv_len=kv, head_dim_v=8)
        assert np.abs(a[0] - b[0]).max() <= 1e-12, "union O"
        assert np.abs(a[1] - b[1]).max() <= 1e-12, "union LSE"


def check_chunk_union_dense(chunk_union_build, chunk_union_attention, seed=11):
    """Ragged requests whose rows index their visible prefix (permuted, no
    duplicates, -1 tails) give dense causal attention per request through
    the ragged union; groups never span requests, so rows of different
    requests with the same local indices still see their own KV range."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D = 4, 1, 16
    qlens, ctxs = [5, 0, 3, 7], [9, 4, 3, 12]
    cu_q = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    cu_kv = np.concatenate([[0], np.cumsum(ctxs)]).astype(np.int64)
    T, KV, width = int(cu_q[-1]), int(cu_kv[-1]), 14
    q = gen.normal_bf16(rng, (T, Hq, D))
    k = gen.normal_bf16(rng, (KV, Hkv, D))
    v = gen.normal_bf16(rng, (KV, Hkv, D))
    idx = np.full((T, width), -1, np.int32)
    ro = np.zeros((T, Hq, D))
    rl = np.zeros((T, Hq))
    for r in range(len(qlens)):
        if qlens[r] == 0:
            continue
        mask = np.full((qlens[r], ctxs[r]), -np.inf)
        for i in range(qlens[r]):
            p = ctxs[r] - qlens[r] + i
            idx[cu_q[r] + i, :p + 1] = rng.permutation(p + 1)
            idx[cu_q[r] + i, p + 1] = ctxs[r] + 2          # out of its request's range
            mask[i, :p + 1] = 0
        rows = slice(cu_q[r], cu_q[r + 1])
        kvs = slice(cu_kv[r], cu_kv[r + 1])
        o, l = _dense_reference(q[rows], k[kvs], v[kvs], mask, 0.3, Hkv)
        ro[rows], rl[rows] = o, l
    for G in (2, 3, 4):
        ui, ub, ul, gr = chunk_union_build(idx, cu_q, cu_kv, G)
        want = sum((n + G - 1) // G for n in qlens)
        assert len(ul) == want, ("group count", G)
        o, lse = chunk_union_attention(q, k, v, ui, ub, ul, gr, cu_q, cu_kv, G,
                                       num_kv_heads=Hkv, scale=0.3)
        assert np.abs(o - ro).max() <= 1e-12, ("chunk union O", G)
        assert np.abs(lse - rl).max() <= 1e-12, ("chunk union LSE", G)


def check_chunk_union_equals_per_token(chunk_union_build, chunk_union_attention, chunk_prefill,
                                       seed=12):
    """On duplicate-free walk rows over ragged requests the ragged union
    equals the per-token chunk prefill."""
    rng = np.random.default_rng(seed)
    qlens, ctxs = [6, 3, 1, 9], [20, 12, 8, 30]
    cu_q = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    cu_kv = np.concatenate([[0], np.cumsum(ctxs)]).astype(np.int64)
    T, KV, width, Hq, D = int(cu_q[-1]), int(cu_kv[-1]), 7, 6, 8
    q = gen.normal_bf16(rng, (T, Hq, D))
    k = gen.normal_bf16(rng, (KV, 1, D))
    v = gen.normal_bf16(rng, (KV, 1, D))
    idx = np.concatenate([gen.random_walk_indices(rng, np.arange(c - n, c), width, swap_frac=0.3)
                          for n, c in zip(qlens, ctxs)]).astype(np.int32)
    idx[1, 2] = -1
    b = chunk_prefill(q, k, v, idx, cu_q, cu_kv, num_kv_heads=1, scale=0.4)
    for G in (2, 4):
        ui, ub, ul, gr = chunk_union_build(idx, cu_q, cu_kv, G)
        a = chunk_union_attention(q, k, v, ui, ub, ul, gr, cu_q, cu_kv, G, num_kv_heads=1,
                                  scale=0.4)
        assert np.abs(a[0] - b[0]).max() <= 1e-12, ("chunk union vs per-token O", G)
        assert np.abs(a[1] - b[1]).max() <= 1e-12, ("chunk union vs per-token LSE", G)


# --------------------------------------------------------------------------
# FP8 MLA records

def check_fp8_decode(fp8_e4m3_to_f64):
    """Every E4M3 code against torch's float8_e4m3fn widening (a library
    routine: OCP e4m3fn, bias 7, NaN at S.1111.111, no infinities)."""
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8_e4m3_to_f64(codes)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), "fp8 NaN codes"
    assert np.array_equal(got[~nan], want[~nan]), "fp8 values"


def check_mla_fp8_rows(mla_fp8_rows_to_f64):
    """Hand-built records: a different scale per 128-value block, known
    codes at block edges, known bf16 rope values."""
    rows = np.zeros((2, 656), np.uint8)
    scales = np.array([[0.5, 3.0, -0.25, 2.0 ** -10], [2.0, 4.0, 8.0, 16.0]], dtype="<f4")
    rows[:, 512:528] = scales.view(np.uint8)
    for b in range(4):
        rows[0, 128 * b] = 0x38          # 1.0
        rows[0, 128 * b + 127] = 0xC0    # -2.0
    rows[1, 5] = 0x01                    # 2^-9, subnormal
    rows[1, 300] = 0x7E                  # 448
    rope = np.array([1.5, -0.75, 0.0, 3.0], dtype=np.float32)
    rb = (rope.view(np.uint32) >> 16).astype("<u2")
    rows[0, 528:536] = rb.view(np.uint8)
    rows[1, 648:656] = rb.view(np.uint8)
    d = mla_fp8_rows_to_f64(rows)
    assert d.shape == (2, 576)
    want0 = np.zeros(576)
    for b in range(4):
        want0[128 * b] = float(scales[0, b])
        want0[128 * b + 127] = -2.0 * float(scales[0, b])
    want0[512:516] = rope
    want1 = np.zeros(576)
    want1[5] = 2.0 ** -9 * 2.0
    want1[300] = 448.0 * 8.0
    want1[572:576] = rope
    assert np.array_equal(d[0], want0), "record 0"
    assert np.array_equal(d[1], want1), "record 1"
    # products that bf16 cannot hold: fp32 product, then nearest-even bf16,
    # against torch's float8 widening, fp32 multiply and bfloat16 cast
    rng = np.random.default_rng(13)
    rows = rng.integers(0, 256, size=(3, 656), dtype=np.uint8)
    rows[:, :512][(rows[:, :512] & 0x7F) == 0x7F] = 0x3A       # no NaN codes
    sc = (rng.random((3, 4)) * 3 + 0.01).astype("<f4")
    rows[:, 512:528] = sc.view(np.uint8)
    rows[:, 528:] = 0
    code = torch.from_numpy(rows[:, :512].copy()).view(torch.float8_e4m3fn).float()
    prod = code * torch.from_numpy(sc).repeat_interleave(128, dim=1)
    want = prod.to(torch.bfloat16).to(torch.float64).numpy()
    got = mla_fp8_rows_to_f64(rows)[:, :512]
    assert np.array_equal(got, want), "fp32 product rounded to bf16"


# --------------------------------------------------------------------------
# pages

def check_page_mark(page_mark, seed=9):
    rng = np.random.default_rng(seed)
    P, ptok = 50, 16
    idx = rng.integers(-3, P * ptok + 20, size=(4, 37)).astype(np.int32)
    mask = page_mark(idx, P, ptok)
    valid = idx[(idx >= 0) & (idx < P * ptok)]
    want = np.zeros(P, np.int8)
    want[np.unique(valid // ptok)] = 1
    assert mask.dtype == np.int8 and np.array_equal(mask, want), "page mark"


def check_page_split(page_split, seed=10):
    rng = np.random.default_rng(seed)
    P, stok, dtok, rb, sb = 6, 8, 2, 5, 3
    ratio = stok // dtok
    src = rng.integers(0, 256, size=(P, stok * (rb + sb)), dtype=np.uint8)
    dst_stride = dtok * (rb + sb) + 4                   # padded destination pages
    dst0 = np.full((P * ratio, dst_stride), 0xA5, np.uint8)
    kw = dict(src_page_tokens=stok, dst_page_tokens=dtok, row_bytes=rb, scale_bytes=sb)
    full = page_split(src, dst0, None, **kw)
    data = src[:, :stok * rb].reshape(P * ratio, dtok * rb)
    scales = src[:, stok * rb:].reshape(P * ratio, dtok * sb)
    assert np.array_equal(full[:, :dtok * rb], data), "split data"
    assert np.array_equal(full[:, dtok * rb:dtok * (rb + sb)], scales), "split scales"
    assert np.all(full[:, dtok * (rb + sb):] == 0xA5), "padding untouched"
    mask = np.array([1, 0, 0, 1, 0, 1], np.int8)
    part = page_split(src, dst0, mask, **kw)
    for p in range(P):
        d = slice(p * ratio, (p + 1) * ratio)
        if mask[p]:
            assert np.array_equal(part[d], full[d]), "masked = full on touched"
        else:
            assert np.all(part[d] == 0xA5), "untouched stays stale"


# --------------------------------------------------------------------------
# sparse MLA decode over split pages

def _record(value_scale):
    """A 656-byte FP8 record whose 512 latent values all equal value_scale
    (code 0x38 = 1.0 times the scale in every block) and whose rope is 0."""
    r = np.zeros(656, np.uint8)
    r[:512] = 0x38
    r[512:528] = np.full(4, value_scale, dtype="<f4").view(np.uint8)
    return r


def check_paged_decode_closed_form(paged_decode):
    """Two 64-token pages, token t's latent values all t + 1: mean values,
    log-counts and a softmax over known scores, in closed form."""
    rng = np.random.default_rng(21)
    ptok, stride = 64, 64 * 660 + 32                   # rows, per-token words, padding
    pool = rng.integers(0, 256, size=(2, stride), dtype=np.uint8)   # garbage elsewhere
    for t in (0, 5, 64, 70, 127):
        p, r = divmod(t, ptok)
        pool[p, r * 656:(r + 1) * 656] = _record(t + 1.0)
    q = np.zeros((3, 2, 576), np.uint16)
    q[1, 0, 3] = 0x3F80                                # head 0 reads latent dim 3
    q[1, 1, 560] = 0x3F80                              # head 1 reads a rope dim (0)
    idx = np.array([[5, 70, -1, 5, 128, -7],
                    [0, 127, 64, -1, -1, -1],
                    [-1, -1, -1, -1, -1, -1]], np.int32)
    scale = 0.05
    o, lse = paged_decode(q, pool, idx, page_tokens=ptok, scale=scale)
    assert o.shape == (3, 2, 512) and lse.shape == (3, 2)
    # request 0: zero query, multiset {6, 71, 6}
    assert np.allclose(o[0], (6 + 71 + 6) / 3, rtol=0, atol=1e-12), "mean over the multiset"
    assert np.allclose(lse[0], math.log(3), rtol=0, atol=1e-12), "log count"
    # request 1, head 0: scores scale * (t + 1) over {1, 128, 65}
    vals = [1.0, 128.0, 65.0]
    w = [math.exp(scale * x) for x in vals]
    assert np.allclose(o[1, 0], sum(a * b for a, b in zip(w, vals)) / sum(w), rtol=0, atol=1e-10)
    assert abs(lse[1, 0] - math.log(sum(w))) < 1e-12, "softmax lse"
    assert np.allclose(o[1, 1], sum(vals) / 3, rtol=0, atol=1e-12), "rope-only head"
    assert np.all(o[2] == 0) and np.all(np.isneginf(lse[2])), "empty support"
    # topk_len: request 0 sees {6, 71}, request 1 nothing past slot 0
    o, lse = paged_decode(q, pool, idx, page_tokens=ptok, scale=scale,
                          topk_len=np.array([2, 1, 6], np.int32))
    assert np.allclose(o[0], 38.5, rtol=0, atol=1e-12) and np.allclose(lse[0], math.log(2))
    assert np.allclose(o[1], 1.0, rtol=0, atol=1e-12), "one slot: its own V"


def check_paged_decode_vs_source(paged_decode, sparse_attention, mla_fp8_rows_to_f64, seed=22):
    """Pages of 64 tokens built from 256-token source pages by numpy
    reshapes; the decode over them equals per-token sparse attention over
    the records in token order (the source layout), duplicates, padding,
    out-of-pool ids and per-request lengths included."""
    rng = np.random.default_rng(seed)
    P, stok, dtok, rb, sb = 3, 256, 64, 656, 4
    tokens = P * stok
    records = gen.mla_fp8_rows(rng, tokens)
    words = rng.integers(0, 256, size=(P, stok * sb), dtype=np.uint8)
    src = np.concatenate([records.reshape(P, stok * rb), words], axis=1)
    ratio = stok // dtok
    data = src[:, :stok * rb].reshape(P * ratio, dtok * rb)
    sc = src[:, stok * rb:].reshape(P * ratio, dtok * sb)
    pad = np.full((P * ratio, 48), 0xA5, np.uint8)
    dst = np.concatenate([data, sc, pad], axis=1)
    B, Hq, k = 5, 4, 40
    q = gen.normal_bf16(rng, (B, Hq, 576))
    idx = rng.integers(-4, tokens + 30, size=(B, k)).astype(np.int32)
    idx[1, 10:20] = idx[1, :10]                      # duplicates
    idx[2] = -1
    topk_len = np.array([k, 33, k, 7, 0], np.int32)
    scale = 1.0 / 24
    rows = mla_fp8_rows_to_f64(records)[:, None, :]   # [tokens, 1, 576] float64
    for tl in (None, topk_len):
        got_o, got_l = paged_decode(q, dst, idx, page_tokens=dtok, scale=scale, topk_len=tl)
        want_o, want_l = sparse_attention(q, rows, None, idx, num_kv_heads=1, scale=scale,
                                          kv_len=tokens, head_dim_v=512, topk_len=tl)
        assert np.allclose(got_o, want_o, rtol=0, atol=1e-12), "decode O"
        fin = np.isfinite(want_l)
        assert np.array_equal(fin, np.isfinite(got_l)), "empty rows"
        assert np.allclose(got_l[fin], want_l[fin], rtol=0, atol=1e-12), "decode LSE"


# --------------------------------------------------------------------------
# indexer top-k selection

def _rank_count_select(row, n, k):
    """Brute force: position j < n is selected iff fewer than k positions
    beat it (a larger score, or an equal score at a lower position)."""
    sel = []
    for j in range(n):
        beat = sum(1 for i in range(n) if row[i] > row[j] or (row[i] == row[j] and i < j))
        if beat < k:
            sel.append(j)
    return sel + [-1] * (k - len(sel))


def check_topk_rank_count(topk_select, seed=31):
    """Small rows with many ties, signed zeros and infinities, lengths from
    0 to past the row, against the rank-count characterisation."""
    rng = np.random.default_rng(seed)
    T, kv = 7, 40
    s = np.round(rng.standard_normal((T, kv)) * 2).astype(np.float32)   # many ties
    s[0, 3], s[0, 9] = -0.0, 0.0
    s[1, [2, 30]] = np.inf
    s[2, [0, 1, 5]] = -np.inf
    row_len = np.array([40, 33, 12, 0, 1, 39, 55], np.int32)
    for k in (1, 7, 12, 39, 40, 45):
        got = topk_select(s, k, row_len)
        assert got.shape == (T, k) and got.dtype == np.int32
        for t in range(T):
            n = max(0, min(int(row_len[t]), kv))
            want = _rank_count_select(s[t].tolist(), n, k)
            assert got[t].tolist() == want, (k, t)
    got = topk_select(s[:2], 5)                       # no lengths: whole rows
    assert got[0].tolist() == _rank_count_select(s[0].tolist(), kv, 5)


def check_topk_library(topk_select, seed=32):
    """Distinct scores: the selected set is torch.topk's index set."""
    rng = np.random.default_rng(seed)
    T, kv, k = 5, 3000, 2051
    s = rng.permutation(T * kv).reshape(T, kv).astype(np.float32) / 7.0   # distinct
    row_len = np.array([3000, 2500, 2052, 2100, 2999], np.int32)
    got = topk_select(s, k, row_len)
    for t in range(T):
        n = int(row_len[t])
        want = torch.topk(torch.from_numpy(s[t, :n].copy()), k).indices.numpy()
        assert np.array_equal(got[t], np.sort(want)), t


def check_topk_closed_forms(topk_select):
    kv, k = 50, 8
    eq = np.zeros((1, kv), np.float32)
    assert topk_select(eq, k).tolist() == [list(range(k))], "equal scores: lowest positions"
    up = np.arange(kv, dtype=np.float32)[None]
    assert topk_select(up, k).tolist() == [list(range(kv - k, kv))], "increasing"
    assert topk_select(-up, k).tolist() == [list(range(k))], "decreasing"
    assert topk_select(up, k, np.array([5])).tolist() == [[0, 1, 2, 3, 4, -1, -1, -1]], "short row"
    assert topk_select(up, k, np.array([0])).tolist() == [[-1] * k], "empty row"
    z = np.full((1, kv), -1.0, np.float32)
    z[0, 7], z[0, 2] = -0.0, 0.0
    assert topk_select(z, 1).tolist() == [[2]], "signed zeros tie"
    assert topk_select(z, 2).tolist() == [[2, 7]]
