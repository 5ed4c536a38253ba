"""The fp64 oracle against definitions outside itself, and planted mistakes.

First part: every pin passes on the oracle as committed.
Second part: copies of the oracle with one plausible mistake planted each (a
dropped term, a wrong sign, index or head mapping, a transposed operand, a
dropped mask) must each fail at least one pin, which shows the pins can see
such mistakes. Mistakes are planted only in the oracle, on the CPU.
"""
import numpy as np
import pytest

import oracle
import oracle.attention as oatt
from tests import oracle_checks as C


# ----------------------------------------------------------------- pins pass

@pytest.mark.parametrize("check", C.ATTN_CHECKS, ids=lambda c: c.__name__)
def test_attention_pins(check):
    check(oracle.sparse_attention)


def test_chunk_prefill_dense():
    C.check_chunk_dense(oracle.chunk_prefill)


def test_union_golden():
    C.check_union_golden(oracle.union_build)


def test_union_contract():
    C.check_union_contract(oracle.union_build)


def test_union_equals_per_token():
    C.check_union_equals_per_token(oracle.union_attention, oracle.sparse_attention,
                                   oracle.union_build)


def test_page_mark():
    C.check_page_mark(oracle.page_mark)


def test_page_split():
    C.check_page_split(oracle.page_split)


def test_bf16_widening_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    a = oracle.bf16_to_f64(bits)
    b = C.f64(bits).numpy()
    same = (a == b) | (np.isnan(a) & np.isnan(b))
    assert same.all()


# ------------------------------------------------------- planted mistakes

def _fails_some(checks):
    for chk in checks:
        try:
            chk()
        except (AssertionError, IndexError, ValueError):
            return True
    return False


def _attn_checks():
    return [lambda c=c: c(oracle.sparse_attention) for c in C.ATTN_CHECKS] + \
           [lambda: C.check_chunk_dense(oracle.chunk_prefill)]


def _mut_row_no_scale(q, k, v, scale):
    return _orig_row(q, k, v, 1.0)


def _mut_row_sign(q, k, v, scale):
    H = q.shape[0]
    if k.shape[0] == 0:
        return np.zeros((H, v.shape[1])), np.full(H, -np.inf)
    s = scale * (q @ k.T)
    m = s.max(axis=1, keepdims=True)
    w = np.exp(m - s)
    l = w.sum(axis=1, keepdims=True)
    return (w @ v) / l, (m + np.log(l))[:, 0]


def _mut_row_lse_no_max(q, k, v, scale):
    o, lse = _orig_row(q, k, v, scale)
    if k.shape[0] == 0:
        return o, lse
    return o, lse - (scale * (q @ k.T)).max(axis=1)


def _mut_row_v_is_k(q, k, v, scale):
    dv = v.shape[1]
    kk = np.zeros((k.shape[0], dv))
    kk[:, :min(dv, k.shape[1])] = k[:, :dv]
    return _orig_row(q, k, kk, scale)


def _mut_row_transposed_scores(q, k, v, scale):
    # softmax taken over heads instead of slots
    H = q.shape[0]
    if k.shape[0] == 0:
        return np.zeros((H, v.shape[1])), np.full(H, -np.inf)
    s = scale * (q @ k.T)
    m = s.max(axis=0, keepdims=True)
    w = np.exp(s - m)
    l = w.sum(axis=0, keepdims=True)
    w = w / l
    return w @ v, (s.max(axis=1) + np.log(np.exp(s - s.max(axis=1, keepdims=True)).sum(1)))


def _mut_row_last_term_dropped(q, k, v, scale):
    if k.shape[0] > 1:
        return _orig_row(q, k[:-1], v[:-1], scale)
    return _orig_row(q, k, v, scale)


def _mut_valid_no_neg(idx_row, kv_len, limit):
    j = np.arange(idx_row.shape[0])
    ok = idx_row < kv_len
    if limit is not None:
        ok &= j < limit
    return idx_row[ok].astype(np.int64)


def _mut_valid_off_by_one(idx_row, kv_len, limit):
    j = np.arange(idx_row.shape[0])
    ok = (idx_row >= 0) & (idx_row < kv_len - 1)
    if limit is not None:
        ok &= j < limit
    return idx_row[ok].astype(np.int64)


def _mut_valid_dedup(idx_row, kv_len, limit):
    return np.unique(_orig_valid(idx_row, kv_len, limit))


_orig_row = oatt.row_attention
_orig_valid = oatt._valid_slots

ROW_MUTANTS = [_mut_row_no_scale, _mut_row_sign, _mut_row_lse_no_max, _mut_row_v_is_k,
               _mut_row_transposed_scores, _mut_row_last_term_dropped]
VALID_MUTANTS = [_mut_valid_no_neg, _mut_valid_off_by_one, _mut_valid_dedup]


@pytest.mark.parametrize("mutant", ROW_MUTANTS, ids=lambda m: m.__name__)
def test_pins_catch_row_mistakes(monkeypatch, mutant):
    monkeypatch.setattr(oatt, "row_attention", mutant)
    assert _fails_some(_attn_checks())


@pytest.mark.parametrize("mutant", VALID_MUTANTS, ids=lambda m: m.__name__)
def test_pins_catch_validity_mistakes(monkeypatch, mutant):
    monkeypatch.setattr(oatt, "_valid_slots", mutant)
    assert _fails_some(_attn_checks())


def test_pins_catch_head_mapping(monkeypatch):
    orig = oatt.sparse_attention

    def wrong_mapping(q, k, v, idx, *, num_kv_heads, **kw):
        # head h served by KV head h % Hkv instead of h // group
        Hq = q.shape[1]
        group = Hq // num_kv_heads
        perm = np.array([(h % num_kv_heads) * group + h // num_kv_heads for h in range(Hq)])
        o, l = orig(q[:, perm], k, v, idx, num_kv_heads=num_kv_heads, **kw)
        inv = np.argsort(perm)
        return o[:, inv], l[:, inv]

    assert _fails_some([lambda c=c: c(wrong_mapping) for c in C.ATTN_CHECKS])


def test_pins_catch_chunk_kv_base():
    def wrong_base(q, k, v, idx, cu_q, cu_kv, **kw):
        # every request reads its KV from the start of the packed buffer
        lens = np.diff(np.asarray(cu_kv))
        out_o, out_l = [], []
        for r in range(len(lens)):
            rows = np.arange(cu_q[r], cu_q[r + 1])
            o, l = oracle.sparse_attention(q, k[:lens[r]], v[:lens[r]], idx, kv_len=int(lens[r]),
                                           rows=rows, **kw)
            out_o.append(o)
            out_l.append(l)
        return np.concatenate(out_o), np.concatenate(out_l)

    assert _fails_some([lambda: C.check_chunk_dense(wrong_base)])


# union mutants -----------------------------------------------------------

def _union_variant(kind):
    def build(idx, kv_len, G):
        T, k = idx.shape
        ng = (T + G - 1) // G
        ui = np.full((ng, G * k), -1, np.int32)
        ub = np.zeros((ng, G * k), np.uint8)
        ul = np.zeros(ng, np.int32)
        for g in range(ng):
            members = range(g * G, min(g * G + G, T))
            if kind == "keep_invalid":
                sets = [set(int(x) for x in idx[t] if int(x) < kv_len) for t in members]
            else:
                sets = [set(int(x) for x in idx[t] if 0 <= int(x) < kv_len) for t in members]
            em, earlier = [], set()
            for s in sets:
                for x in (sorted(s, reverse=True) if kind == "descending" else sorted(s)):
                    if kind == "duplicates" or x not in earlier:
                        em.append(x)
                earlier |= s
            for r, x in enumerate(em):
                bits = 0
                for j, s in enumerate(sets):
                    if x in s:
                        bj = (G - 1 - j) if kind == "reversed_bits" else j
                        bits |= 1 << bj
                        if kind == "first_owner_only":
                            break
                ui[g, r], ub[g, r] = x, bits
            ul[g] = len(em)
        return ui, ub, ul
    return build


@pytest.mark.parametrize("kind", ["keep_invalid", "descending", "duplicates",
                                  "reversed_bits", "first_owner_only"])
def test_pins_catch_union_mistakes(kind):
    bad = _union_variant(kind)
    assert _fails_some([
        lambda: C.check_union_golden(bad),
        lambda: C.check_union_contract(bad),
        lambda: C.check_union_equals_per_token(oracle.union_attention, oracle.sparse_attention, bad),
    ])


def test_pins_catch_union_attention_bit_order():
    def bad_attention(q, k, v, ui, ub, ul, G, **kw):
        flipped = np.zeros_like(ub)
        for j in range(G):
            flipped |= ((ub >> j) & 1) << (G - 1 - j)
        return oracle.union_attention(q, k, v, ui, flipped.astype(np.uint8), ul, G, **kw)

    assert _fails_some([lambda: C.check_union_equals_per_token(
        bad_attention, oracle.sparse_attention, oracle.union_build)])


# page mutants ------------------------------------------------------------

def test_pins_catch_page_mistakes():
    def mark(idx, P, ptok, shift=0, size=None):
        size = ptok if size is None else size
        m = np.zeros(P, np.int8)
        for t in np.asarray(idx).ravel():
            if 0 <= t < P * ptok:
                m[min(P - 1, t // size + shift)] = 1
        return m

    for bad in (lambda i, P, pt: mark(i, P, pt, shift=1), lambda i, P, pt: mark(i, P, pt, size=2 * pt)):
        assert _fails_some([lambda b=bad: C.check_page_mark(b)])

    def split_ignores_mask(src, dst, mask, **kw):
        return oracle.page_split(src, dst, None, **kw)

    def split_scale_offset(src, dst, mask, **kw):
        out = oracle.page_split(src, dst, mask, **kw)
        # scales taken from the start of the source page's scale block
        dtok, rb, sb, stok = kw["dst_page_tokens"], kw["row_bytes"], kw["scale_bytes"], kw["src_page_tokens"]
        for p in range(src.shape[0]):
            if mask is None or mask[p]:
                for s in range(stok // dtok):
                    out[p * (stok // dtok) + s, dtok * rb:dtok * (rb + sb)] = src[p, stok * rb:stok * rb + dtok * sb]
        return out

    for bad in (split_ignores_mask, split_scale_offset):
        assert _fails_some([lambda b=bad: C.check_page_split(b)])


# ragged union -------------------------------------------------------------

def _one_request_build(idx, kv_len, G):
    ui, ub, ul, _ = oracle.chunk_union_build(idx, np.array([0, idx.shape[0]], np.int32),
                                             np.array([0, kv_len], np.int64), G)
    return ui, ub, ul


def test_chunk_union_single_request_is_the_union_build():
    # one request reduces to the pinned single-batch contract and fixture
    C.check_union_golden(_one_request_build)
    C.check_union_contract(_one_request_build)


def test_chunk_union_dense():
    C.check_chunk_union_dense(oracle.chunk_union_build, oracle.chunk_union_attention)


def test_chunk_union_equals_per_token():
    C.check_chunk_union_equals_per_token(oracle.chunk_union_build, oracle.chunk_union_attention,
                                         oracle.chunk_prefill)


def test_pins_catch_chunk_union_mistakes():
    # groups formed over the whole batch, spanning requests
    def spanning(idx, cu_q, cu_kv, G):
        ui, ub, ul = oracle.union_build(idx, int(cu_kv[-1]), G)
        starts = np.arange(0, idx.shape[0], G)
        return ui, ub, ul, (np.searchsorted(cu_q, starts, side="right") - 1).astype(np.int32)
    assert _fails_some([lambda: C.check_chunk_union_dense(spanning, oracle.chunk_union_attention)])
    # attention reading from the start of the KV buffer, not the request's range
    assert _fails_some([lambda: C.check_chunk_union_dense(oracle.chunk_union_build,
                                                          _no_base_attention)])
    # validity checked against the whole KV buffer, not the request's length
    assert _fails_some([lambda: C.check_chunk_union_dense(_loose_build,
                                                          oracle.chunk_union_attention)])


def _no_base_attention(q, k, v, ui, ub, ul, gr, cu_q, cu_kv, G, *, num_kv_heads, scale,
                       head_dim_v=None, rows=None):
    T = q.shape[0]
    dv = v.shape[2]
    out = np.zeros((T, q.shape[1], dv))
    lse = np.zeros((T, q.shape[1]))
    for r in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[r]), int(cu_q[r + 1])
        if q1 <= q0:
            continue
        g = np.flatnonzero(gr == r)
        o, s = oracle.union_attention(q[q0:q1], k, v, ui[g], ub[g], ul[g], G,
                                      num_kv_heads=num_kv_heads, scale=scale)
        out[q0:q1], lse[q0:q1] = o, s
    return out, lse


def _loose_build(idx, cu_q, cu_kv, G):
    parts = []
    for r in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[r]), int(cu_q[r + 1])
        if q1 <= q0:
            continue
        ui, ub, ul = oracle.union_build(idx[q0:q1], int(cu_kv[-1]), G)
        parts.append((ui, ub, ul, np.full(len(ul), r, np.int32)))
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(4))


# FP8 MLA records ----------------------------------------------------------

def test_fp8_decode():
    C.check_fp8_decode(oracle.fp8_e4m3_to_f64)


def test_mla_fp8_rows():
    C.check_mla_fp8_rows(oracle.mla_fp8_rows_to_f64)


def _fnuz(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e, m = (c >> 3) & 0xF, (c & 7).astype(np.float64)
    v = np.where(e == 0, m / 8 * 2.0 ** -7, (1 + m / 8) * np.exp2(e - 8.0))
    return np.where(c & 0x80, -v, v)


def test_pins_catch_fp8_mistakes():
    assert _fails_some([lambda: C.check_fp8_decode(_fnuz)])
    from oracle import fp8 as F

    def blocks64(rows):
        r = np.ascontiguousarray(rows)
        lat = F.fp8_e4m3_to_f64(r[..., :512])
        sc = r[..., 512:528].copy().view("<f4").astype(np.float64)
        lat = lat * np.tile(np.repeat(sc, 64, axis=-1), 2)    # scales per 64 values
        rope = oracle.bf16_to_f64(r[..., 528:].copy().view("<u2"))
        return np.concatenate([lat, rope], axis=-1)

    def rope_shift(rows):
        r = np.ascontiguousarray(rows)
        lat = F.fp8_e4m3_to_f64(r[..., :512]) * np.repeat(
            r[..., 512:528].copy().view("<f4").astype(np.float64), 128, axis=-1)
        rope = oracle.bf16_to_f64(r[..., 512:640].copy().view("<u2"))
        return np.concatenate([lat, rope], axis=-1)

    def big_endian(rows):
        r = np.ascontiguousarray(rows)
        lat = F.fp8_e4m3_to_f64(r[..., :512]) * np.repeat(
            r[..., 512:528].copy().view(">f4").astype(np.float64), 128, axis=-1)
        rope = oracle.bf16_to_f64(r[..., 528:].copy().view("<u2"))
        return np.concatenate([lat, rope], axis=-1)

    def exact_product(rows):
        r = np.ascontiguousarray(rows)
        lat = F.fp8_e4m3_to_f64(r[..., :512]) * np.repeat(
            r[..., 512:528].copy().view("<f4").astype(np.float64), 128, axis=-1)
        rope = oracle.bf16_to_f64(r[..., 528:].copy().view("<u2"))
        return np.concatenate([lat, rope], axis=-1)

    for bad in (blocks64, rope_shift, big_endian, exact_product):
        assert _fails_some([lambda: C.check_mla_fp8_rows(bad)]), bad.__name__


# sparse MLA decode over split pages ---------------------------------------

def test_paged_decode_closed_form():
    C.check_paged_decode_closed_form(oracle.paged_decode)


def test_paged_decode_vs_source():
    C.check_paged_decode_vs_source(oracle.paged_decode, oracle.sparse_attention,
                                   oracle.mla_fp8_rows_to_f64)


def _decode_mutant(record, tokens_of=None, dedupe=False):
    """oracle.paged_decode with its record lookup (or validity bound, or
    multiplicity) replaced."""
    from oracle import decode as D

    def run(q, pool, idx, *, page_tokens, scale, topk_len=None, row_bytes=656):
        B, Hq, _ = q.shape
        tokens = pool.shape[0] * page_tokens if tokens_of is None else tokens_of(pool, page_tokens)
        out, lse = np.zeros((B, Hq, 512)), np.zeros((B, Hq))
        for b in range(B):
            lim = idx.shape[1] if topk_len is None else max(0, min(int(topk_len[b]), idx.shape[1]))
            tok = [int(t) for t in idx[b, :lim] if 0 <= t < tokens]
            if dedupe:
                tok = sorted(set(tok))
            rec = np.zeros((len(tok), 656), np.uint8)
            for i, t in enumerate(tok):
                rec[i] = record(pool, t, page_tokens)
            rows = oracle.mla_fp8_rows_to_f64(rec)
            out[b], lse[b] = oracle.row_attention(oracle.bf16_to_f64(q[b]), rows, rows[:, :512], scale)
        return out, lse
    return run


def _decode_checks(fn):
    return [lambda: C.check_paged_decode_closed_form(fn),
            lambda: C.check_paged_decode_vs_source(fn, oracle.sparse_attention,
                                                   oracle.mla_fp8_rows_to_f64)]


def test_pins_catch_decode_mistakes():
    def src_pages(pool, t, ptok):             # 256-token source geometry on 64-token pages
        p, r = divmod(t, 256)
        return pool[p, r * 656:(r + 1) * 656]

    def pitch660(pool, t, ptok):              # row pitch counts the per-token word
        p, r = divmod(t, ptok)
        return pool[p, r * 660:r * 660 + 656]

    def scales_first(pool, t, ptok):          # per-token words before the rows
        p, r = divmod(t, ptok)
        return pool[p, ptok * 4 + r * 656:ptok * 4 + (r + 1) * 656]

    def good(pool, t, ptok):
        return oracle.paged_record(pool, t, page_tokens=ptok)

    mutants = [_decode_mutant(src_pages), _decode_mutant(pitch660), _decode_mutant(scales_first),
               _decode_mutant(good, dedupe=True),
               _decode_mutant(good, tokens_of=lambda pool, ptok: pool.shape[0] * 256)]   # source-page bound
    for m in mutants:
        assert _fails_some(_decode_checks(m))
    # the unmutated copy passes, so the mutants fail for their mistake alone
    for chk in _decode_checks(_decode_mutant(good)):
        chk()


# indexer top-k selection ---------------------------------------------------

def test_topk_rank_count():
    C.check_topk_rank_count(oracle.topk_select)


def test_topk_library():
    C.check_topk_library(oracle.topk_select)


def test_topk_closed_forms():
    C.check_topk_closed_forms(oracle.topk_select)


def _topk_mutant(order_of, n_of=lambda rl, kv: min(int(rl), kv), pad=-1, ascending=True):
    def run(scores, k, row_len=None):
        T, kv = scores.shape
        out = np.full((T, k), pad, np.int32)
        for t in range(T):
            n = kv if row_len is None else max(0, n_of(row_len[t], kv))
            if n <= k:
                out[t, :n] = np.arange(n)
                continue
            sel = np.sort(order_of(scores[t, :n])[:k])
            out[t] = sel if ascending else sel[::-1]
        return out
    return run


def test_pins_catch_topk_mistakes():
    good = lambda v: np.lexsort((np.arange(len(v)), -v.astype(np.float64)))
    high_ties = lambda v: np.lexsort((-np.arange(len(v)), -v.astype(np.float64)))
    bits = lambda v: np.lexsort((np.arange(len(v)),
                                 -np.where(np.signbit(v) & (v == 0), -1e-300, v.astype(np.float64))))
    mutants = [_topk_mutant(high_ties), _topk_mutant(bits), _topk_mutant(good, ascending=False),
               _topk_mutant(good, n_of=lambda rl, kv: min(int(rl) + 1, kv)),
               _topk_mutant(good, n_of=lambda rl, kv: kv), _topk_mutant(good, pad=0)]
    checks = lambda f: [lambda: C.check_topk_rank_count(f), lambda: C.check_topk_library(f),
                        lambda: C.check_topk_closed_forms(f)]
    for m in mutants:
        assert _fails_some(checks(m))
    for chk in checks(_topk_mutant(good)):
        chk()
