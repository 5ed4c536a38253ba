"""GPU parity: MLA over 656-byte FP8 latent records (E4M3 latent values with
fp32 block scales, bf16 rope) against the fp64 oracle on the decoded rows."""
import numpy as np
import pytest
import torch

import gen
import oracle
import top_index_sparse_amd as sa
from tests.gpu_util import bf16_dev, check_close, config, i32_dev, i64_dev, sample_rows, say

pytestmark = pytest.mark.gpu


def _dec(case):
    return oracle.mla_fp8_rows_to_f64(case.k)          # float64 [kv, 1, 576]


def _u8_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _small(seed, T, kv, first, Hq, topk):
    return gen.make_attn_case("fp8", seed=seed, num_rows=T, kv_len=kv, first_pos=first,
                              num_q_heads=Hq, num_kv_heads=1, head_dim_qk=576, head_dim_v=512,
                              topk=topk, v_in_k=True, kv_fp8=True)


@pytest.mark.parametrize("Hq", [8, 16, 3, 1, 32])
def test_fp8_small_padding_and_invalid(Hq):
    say(f"[fp8] MLA records, {Hq} heads: -1 padding, out-of-range, duplicates")
    c = _small(70 + Hq, 37, 400, 0, Hq, 256)
    c.idx[5, 3] = 400
    c.idx[9, 10:20] = c.idx[9, 9]
    q, k, idx = bf16_dev(c.q), _u8_dev(c.k), i32_dev(c.idx)
    out, lse = sa.sparse_attn_prefill(q, k, None, idx, sm_scale=c.scale, head_dim_v=512)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_attention(c.q, _dec(c), None, c.idx, num_kv_heads=1, scale=c.scale,
                                     kv_len=c.kv_len, head_dim_v=512)
    check_close(out, lse, ro, rl, f"fp8 Hq={Hq}")


def test_fp8_padded_record_stride():
    say("[fp8] records at a 672-byte stride")
    c = _small(75, 21, 300, 200, 8, 128)
    kp = torch.zeros((300, 1, 672), dtype=torch.uint8, device="cuda")
    kp[:, :, :656] = _u8_dev(c.k)
    out, lse = sa.sparse_attn_prefill(bf16_dev(c.q), kp[:, :, :656], None, i32_dev(c.idx),
                                      sm_scale=c.scale, head_dim_v=512)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_attention(c.q, _dec(c), None, c.idx, num_kv_heads=1, scale=c.scale,
                                     kv_len=c.kv_len, head_dim_v=512)
    check_close(out, lse, ro, rl, "fp8 stride 672")


def test_fp8_c3_per_token_and_union():
    say("[fp8] C3fp8 full size: per-token and union G=2/4, sampled rows")
    c = config("C3fp8")
    kd = _dec(c)
    q, k, idx = bf16_dev(c.q), _u8_dev(c.k), i32_dev(c.idx)
    rows = sample_rows(c.num_rows, 32)
    sel = torch.from_numpy(rows).cuda()
    ro, rl = oracle.sparse_attention(c.q, kd, None, c.idx, num_kv_heads=1, scale=c.scale,
                                     kv_len=c.kv_len, head_dim_v=512, rows=rows)
    po, pl = sa.sparse_attn_prefill(q, k, None, idx, sm_scale=c.scale, head_dim_v=512)
    torch.cuda.synchronize()
    e, el = check_close(po[sel], pl[sel], ro, rl, "C3fp8 per-token")
    say(f"  per-token: max abs err O {e:.2e} LSE {el:.2e}")
    for G in (2, 4):
        uo, ul, st = sa.sparse_attn_prefill_union(q, k, None, idx, G, sm_scale=c.scale,
                                                  head_dim_v=512)
        torch.cuda.synchronize()
        assert st == sa.SA_OK
        check_close(uo[sel], ul[sel], ro, rl, f"C3fp8 union G={G}")
        assert (ul - pl).abs().max().item() < 2e-5
        assert ((uo - po).abs() <= 2e-2 + 1e-2 * po.abs()).all()


def test_fp8_ragged_chunk_prefill():
    say("[fp8] ragged chunk prefill over FP8 records, per-token and union G=2")
    rng = np.random.default_rng(77)
    qlens, ctxs = [9, 0, 14, 5], [700, 100, 900, 300]
    cu_q = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    cu_kv = np.concatenate([[0], np.cumsum(ctxs)]).astype(np.int64)
    T, KV = int(cu_q[-1]), int(cu_kv[-1])
    q = gen.normal_bf16(rng, (T, 8, 576))
    k = gen.mla_fp8_rows(rng, KV).reshape(KV, 1, 656)
    idx = np.concatenate([gen.random_walk_indices(rng, np.arange(c - n, c), 256, swap_frac=0.1)
                          for n, c in zip(qlens, ctxs)]).astype(np.int32)
    scale = 1 / 24
    dq, dk, di = bf16_dev(q), _u8_dev(k), i32_dev(idx)
    dcq, dck = i32_dev(cu_q), i64_dev(cu_kv)
    kd = oracle.mla_fp8_rows_to_f64(k)
    ro, rl = oracle.chunk_prefill(q, kd, None, idx, cu_q, cu_kv, num_kv_heads=1, scale=scale,
                                  head_dim_v=512)
    out, lse = sa.sparse_attn_chunk_prefill(dq, dk, None, di, dcq, dck, sm_scale=scale,
                                            head_dim_v=512)
    torch.cuda.synchronize()
    check_close(out, lse, ro, rl, "fp8 ragged")
    uo, ul, st = sa.sparse_attn_chunk_prefill_union(dq, dk, None, di, dcq, dck, 2, sm_scale=scale,
                                                    head_dim_v=512)
    torch.cuda.synchronize()
    assert st == sa.SA_OK
    check_close(uo, ul, ro, rl, "fp8 ragged union")


@pytest.mark.parametrize("fp8", [False, True])
def test_mla_membership_teams_edge_cases(fp8):
    # Two-row MLA teams (8 heads) match their rows by membership through a
    # bitmap pair the team's two waves share: shuffled slot order, odd request
    # lengths (teams straddling two requests), a request longer than the
    # 32768-token bitmaps, a row holding a token twice and a row of padding
    # fall back to matching by position.
    say(f"[chunk] MLA membership teams ({'FP8 records' if fp8 else 'bf16 rows'}): shuffled, "
        "straddling, long request, duplicates")
    rng = np.random.default_rng(91 + fp8)
    qlens, ctxs, topk = [7, 0, 12, 5, 9], [3000, 500, 33000, 900, 40000], 300
    cu_q = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    cu_kv = np.concatenate([[0], np.cumsum(ctxs)]).astype(np.int64)
    T, KV = int(cu_q[-1]), int(cu_kv[-1])
    q = gen.normal_bf16(rng, (T, 8, 576))
    k = (gen.mla_fp8_rows(rng, KV).reshape(KV, 1, gen.FP8_ROW_BYTES) if fp8
         else gen.normal_bf16(rng, (KV, 1, 576)))
    idx = np.concatenate([gen.random_walk_indices(rng, np.arange(c - n, c), topk)
                          for n, c in zip(qlens, ctxs) if n > 0]).astype(np.int32)
    idx = gen.shuffle_slots(idx, 5)
    idx[2, 10:20] = idx[2, 5]          # duplicates (row 2 and its team mate fall back)
    idx[4, :] = -1                     # an empty row
    idx[9, ::7] = 10 ** 6              # out-of-range slots
    scale = 1 / 24
    kd = oracle.mla_fp8_rows_to_f64(k) if fp8 else k
    out, lse = sa.sparse_attn_chunk_prefill(bf16_dev(q), _u8_dev(k) if fp8 else bf16_dev(k), None,
                                            i32_dev(idx), i32_dev(cu_q), i64_dev(cu_kv),
                                            sm_scale=scale, head_dim_v=512)
    torch.cuda.synchronize()
    ro, rl = oracle.chunk_prefill(q, kd, None, idx, cu_q, cu_kv, num_kv_heads=1, scale=scale,
                                  head_dim_v=512)
    e, el = check_close(out, lse, ro, rl, "MLA membership edge cases")
    say(f"  max abs err O {e:.2e}  LSE {el:.2e}")


def _bf16_bits_to_f64(t):
    return t.view(torch.int16).cpu().numpy().astype(np.uint16).astype(np.uint32) \
        .__lshift__(16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("hkv,pad", [(1, 0), (2, 32)])
def test_fp8_records_to_bf16_exact(hkv, pad):
    # every converted value equals the oracle's dequantised bf16 value bit
    # for bit; masked-off rows keep their previous contents
    say(f"[fp8] records -> bf16 rows, {hkv} KV heads, strides padded by {pad}")
    rng = np.random.default_rng(300 + hkv)
    T = 777
    rec = gen.mla_fp8_rows(rng, T * hkv).reshape(T, hkv, gen.FP8_ROW_BYTES)
    pool = torch.zeros((T, hkv * 656 + pad), dtype=torch.uint8, device="cuda")
    pool[:, :hkv * 656] = _u8_dev(rec).reshape(T, -1)
    pv = pool[:, :hkv * 656].view(T, hkv, 656)
    outb = torch.full((T, hkv * 576 + pad), -7.0, dtype=torch.bfloat16, device="cuda")
    ov = outb[:, :hkv * 576].view(T, hkv, 576)
    sa.fp8_records_to_bf16(pv, out=ov)
    torch.cuda.synchronize()
    want = oracle.mla_fp8_rows_to_f64(rec)
    got = _bf16_bits_to_f64(ov.contiguous())
    assert np.array_equal(got, want)
    assert (outb[:, hkv * 576:] == -7.0).all()
    # masked: only marked tokens are written
    mask = torch.from_numpy((rng.random(T) < 0.3).astype(np.int8)).cuda()
    outm = torch.full((T, hkv, 576), -7.0, dtype=torch.bfloat16, device="cuda")
    sa.fp8_records_to_bf16(pv, mask=mask, out=outm)
    torch.cuda.synchronize()
    m = mask.cpu().numpy().astype(bool)
    gm = _bf16_bits_to_f64(outm)
    assert np.array_equal(gm[m], want[m])
    assert (gm[~m] == -7.0).all()


def test_fp8_staged_chain_matches_oracle():
    # page_mark over one-token pages marks the tokens the index rows touch;
    # the marked records are converted once; the bf16 MLA kernel then runs
    # over the converted rows. Same definition as the FP8 kernels.
    say("[fp8] staged chain: page_mark (one-token pages) -> records to bf16 -> bf16 prefill")
    c = _small(81, 45, 3000, 2950, 8, 400)
    c.idx[3, 5:9] = -1
    c.idx[7, 2] = 5000
    q, k, idx = bf16_dev(c.q), _u8_dev(c.k), i32_dev(c.idx)
    mask = sa.page_mark(idx, c.kv_len, 1)
    rows = torch.empty((c.kv_len, 1, 576), dtype=torch.bfloat16, device="cuda")
    sa.fp8_records_to_bf16(k, mask=mask, out=rows)
    out, lse = sa.sparse_attn_prefill(q, rows, None, idx, sm_scale=c.scale, head_dim_v=512)
    fo, fl = sa.sparse_attn_prefill(q, k, None, idx, sm_scale=c.scale, head_dim_v=512)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_attention(c.q, _dec(c), None, c.idx, num_kv_heads=1, scale=c.scale,
                                     kv_len=c.kv_len, head_dim_v=512)
    check_close(out, lse, ro, rl, "staged fp8")
    say(f"  staged vs in-kernel FP8: max |dO| {(out - fo).abs().max().item():.2e}, "
        f"max |dLSE| {(lse - fl).abs().max().item():.2e}")
