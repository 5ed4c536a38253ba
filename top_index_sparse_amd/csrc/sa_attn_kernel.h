// Index-gathered sparse attention forward: one kernel template for gfx950.
//
// What it computes (sglang PR 37275, "Motivation" and the mechanism note
// under it; PR 32779, "Motivation" and "Modifications"): every query row
// gathers its own selected K/V slots; the query heads that share a KV head
// are padded into one 16-row matrix tile; the online softmax stays in
// registers and no split partials reach HBM. In union mode several adjacent
// rows share one deduplicated slot list, and a per-slot ownership bitmask
// restores each row's own support (PR 32779, --dsa-triton-union).
//
// gfx950 design. One wavefront owns one 16-column tile of query rows (the
// heads of one row for the per-token paths; up to 16 / group rows of a union
// group for the union path) and streams that tile's slot list in tiles of 16
// slots. The MFMA operand layouts are chosen so that every gathered byte goes
// from global memory straight into the register where the matrix core wants
// it, with no LDS and no barrier:
//
//   Slot indices: lane (g = l/16, m = l%16) loads the index of slot
//     4g + (m & 3) and turns it into the slot's K and V row byte offsets
//     (one 32 x 32 -> 64-bit multiply per stride for all 16 slots); a DPP
//     quad broadcast hands slots 4g..4g+3 to all sixteen lanes of group g.
//   S^T[slot, col] = K_tile(16 x DQK) . Q^T(DQK x 16)       mfma 16x16x32 bf16
//     lane (g, m) loads the K rows of slots 4g+i at bytes 256h + 16m and
//     writes them to a wave-private LDS tile, from which lane (g, m) reads
//     slot m at d = 32s + 8g (the A operand).
//   P^T = exp2(S^T - max): the S^T accumulator (lane (g, n) holds slots
//     4g..4g+3 of column n) is already the B operand of the next product.
//   O^T[d, col] += V^T(16 x 16 slots) . P^T(16 slots x 16)   mfma 16x16x16 bf16
//     lane (g, m) loads the V rows of slots 4g+i (i < 4) at bytes 256h + 16m
//     (h < DV/128): sixteen lanes read 256 contiguous bytes of one row.
//     In M-tile mt, row m of the A operand stands for
//     d = 128(mt/8) + 8m + mt%8, element mt%8 of chunk mt/8 that the lane
//     already holds, so V needs no transpose.
//   All O^T accumulators of lane (g, n) belong to column n, whose running
//   max and partial sum the lane holds after two cross-lane max steps per
//   tile; the sum is accumulated from the unrounded fp32 probabilities. The
//   reference max only moves when a score passes it by more than kSlack
//   (log2 units), so the O^T rescale is rare; probabilities up to 2^kSlack
//   are exact in fp32 and bf16 rounding is relative, so nothing is lost.
//
// With WSPLIT = 2 a 16-column tile is shared by two wavefronts: each
// computes half of the S^T k-steps (the two partial accumulators are summed
// through a 2 KB LDS exchange, one barrier per slot tile, in the same order
// in both waves so their softmax state stays bitwise identical) and half of
// the O^T d-columns. That halves the registers per wavefront, so more
// wavefronts (and more gathered bytes) are in flight per SIMD.
//
// With WSPLIT = 1, four independent wavefronts form a workgroup; with
// WSPLIT = 2 a workgroup holds the two wavefronts of one column tile. The
// block id is remapped so that each XCD (own L2) works on a
// contiguous band of rows, which share most of their slots. Invalid slots (outside [0, kv_len), past topk or
// topk_len, or owned by none of the wave's rows) issue no memory traffic
// and are masked to -inf before the softmax.
#pragma once

#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

// kPaired / kPairedRagged: per-token results computed for two consecutive
// rows per wavefront; each slot position either serves both rows (same
// token) or is split, the second row's differing tokens being queued and
// gathered as extra tiles.
enum : int { kPerToken = 0, kRagged = 1, kUnion = 2, kPaired = 3, kPairedRagged = 4 };

// Headroom of the running max in log2 units: probabilities stay <= 2^kSlack.
constexpr float kSlack = 8.f;


template <int DQK, int DV, bool V_IN_K, int MODE, int NBUF, int WSPLIT>
struct AttnTile {
  static constexpr int KSTEPS = DQK / 32 / WSPLIT;   // this wave's k-steps of S^T
  static constexpr int VCH = DV / 128 / WSPLIT;      // this wave's 16-byte V chunks per slot
  static constexpr int MTILES = DV / 16 / WSPLIT;    // this wave's 16-wide d blocks of O^T
  static_assert(DQK % (32 * WSPLIT) == 0 && DV % (128 * WSPLIT) == 0, "head dims");
  static constexpr bool UNION = MODE == kUnion;
  static constexpr bool PAIRED = MODE == kPaired || MODE == kPairedRagged;
  static constexpr bool OWN = UNION || PAIRED;      // per-slot ownership bits
  static_assert(!PAIRED || NBUF == 1, "the pair queue reuses the data buffer");
  // V inside the latent K row: the wave's K slice is its V columns
  // [split*MAIN, +MAIN) plus its rope columns [DV + split*ROPE, +ROPE), so V
  // is part of the one gathered slice and both operands are read from LDS.
  static constexpr int MAIN = DV / WSPLIT;
  static constexpr int ROPE = (DQK - DV) / WSPLIT;
  static constexpr bool VKLDS = V_IN_K && MAIN % 32 == 0 && ROPE % 32 == 0;
  static constexpr int CPR = VKLDS ? (MAIN + ROPE) / 8 : 1;  // 16-byte chunks per slot row
  // K staged through LDS when this wave's K slice is a whole number of
  // 256-byte halves per slot (16 lanes x 16 B each).
  static constexpr bool KLDS = !VKLDS && KSTEPS % 4 == 0;
  static_assert(KLDS || VKLDS, "K is staged through LDS");
  static_assert(!V_IN_K || VKLDS, "V inside K is read from the staged K slice");
  static constexpr int KCH = KLDS ? KSTEPS / 4 : 0;   // 16-byte K chunks per slot per lane
  static constexpr int KROW = 64 * KSTEPS + 16;       // LDS row pitch (bytes): 16 (mod 32) * odd
  static constexpr int KLDS_BYTES = (KLDS || VKLDS) ? 16 * KROW : 16;
  // wavefronts per workgroup: four independent column tiles, or the
  // WSPLIT halves of one column tile
  static constexpr int WG_WAVES = WSPLIT == 1 ? 4 : WSPLIT;

  struct Idx {
    int xk;          // index of slot 4g + (m & 3) at lane (g, m)
    uint32_t bk;     // its ownership bits (union, paired)
    int xb;          // paired: the second row's index at the same position
  };
  struct Data {
    u32x4_t kd[KSTEPS];    // raw K chunks, staged through LDS before the MFMA
    u32x4_t vd[4 * VCH];   // vd[VCH*i + h]: slot 4g+i, d = 128h + 8m .. +7
    uint32_t vmask;        // bit i: slot 4g+i contributes to this lane's column
  };
};

// One 16-column tile of query rows (the virtual wave `wave_id`), or its half
// `split` of WSPLIT. xch is the workgroup's exchange buffer [2][4][64].
template <int DQK, int DV, bool V_IN_K, int MODE, int NBUF, int WSPLIT>
__device__ __forceinline__ void attn_wave(const AttnParams& p, int wave_id, int split,
                                          f32x4_t (*xch)[64], uint8_t* klds, int32_t* pqs) {
  using TT = AttnTile<DQK, DV, V_IN_K, MODE, NBUF, WSPLIT>;
  constexpr int KSTEPS = TT::KSTEPS;
  constexpr int VCH = TT::VCH;
  constexpr int MTILES = TT::MTILES;
  constexpr bool UNION = TT::UNION;
  constexpr bool PAIRED = TT::PAIRED;
  constexpr bool OWN = TT::OWN;
  constexpr bool VKLDS = TT::VKLDS;
  constexpr int KCH = TT::KCH;
  constexpr int KROW = TT::KROW;
  constexpr int MAIN = TT::MAIN;
  constexpr int ROPE = TT::ROPE;
  constexpr int CPR = TT::CPR;
  constexpr int TILE = 16;
  using Idx = typename TT::Idx;
  using Data = typename TT::Data;

  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int n = lane & 15;
  const int group = p.group;

  // ---- which rows this wave serves ------------------------------------
  int kvh, t_col;            // KV head; query row of column n
  bool col_live;             // column n is a real (row, head)
  int head_col;              // query head of column n
  uint32_t col_bit = 0;      // union: ownership bit of column n's row
  uint32_t wave_bits = 0;    // union: bits of all rows this wave serves
  const int32_t* irow;       // slot list
  const uint8_t* brow = nullptr;
  int jmax;
  int64_t kv_base = 0;
  int kv_len = p.kv_len;
  // paired: the two rows' request bases, lengths, index rows and limits
  int64_t base0 = 0, base1 = 0;
  int len0 = p.kv_len, len1 = p.kv_len, jmax0 = 0, jmax1 = 0;
  const int32_t* irow1 = nullptr;
  if (PAIRED) {
    const int pairs = (p.num_rows + 1) >> 1;
    const int pairs4 = (pairs + 3) & ~3;
    kvh = wave_id / pairs4;
    const int pr = wave_id - kvh * pairs4;
    if (pr >= pairs || kvh >= p.num_kv_heads) return;
    const int t0 = 2 * pr;
    const int rows = t0 + 1 < p.num_rows ? 2 : 1;
    const int j = n / group;
    col_live = n < rows * group;
    head_col = kvh * group + (n - j * group);
    t_col = t0 + (col_live ? j : 0);
    col_bit = col_live ? (1u << j) : 0u;
    wave_bits = rows == 2 ? 3u : 1u;
    auto request = [&](int t, int64_t& base, int& len) {
      int lo = 0, hi = p.num_reqs - 1;  // last request whose first row is <= t
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.cu_q[mid] <= t) lo = mid; else hi = mid - 1;
      }
      base = p.cu_kv[lo];
      len = (int)(p.cu_kv[lo + 1] - base);
    };
    if (MODE == kPairedRagged) {
      request(t0, base0, len0);
      if (rows == 2) request(t0 + 1, base1, len1);
    }
    auto limit = [&](int t, int len) {
      int jm = p.topk;
      if (p.topk_len) {
        const int tl = p.topk_len[t];
        jm = tl < 0 ? 0 : (tl < jm ? tl : jm);
      }
      return len > 0 ? jm : 0;
    };
    jmax0 = limit(t0, len0);
    jmax1 = rows == 2 ? limit(t0 + 1, len1) : 0;
    irow = p.idx + (int64_t)t0 * p.idx_row_stride;
    irow1 = irow + p.idx_row_stride;
    jmax = jmax0 > jmax1 ? jmax0 : jmax1;
    kv_len = 0x7fffffff;   // slots carry global token ids; -1 marks invalid
  } else if (UNION) {
    const int per_head = p.num_groups * p.waves_per_group;
    kvh = wave_id / per_head;
    if (kvh >= p.num_kv_heads) return;
    const int r = wave_id - kvh * per_head;
    const int gi = r / p.waves_per_group;
    const int ts = r - gi * p.waves_per_group;
    const int j0 = ts * p.tokens_per_wave;                     // first member served
    int members = p.G - j0;
    if (members > p.tokens_per_wave) members = p.tokens_per_wave;
    const int tail = p.num_rows - gi * p.G - j0;             // rows that exist
    if (members > tail) members = tail;
    if (members <= 0) return;   // the whole workgroup (one column tile) leaves
    const int j = n / group;
    col_live = j < members;
    head_col = kvh * group + (n - j * group);
    t_col = gi * p.G + j0 + (col_live ? j : 0);
    col_bit = col_live ? (1u << (j0 + j)) : 0u;
    wave_bits = ((1u << members) - 1u) << j0;
    irow = p.union_idx + (int64_t)gi * p.union_stride;
    brow = p.union_bits + (int64_t)gi * p.union_stride;
    jmax = p.union_len[gi];
  } else {
    const int quads = (p.num_rows + 3) >> 2;
    kvh = wave_id / (quads * 4);
    const int t = wave_id - kvh * quads * 4;
    if (t >= p.num_rows || kvh >= p.num_kv_heads) return;
    col_live = n < group;
    head_col = kvh * group + n;
    t_col = t;
    if (MODE == kRagged) {
      int lo = 0, hi = p.num_reqs - 1;  // last request whose first row is <= t
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.cu_q[mid] <= t) lo = mid; else hi = mid - 1;
      }
      kv_base = p.cu_kv[lo];
      kv_len = (int)(p.cu_kv[lo + 1] - kv_base);
    }
    irow = p.idx + (int64_t)t * p.idx_row_stride;
    jmax = p.topk;
    if (p.topk_len) {
      const int tl = p.topk_len[t];
      jmax = tl < 0 ? 0 : (tl < jmax ? tl : jmax);
    }
  }
  if (kv_len <= 0) jmax = 0;
  const int ntiles = (jmax + TILE - 1) / TILE;

  const int wv = threadIdx.x >> 6;
  // Wave-uniform K/V bases; lane offsets are added per load.
  const uint16_t* kw = p.k + kv_base * p.k_row_stride + kvh * DQK + (VKLDS ? 0 : 32 * KSTEPS * split);
  const uint16_t* vw = p.v + kv_base * p.v_row_stride + kvh * (V_IN_K ? DQK : DV) + 128 * VCH * split;

  // ---- Q^T operand: lane (g, n) holds column n, d = 32s + 8g .. +7 -------
  u32x4_t qop[KSTEPS];
  {
    const uint16_t* qp = p.q + (int64_t)t_col * p.q_row_stride + (int64_t)head_col * DQK + 8 * g;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      // d of k-step s: the wave's slice in k-step order
      const int d = VKLDS ? (s < MAIN / 32 ? split * MAIN + 32 * s : DV + split * ROPE + 32 * (s - MAIN / 32))
                          : 32 * KSTEPS * split + 32 * s;
      qop[s] = col_live ? ld16(qp + d) : (u32x4_t){0, 0, 0, 0};
    }
  }

  // One index (and ownership byte) load per lane per tile: lane (g, m)
  // reads slot 4g + (m & 3), so each quad of lanes holds the four slots
  // whose rows lane group g gathers.
  const int own_slot = 4 * g + (n & 3);
  auto load_idx = [&](Idx& ti, int j0) {
    const int jk = j0 + own_slot;
    if (PAIRED) {
      ti.xk = jk < jmax0 ? irow[jk] : -1;
      ti.xb = jk < jmax1 ? irow1[jk] : -1;
    } else {
      ti.xk = jk < jmax ? irow[jk] : -1;
    }
    if (UNION) ti.bk = jk < jmax ? (uint32_t)brow[jk] : 0u;
  };

  // Paired rows: position m serves both rows when they select the same
  // token; otherwise the second row's token is queued (per wave, in LDS)
  // and gathered later with other queued tokens as a tile of its own.
  int32_t* pq = pqs + (threadIdx.x >> 6) * 32;
  int qcount = 0;
  auto resolve_pair = [&](Idx& ti) {
    const int ga = (unsigned)ti.xk < (unsigned)len0 ? (int)(base0 + ti.xk) : -1;
    const int gb = (unsigned)ti.xb < (unsigned)len1 ? (int)(base1 + ti.xb) : -1;
    const bool same = ga >= 0 && ga == gb;
    const bool diff = gb >= 0 && !same;
    ti.xk = ga;
    ti.bk = (ga >= 0 ? 1u : 0u) | (same ? 2u : 0u);
    // one lane per slot: lanes (g, 0..3) hold slots 4g .. 4g+3
    const uint64_t dm = (uint64_t)__ballot(diff) & 0x000f000f000f000full;
    if (n < 4 && diff) pq[qcount + __popcll(dm & ((1ull << lane) - 1ull))] = gb;
    qcount += __popcll(dm);
  };

  // Invalid slots skip their loads. Their K registers keep stale values
  // (their scores are forced to -inf), and their V registers keep stale
  // finite values from an earlier tile, or the zeros set before the loop,
  // which are multiplied by p = 0.
  const uint32_t k_row_bytes = (uint32_t)(2 * p.k_row_stride);   // < 2^32 (host check)
  const uint32_t v_row_bytes = (uint32_t)(2 * p.v_row_stride);
  const uint8_t* kwb = reinterpret_cast<const uint8_t*>(kw);
  const uint8_t* kbn = kwb + 16 * n;   // this lane's 16 bytes of a 256-byte half row
  const uint8_t* vbn = reinterpret_cast<const uint8_t*>(vw) + 16 * n;
  auto load_data = [&](Data& td, const Idx& ti) {
    // Byte offsets of this lane's slot rows; -1 when no row of this wave
    // uses the slot.
    bool ok = (unsigned)ti.xk < (unsigned)kv_len;
    if (OWN) ok = ok && (ti.bk & wave_bits);
    const int64_t koff = ok ? (int64_t)((uint64_t)(uint32_t)ti.xk * k_row_bytes) : -1;
    int khi[4];
    quad_bcast4((int)(koff >> 32), khi);
    uint32_t mask = 0;
    if (OWN) {
      int bq[4];
      quad_bcast4((int)ti.bk, bq);
#pragma unroll
      for (int i = 0; i < 4; ++i) mask |= (uint32_t)(khi[i] >= 0 && ((uint32_t)bq[i] & col_bit)) << i;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) mask |= (uint32_t)(khi[i] >= 0) << i;
    }
    td.vmask = mask;   // bit i: slot 4g+i contributes to this lane's column
    if (VKLDS) {
      // Linear chunk order: load c covers chunks 64c .. 64c+63 of the tile's
      // 16 slot rows (CPR chunks each), so consecutive lanes read
      // consecutive 16-byte pieces of the same row. Slot s's offset sits in
      // lane 16(s/4) + s%4; the permutes run with every lane active.
#pragma unroll
      for (int c = 0; c < KSTEPS; ++c) {
        const int q = 64 * c + lane;
        const int slot = q / CPR;
        const int ch = q - slot * CPR;
        const int src = (16 * (slot >> 2) + (slot & 3)) << 2;
        const int lo = __builtin_amdgcn_ds_bpermute(src, (int)koff);
        const int hi = __builtin_amdgcn_ds_bpermute(src, (int)(koff >> 32));
        const int d = ch < MAIN / 8 ? split * MAIN + 8 * ch : DV + split * ROPE + 8 * (ch - MAIN / 8);
        if (hi >= 0) td.kd[c] = ld16(kwb + join64(lo, hi) + 2 * d);
      }
      return;
    }
    const int64_t voff = ok ? (int64_t)((uint64_t)(uint32_t)ti.xk * v_row_bytes) : -1;
    int klo[4], vlo[4], vhi[4];
    quad_bcast4((int)koff, klo);
    quad_bcast4((int)voff, vlo);
    quad_bcast4((int)(voff >> 32), vhi);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (khi[i] >= 0) {
        // K and V rows of slot 4g+i, bytes 256h + 16m: sixteen lanes per row
        const uint8_t* kp = kbn + join64(klo[i], khi[i]);
#pragma unroll
        for (int h = 0; h < KCH; ++h) td.kd[KCH * i + h] = ld16(kp + 256 * h);
        const uint8_t* vp = vbn + join64(vlo[i], vhi[i]);
#pragma unroll
        for (int h = 0; h < VCH; ++h) td.vd[VCH * i + h] = ld16(vp + 256 * h);
      }
    }
  };

  float m_run = -INFINITY;  // running max of column n (log2 domain)
  float l_run = 0.f;        // this lane's share of column n's running sum
  f32x4_t acc[MTILES];
#pragma unroll
  for (int mt = 0; mt < MTILES; ++mt) acc[mt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  const float c = p.scale_log2e;

  int par = 0;
  uint8_t* lk = klds + wv * (16 * KROW);   // this wave's K tile in LDS
  auto compute = [&](const Data& td) {
    f32x4_t st = {0.f, 0.f, 0.f, 0.f};
    if (VKLDS) {
#pragma unroll
      for (int c = 0; c < KSTEPS; ++c) {
        const int q = 64 * c + lane;
        const int slot = q / CPR;
        *reinterpret_cast<u32x4_t*>(lk + slot * KROW + 16 * (q - slot * CPR)) = td.kd[c];
      }
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(lk + n * KROW + 64 * s + 16 * g);
        st = mfma_16x16x32(a, qop[s], st);
      }
    } else {
      // Transpose the gathered K rows into the MFMA A layout through LDS:
      // write slot 4g+i, bytes 256h + 16m; read slot m, bytes 64s + 16g.
      // The pitch KROW = 16 (mod 256) keeps both sides bank-conflict free.
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < KCH; ++h)
          *reinterpret_cast<u32x4_t*>(lk + (4 * g + i) * KROW + 256 * h + 16 * n) = td.kd[KCH * i + h];
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(lk + n * KROW + 64 * s + 16 * g);
        st = mfma_16x16x32(a, qop[s], st);
      }
    }
    if (WSPLIT > 1) {
      // partial S^T of the other half of d; both waves form half0 + half1
      constexpr int WGW = TT::WG_WAVES;
      xch[par * WGW + wv][lane] = st;
      __syncthreads();
      const f32x4_t o = xch[par * WGW + (wv ^ 1)][lane];
      st = split == 0 ? st + o : o + st;
      par ^= 1;
    }
    float s2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s2[i] = ((td.vmask >> i) & 1u) ? st[i] * c : -INFINITY;
    float mx = fmaxf(fmaxf(s2[0], s2[1]), fmaxf(s2[2], s2[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_cand = fmaxf(m_run, mx);
    const float m_new = m_cand > m_run + kSlack ? m_cand : m_run;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(s2[i] - m_use);
    l_run = l_run * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    // Rescale only when some column's reference max moved (alpha == 1
    // elsewhere).
    if (__builtin_amdgcn_ballot_w64(m_new != m_run)) {
#pragma unroll
      for (int mt = 0; mt < MTILES; ++mt) acc[mt] *= alpha;
    }
    m_run = m_new;
    const i16x4_t pop = __builtin_bit_cast(
        i16x4_t, (u32x2_t){pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])});
    u32x4_t vv[4 * VCH];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < VCH; ++h)
        vv[VCH * i + h] = VKLDS ? *reinterpret_cast<const u32x4_t*>(lk + (4 * g + i) * KROW + 256 * h + 16 * n)
                                : td.vd[VCH * i + h];
#pragma unroll
    for (int mt = 0; mt < MTILES; ++mt) {
      const int h = mt >> 3, e = mt & 7;
      const i16x4_t a = gather_col4(vv[h], vv[VCH + h], vv[2 * VCH + h], vv[3 * VCH + h], e);
      acc[mt] = mfma_16x16x16(a, pop, acc[mt]);
    }
  };

  // Software pipeline: NBUF data buffers, NBUF + 1 index buffers. At step
  // `cur` the index loads of tile cur+NBUF are issued first, then the data
  // loads of tile cur+NBUF-1 (whose indices arrived a step earlier), then
  // tile cur is consumed. Loads retire in issue order, so issuing indices
  // before data lets the data of NBUF-1 tiles stay in flight while the
  // indices of the next one are awaited. The loop is unrolled NBUF*(NBUF+1)
  // times so every buffer index is a compile-time constant.
  constexpr int NI = NBUF + 1;
  constexpr int UNROLL = NBUF * NI;
  Idx ib[NI];
  Data db[NBUF];

  // Gathers and consumes queued second-row tokens, 16 at a time (all of
  // them when flushing). With one data buffer, the buffer is free here.
  auto run_queue = [&](bool flush) {
    while (qcount >= 16 || (flush && qcount > 0)) {
      Idx si;
      si.xk = own_slot < qcount ? pq[own_slot] : -1;
      si.bk = 2u;
      si.xb = -1;
      load_data(db[0], si);
      compute(db[0]);
      const int rem = qcount > 16 ? qcount - 16 : 0;
      const int v = n < rem ? pq[16 + n] : 0;
      if (g == 0 && n < rem) pq[n] = v;
      qcount = rem;
    }
  };

#pragma unroll
  for (int u = 0; u < NBUF; ++u) {
#pragma unroll
    for (int h = 0; h < 4 * VCH; ++h) db[u].vd[h] = (u32x4_t){0, 0, 0, 0};
    if (VKLDS) {
#pragma unroll
      for (int c = 0; c < KSTEPS; ++c) db[u].kd[c] = (u32x4_t){0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int u = 0; u < NBUF; ++u)
    if (u < ntiles) load_idx(ib[u], u * TILE);
#pragma unroll
  for (int u = 0; u + 1 < NBUF; ++u)
    if (u < ntiles) load_data(db[u], ib[u]);
  for (int tile = 0; tile < ntiles; tile += UNROLL) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int cur = tile + u;
      if (cur >= ntiles) break;
      if (cur + NBUF < ntiles) load_idx(ib[(u + NBUF) % NI], (cur + NBUF) * TILE);
      __builtin_amdgcn_sched_barrier(0);
      if (cur + NBUF - 1 < ntiles) {
        if (PAIRED) resolve_pair(ib[(u + NBUF - 1) % NI]);
        load_data(db[(u + NBUF - 1) % NBUF], ib[(u + NBUF - 1) % NI]);
      }
      __builtin_amdgcn_sched_barrier(0);
      compute(db[u % NBUF]);
      if (PAIRED) run_queue(false);
    }
  }
  if (PAIRED) run_queue(true);

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ---------------------
  float l = l_run + __shfl_xor(l_run, 16);
  l += __shfl_xor(l, 32);
  if (col_live) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* orow = p.out + (int64_t)t_col * p.out_row_stride + (int64_t)head_col * DV;
#pragma unroll
    for (int h = 0; h < VCH; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 128 * (VCH * split + h) + 32 * g + 8 * i;
        const f32x4_t lo = {acc[8 * h + 0][i], acc[8 * h + 1][i], acc[8 * h + 2][i],
                            acc[8 * h + 3][i]};
        const f32x4_t hi = {acc[8 * h + 4][i], acc[8 * h + 5][i], acc[8 * h + 6][i],
                            acc[8 * h + 7][i]};
        st16(orow + d0, lo * inv);
        st16(orow + d0 + 4, hi * inv);
      }
    }
    if (g == 0 && split == 0)
      p.lse[(int64_t)t_col * p.num_q_heads + head_col] =
          l > 0.f ? (m_run + fast_log2(l)) * kLn2 : -INFINITY;
  }
}

// WSPLIT = 1: four independent column tiles ("virtual waves") per
// workgroup. WSPLIT = 2: one column tile per workgroup, its two halves on
// two wavefronts that exchange partial scores through LDS.
template <int DQK, int DV, bool V_IN_K, int MODE, int NBUF, int WSPLIT, int WAVES>
__global__ void __attribute__((amdgpu_flat_work_group_size(64, 256),
                               amdgpu_waves_per_eu(WAVES, WAVES)))
attn_kernel(AttnParams p) {
  using TT = AttnTile<DQK, DV, V_IN_K, MODE, NBUF, WSPLIT>;
  __shared__ f32x4_t xch[(WSPLIT > 1 ? 2 : 1) * TT::WG_WAVES][64];
  __shared__ __attribute__((aligned(16))) uint8_t klds[TT::WG_WAVES * TT::KLDS_BYTES];
  __shared__ int32_t pqs[TT::PAIRED ? TT::WG_WAVES * 32 : 1];
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (WSPLIT == 1)
    attn_wave<DQK, DV, V_IN_K, MODE, NBUF, 1>(p, bid * 4 + w, 0, xch, klds, pqs);
  else
    attn_wave<DQK, DV, V_IN_K, MODE, NBUF, WSPLIT>(p, bid, w, xch, klds, pqs);
}

// Workgroups and threads per workgroup for a launch.
template <int WSPLIT>
inline void attn_grid(const AttnParams& p, int mode, dim3* grid, dim3* block) {
  int64_t vwaves;
  if (mode == kUnion)
    vwaves = (int64_t)p.num_groups * p.waves_per_group * p.num_kv_heads;
  else if (mode == kPaired || mode == kPairedRagged)
    vwaves = (int64_t)((((p.num_rows + 1) >> 1) + 3) & ~3) * p.num_kv_heads;
  else
    vwaves = (int64_t)((p.num_rows + 3) / 4) * 4 * p.num_kv_heads;
  if (WSPLIT == 1) {
    *grid = dim3((unsigned)((vwaves + 3) / 4));
    *block = dim3(256);
  } else {
    *grid = dim3((unsigned)vwaves);
    *block = dim3(64 * WSPLIT);
  }
}

}  // namespace sa
