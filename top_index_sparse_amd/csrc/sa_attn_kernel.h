// Index-gathered sparse attention forward: one kernel template for gfx950.
//
// What it computes (sglang PR 37275, "Motivation" and the mechanism note
// under it; PR 32779, "Motivation" and "Modifications"): every query row
// gathers its own selected K/V slots; the query heads that share a KV head
// are padded into 16-row matrix tiles; the online softmax stays in registers
// and no split partials reach HBM. In union mode several adjacent rows share
// one deduplicated slot list, and a per-slot ownership bitmask restores each
// row's own support (PR 32779, --dsa-triton-union).
//
// gfx950 design.
//
// Teams. A team of WSPLIT wavefronts serves query rows of one KV head (up to
// four consecutive rows in the per-token modes, up to eight members of one
// union group in union mode) as C tiles of 16 columns, a column being one
// (row, head).
// Each wavefront computes half of the S^T k-steps and half of the O^T
// d-columns when WSPLIT = 2 (the partial scores are summed through LDS, one
// barrier per slot tile, in the same order in both wavefronts so their
// softmax state stays bitwise identical). Every gathered K/V row feeds the
// products of all C column tiles, so the gathered bytes per row shrink with
// the number of rows a team serves.
//
// Slot tiles. A team streams its slots in tiles of 16. Per-token modes: the
// team's rows are read position by position; a position is gathered once
// for every row that selected the same token there as the team's first row
// (ownership bits say which), and every other token is queued, once per run
// of consecutive rows that share it, to be gathered with other queued tokens
// as a tile of its own. Each row therefore sees each of its slots exactly
// once (duplicates and ragged rows included), as in the per-token
// definition. Two-row teams of one request match by membership instead
// (kRowsMember, below). Union mode: the prebuilt union list with its
// ownership bits.
//
// Index lanes. Lane (g = l/16, m = l%16) reads the index of slot
// 4g + m/4 of row m%4, so each quad of lanes holds one slot of all four rows
// and compares them with quad DPP moves. A DPP row broadcast then hands the
// tokens of slots 4g..4g+3 to all sixteen lanes of group g, which gather
// the rows through buffer descriptors (row index x stride + lane offset;
// launches whose rows span more than 2 GiB, or whose strides do not fit the
// descriptor, turn the token into a 64-bit byte offset instead).
//
// Products (MFMA operand layouts chosen so gathered bytes need no transpose):
//   S^T[slot, col] = K_tile(16 x DQK) . Q^T(DQK x 16)       mfma 16x16x32 bf16
//     lane (g, m) loads the K rows of slots 4g+i at bytes 256h + 16m and
//     writes them to a wave-private LDS tile, from which lane (g, m) reads
//     slot m at d = 32s + 8g (the A operand, shared by the C column tiles).
//   P^T = exp2(S^T - max): the S^T accumulator (lane (g, n) holds slots
//     4g..4g+3 of column n) is already the B operand of the next product.
//   O^T[d, col] += V^T(16 x 16 slots) . P^T(16 slots x 16)   mfma 16x16x16 bf16
//     lane (g, m) loads the V rows of slots 4g+i at bytes 256h + 16m. In
//     M-tile mt, row m of the A operand stands for d = 128(mt/8) + 8m + mt%8,
//     element mt%8 of chunk mt/8 that the lane already holds (two byte
//     permutes per operand), so V needs no transpose.
//   All O^T accumulators of lane (g, n) belong to column n, whose running
//   max and partial sum the lane holds after two cross-lane max steps per
//   tile; the sum is accumulated from the unrounded fp32 probabilities. The
//   reference max only moves when a score passes it by more than kSlack
//   (log2 units), so the O^T rescale is rare; probabilities up to 2^kSlack
//   are exact in fp32 and bf16 rounding is relative, so nothing is lost.
//   MLA (V inside the 576-wide latent row): each wavefront gathers its V
//   columns plus its rope columns and stages the slice in LDS for S^T. With
//   row descriptors the latent chunks are gathered in the V operand's order
//   and serve as V from the registers (FP8 records in per-token teams: their
//   codes, dequantised in registers); the 64-bit path and the FP8 union team
//   read V back from the staged slice.
//
// Invalid slots (outside [0, kv_len), past topk or topk_len, or owned by
// none of the team's rows) read zeros (a row index the buffer descriptor's
// range check rejects, or a cache-resident zero row on the 64-bit path) and
// are masked to -inf before the softmax; a tile with no valid slot for the
// team is skipped whole. Workgroups are remapped so that each XCD (own L2)
// works on bands of consecutive rows, which share most of their slots.
#pragma once

#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

// kRows: per-token results (one request, or ragged requests when cu_q is
// set), rows grouped into teams by position. kRowsMember: the same for
// two-row teams (one wave, or two waves sharing the team's bitmaps), which
// match their rows' tokens by membership (LDS bitmaps of each row's set)
// instead of by slot position wherever the team qualifies (see below), and
// by position elsewhere. kUnion: prebuilt
// union lists. kDecode: one team per (request, slot range) over paged FP8
// records, each writing that range's normalised result for a later merge;
// range s of S takes the request's slot tiles s, s + S, s + 2S, ...
enum : int { kRows = 0, kUnion = 1, kDecode = 2, kRowsMember = 3 };

// Membership bitmaps: one bit per token of the team's request, one bitmap
// per row, per team; requests longer than this match by position.
constexpr int kMemberTokens = 32768;
constexpr int kMemberWords = kMemberTokens / 32;

// Headroom of the running max in log2 units: probabilities stay <= 2^kSlack.
constexpr float kSlack = 8.f;
// Queued tokens per wavefront: fewer than 16 wait between tiles and one
// slot tile adds at most 3 x 16.
constexpr int kQueueCap = 64;
// Membership teams queue their whole token list, a chunk of bitmap words at
// a time: fewer than 16 wait when a chunk is appended, and a chunk stops
// before it would overflow.
constexpr int kMemberQueueCap = 256;

template <int DQK, int DV, bool V_IN_K, int MODE, int C, int WSPLIT, bool FP8>
struct AttnTile {
  static constexpr int KSTEPS = DQK / 32 / WSPLIT;   // this wave's k-steps of S^T
  static constexpr int VCH = DV / 128 / WSPLIT;      // this wave's 16-byte V chunks per slot
  static constexpr int MTILES = DV / 16 / WSPLIT;    // this wave's 16-wide d blocks of O^T
  static_assert(DQK % (32 * WSPLIT) == 0 && DV % (128 * WSPLIT) == 0, "head dims");
  static_assert(C >= 1 && C <= 3, "column tiles per team");
  static constexpr bool UNION = MODE == kUnion;
  // V inside the latent K row: the wave's K slice is its V columns
  // [split*MAIN, +MAIN) plus its rope columns [DV + split*ROPE, +ROPE), so V
  // is part of the one gathered slice and both operands are read from LDS.
  static constexpr int MAIN = DV / WSPLIT;
  static constexpr int ROPE = (DQK - DV) / WSPLIT;
  static constexpr bool VKLDS = V_IN_K && MAIN % 32 == 0 && ROPE % 32 == 0;
  static constexpr int CPR = VKLDS ? (MAIN + ROPE) / 8 : 1;  // 16-byte chunks per slot row
  // K staged through LDS in whole 256-byte halves per slot (16 lanes x 16 B).
  static constexpr bool KLDS = !VKLDS && KSTEPS % 4 == 0;
  static_assert(KLDS || VKLDS, "K is staged through LDS");
  static_assert(!V_IN_K || VKLDS, "V inside K is read from the staged K slice");
  // FP8: K rows are 656-byte records (512 E4M3 latent values, four fp32
  // block scales, 64 bf16 rope values), dequantised into the same bf16 slice
  static_assert(!FP8 || (VKLDS && DQK == 576 && DV == 512 && WSPLIT == 2), "FP8 records");
  static_assert(MODE != kDecode || (FP8 && C == 1), "decode reads paged FP8 records, one row per team");
  static_assert(MODE != kRowsMember || C == 1, "membership: two-row, one-tile teams");
  // membership bitmaps per workgroup: one pair per team
  static constexpr int TEAMS_PER_WG = WSPLIT == 1 ? 4 : 1;
  static constexpr int KCH = KLDS ? KSTEPS / 4 : 0;   // 16-byte K chunks per slot per lane
  static constexpr int KROW = 64 * KSTEPS + 16;       // LDS row pitch (bytes): 16 (mod 32) * odd
  static constexpr int KLDS_BYTES = 16 * KROW;
  // wavefronts per workgroup: four one-wave teams, or the two halves of one
  static constexpr int WG_WAVES = WSPLIT == 1 ? 4 : WSPLIT;

  struct Data {
    u32x4_t kd[KSTEPS];    // raw K chunks (VKLDS: the K|V slice), staged through LDS
    u32x4_t vd[4 * VCH];   // vd[VCH*i + h]: slot 4g+i, d = 128h + 8m .. +7
  };
};

// Invalid slots load zeros, so the loads need no branch (a load under a
// per-lane branch cannot be counted, and waiting for any later load then
// waits for all of them) and an invalid slot's V is exactly 0. Row gathers
// through buffer descriptors (BUF) name the absent row kNoRow; 64-bit
// addressed gathers (windows past 2 GiB, strides past the descriptor's
// field, paged records) read this zero row instead. Every row offset read
// here is below 2 KB.
static __device__ __attribute__((aligned(16))) uint8_t kZeroRow[2048];

// Team `team_id`, wavefront `split` of WSPLIT. xch: partial-score exchange
// [2][WG_WAVES][C][64]; klds: per-wave K tiles; qtok/qbits: per-wave queues.
template <int DQK, int DV, bool V_IN_K, int MODE, int C, int WSPLIT, bool FP8, bool BUF>
__device__ __forceinline__ void attn_team(const AttnParams& p, int team_id, int split,
                                          f32x4_t* xch, uint8_t* klds, int32_t* qtok_all,
                                          uint32_t* qbits_all, uint32_t* bmap_all) {
  using TT = AttnTile<DQK, DV, V_IN_K, MODE, C, WSPLIT, FP8>;
  constexpr int KSTEPS = TT::KSTEPS;
  constexpr int VCH = TT::VCH;
  constexpr int MTILES = TT::MTILES;
  constexpr bool UNION = TT::UNION;
  constexpr bool DECODE = MODE == kDecode;
  constexpr bool MEMBER = MODE == kRowsMember;
  constexpr bool VKLDS = TT::VKLDS;
  // V inside K, gathered through row descriptors: lane (g, n) reads latent
  // chunks n and 16 + n of slots 4g .. 4g+3 (the V operand's order, as for a
  // separate V) plus rope chunk n % 4 of slot 4g + n / 4; the chunks are
  // staged for S^T and the latent ones kept in registers as V, so LDS
  // carries only the S^T transpose.
  constexpr bool VDIRECT = VKLDS && BUF && !FP8;
  // FP8 records, per-token teams: the codes of chunks n and 16 + n, dequantised
  // in registers, staged for S^T and kept as V (the three-wave union team
  // would spill the extra registers, so it reads V back from the slice)
  constexpr bool FP8DIRECT = FP8 && BUF && MODE != kUnion;
  static_assert(!VDIRECT || (TT::MAIN == 256 && TT::ROPE == 32 && TT::VCH == 2 && KSTEPS == 9),
                "direct V: 32 latent and 4 rope chunks per slot and wave");
  constexpr int KCH = TT::KCH;
  constexpr int KROW = TT::KROW;
  constexpr int MAIN = TT::MAIN;
  constexpr int ROPE = TT::ROPE;
  constexpr int CPR = TT::CPR;
  constexpr int TILE = 16;
  using Data = typename TT::Data;
  static_assert(!(BUF && DECODE), "paged records are gathered with 64-bit addresses");

  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int n = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int group = p.group;
  const int slot_l = 4 * g + (n >> 2);   // index lanes: slot and row read by this lane
  const int row_l = n & 3;

  // ---- which rows this team serves ------------------------------------
  int kvh, t0, rows;          // KV head, first row, rows served
  int bit0 = 0;               // ownership bit of the team's first row
  const int32_t* irow;        // per-token: this lane's row; union: the group's list
  const uint8_t* brow = nullptr;
  int jmax_l = 0;             // per-token: slots of this lane's row
  int jmax;                   // slots the team streams
  int base_l = 0;             // per-token: first KV row of this lane's request
  int len_l = 0;              // and its length
  int64_t team_kv = 0;        // union over ragged requests: the group's first KV row
  int qrow_div = 1;           // decode: a virtual row's query row is row / dec_splits
  int tile_first = 0;         // decode: the range's first slot tile and tile stride
  int tile_step = 1;
  if constexpr (UNION) {
    const int per_head = p.num_groups * p.teams_per_group;
    kvh = team_id / per_head;
    if (kvh >= p.num_kv_heads) return;
    const int r = team_id - kvh * per_head;
    const int gi = r / p.teams_per_group;
    const int ts = r - gi * p.teams_per_group;
    int first, members;
    len_l = p.kv_len;
    if (p.gstart) {
      if (!ragged_group(p.gstart, p.cu_q, p.cu_kv, p.num_reqs, p.G, gi, first, members, team_kv,
                        len_l))
        return;
    } else {
      first = gi * p.G;
      members = p.G;
    }
    if (members > p.num_rows - first) members = p.num_rows - first;   // rows that exist
    bit0 = ts * p.rows_per_team;                      // first member served
    rows = members - bit0;
    if (rows > p.rows_per_team) rows = p.rows_per_team;
    if (rows <= 0) return;
    t0 = first + bit0;
    irow = p.union_idx + (int64_t)gi * p.union_stride;
    brow = p.union_bits + (int64_t)gi * p.union_stride;
    jmax = p.union_len[gi];
  } else if constexpr (DECODE) {
    // virtual row t0 = b * dec_splits + s: slot tiles s, s + S, ... of request b
    kvh = team_id / p.num_rows;
    if (kvh >= p.num_kv_heads) return;
    t0 = team_id - kvh * p.num_rows;
    rows = 1;
    qrow_div = p.dec_splits;
    const int b = t0 / p.dec_splits;
    tile_first = t0 - b * p.dec_splits;
    tile_step = p.dec_splits;
    if (row_l == 0) {
      len_l = p.kv_len;   // tokens in the pool
      jmax_l = p.topk;
      if (p.topk_len) {
        const int tl = p.topk_len[b];
        jmax_l = tl < 0 ? 0 : (tl < jmax_l ? tl : jmax_l);
      }
    }
    irow = p.idx + (int64_t)b * p.idx_row_stride;
    int jm = jmax_l;
    jm = max(jm, __builtin_amdgcn_mov_dpp(jm, 0xb1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
    jm = max(jm, __builtin_amdgcn_mov_dpp(jm, 0x4e, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
    jmax = __builtin_amdgcn_readfirstlane(jm);
  } else {
    const int per_head = (p.num_rows + p.rows_per_team - 1) / p.rows_per_team;
    kvh = team_id / per_head;
    if (kvh >= p.num_kv_heads) return;
    t0 = (team_id - kvh * per_head) * p.rows_per_team;
    rows = p.num_rows - t0;
    if (rows > p.rows_per_team) rows = p.rows_per_team;
    // this lane's row: its request, its slot count
    const int t = t0 + row_l;
    if (row_l < rows) {
      len_l = p.kv_len;
      if (p.cu_q) {
        int lo = 0, hi = p.num_reqs - 1;   // last request whose first row is <= t
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (p.cu_q[mid] <= t) lo = mid; else hi = mid - 1;
        }
        base_l = (int)p.cu_kv[lo];   // KV rows are below 2^31 (host contract)
        len_l = (int)(p.cu_kv[lo + 1] - p.cu_kv[lo]);
      }
      jmax_l = p.topk;
      if (p.topk_len) {
        const int tl = p.topk_len[t];
        jmax_l = tl < 0 ? 0 : (tl < jmax_l ? tl : jmax_l);
      }
      if (len_l <= 0) jmax_l = 0;
    }
    irow = p.idx + (int64_t)(row_l < rows ? t : t0) * p.idx_row_stride;
    // the team streams as many tiles as its longest row needs
    int jm = jmax_l;
    jm = max(jm, __builtin_amdgcn_mov_dpp(jm, 0xb1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
    jm = max(jm, __builtin_amdgcn_mov_dpp(jm, 0x4e, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
    jmax = __builtin_amdgcn_readfirstlane(jm);
  }

  // ---- membership (two-row teams): each row's token set as an LDS bitmap --
  // A team qualifies when both rows exist, share one request of at most
  // kMemberTokens tokens and hold no token twice. It then streams the union
  // of its rows' sets in ascending token order, read off the two bitmaps,
  // each token with the bits of the rows that hold it: each row sees each of
  // its tokens once whatever its slot order, and neighbouring teams sweep the
  // KV rows in the same order (their gathers meet in the caches). Otherwise
  // the team matches its rows by slot position.
  bool member = false;
  uint32_t* bmp = nullptr;
  int member_words = 0, member_base = 0;
  if constexpr (MEMBER) {
    // one wave marks both rows; a two-wave team marks one row per wave into
    // the team's shared pair and meets at a barrier before either reads it
    bmp = bmap_all + (WSPLIT == 1 ? wv : 0) * 2 * kMemberWords;
    const int b0 = __builtin_amdgcn_readlane(base_l, 0), b1 = __builtin_amdgcn_readlane(base_l, 1);
    const int n0 = __builtin_amdgcn_readlane(len_l, 0), n1 = __builtin_amdgcn_readlane(len_l, 1);
    if (rows == 2 && b0 == b1 && n0 == n1 && n0 <= kMemberTokens) {   // team-uniform
      member_words = (n0 + 31) >> 5;
      member_base = b0;
      constexpr int kRowsPerWave = WSPLIT == 1 ? 2 : 1;
      const int r0 = WSPLIT == 1 ? 0 : split;
      for (int w = lane; w < kRowsPerWave * kMemberWords; w += 64) {
        const int r = w >= kMemberWords;
        if (w - r * kMemberWords < member_words) bmp[r0 * kMemberWords + w] = 0u;
      }
      uint32_t dup = 0;
#pragma unroll
      for (int r = r0; r < r0 + kRowsPerWave; ++r) {
        const int jr = __builtin_amdgcn_readlane(jmax_l, r);
        const int32_t* ir = p.idx + (int64_t)(t0 + r) * p.idx_row_stride;
        uint32_t* br = bmp + r * kMemberWords;
        // all of a row's index loads are issued before its marks
        constexpr int kBatch = 36;
        for (int j0 = 0; j0 < jr; j0 += kBatch * 64) {
          int x[kBatch];
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            const int j = j0 + 64 * u + lane;
            x[u] = j < jr ? ir[j] : -1;
          }
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            if ((unsigned)x[u] < (unsigned)n0) {
              const uint32_t bit = 1u << (x[u] & 31);
              dup |= atomicOr(br + (x[u] >> 5), bit) & bit;
            }
          }
        }
      }
      member = __ballot(dup != 0u) == 0;
      if constexpr (WSPLIT > 1) {
        // both rows marked, and both waves take the same decision
        if (lane == 0) bmp[2 * kMemberWords + split] = member ? 0u : 1u;
        __syncthreads();
        member = (bmp[2 * kMemberWords] | bmp[2 * kMemberWords + 1]) == 0u;
      }
    }
  }

  const uint32_t team_bits = ((1u << rows) - 1u) << bit0;
  const int tiles_all = (jmax + TILE - 1) / TILE;
  const int ntiles = tiles_all > tile_first ? (tiles_all - tile_first + tile_step - 1) / tile_step : 0;

  // ---- columns: tile c, lane n -> row j, head ----------------------------
  // (recomputed in the epilogue so that only the ownership bits stay live)
  auto column = [&](int c, bool& live, int& t, int& head) {
    const int col = 16 * c + n;
    const int j = col / group;
    live = j < rows;
    head = kvh * group + (col - j * group);
    t = t0 + (live ? j : 0);
    return live ? (1u << (bit0 + j)) : 0u;
  };
  int col_sh[C];   // the column's ownership bit (31 for a dead column: no bit is that high)
  // Wave-uniform K/V bases; lane offsets are added per load.
  const uint16_t* kw = p.k + team_kv * p.k_row_stride + kvh * DQK + (VKLDS ? 0 : 32 * KSTEPS * split);
  const uint16_t* vw = p.v + team_kv * p.v_row_stride + kvh * (V_IN_K ? DQK : DV) + 128 * VCH * split;

  // ---- Q^T operands: lane (g, n) of tile c holds column n, d = 32s + 8g ----
  u32x4_t qop[C][KSTEPS];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    bool live;
    int t, head;
    const uint32_t cb = column(c, live, t, head);
    col_sh[c] = live ? __builtin_ctz(cb) : 31;
    const uint16_t* qp = p.q + (int64_t)(t / qrow_div) * p.q_row_stride + (int64_t)head * DQK + 8 * g;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      // d of k-step s: the wave's slice in k-step order
      const int d = VKLDS ? (s < MAIN / 32 ? split * MAIN + 32 * s : DV + split * ROPE + 32 * (s - MAIN / 32))
                          : 32 * KSTEPS * split + 32 * s;
      qop[c][s] = live ? ld16(qp + d) : (u32x4_t){0, 0, 0, 0};
    }
  }

  // One index load per lane per tile (plus the ownership byte in union mode).
  // Lanes past their row's end read entry 0 (every row that has a tile has
  // one) and the entry is discarded where it is used: the load carries no
  // branch and nothing reads it early, so waiting for this tile's indices
  // does not wait for the next tile's, issued after them.
  const int jlim = UNION ? jmax : jmax_l;   // this lane's entries
  struct Idx {
    int x;        // per-token: index of (row_l, slot_l); union: list entry slot_l
    int j;        // its position (the entry exists iff j < jlim)
    uint32_t b;   // union: its ownership bits
  };
  auto load_idx = [&](Idx& ti, int j0) {
    const int jk = j0 + slot_l;
    const int jr = jk < jlim ? jk : 0;
    ti.x = irow[jr];
    ti.j = jk;
    if (UNION) ti.b = brow[jr];
  };

  // The queue of tokens still to gather (per wave, in LDS).
  constexpr int QCAP = MEMBER ? kMemberQueueCap : kQueueCap;
  int32_t* qtok = qtok_all + wv * QCAP;
  uint32_t* qbits = qbits_all + wv * QCAP;
  int qcount = 0;

  // A tile to gather, as seen by an index lane: the token of slot slot_l
  // (global KV row, -1 for none) and the team rows it serves.
  struct Tile {
    int tok;
    uint32_t bits;
  };
  // Per-token modes: slot slot_l serves every row whose token there equals
  // row 0's; every other token is queued once per run of consecutive rows
  // that hold it.
  auto resolve = [&](const Idx& ti) -> Tile {
    const int gt = ti.j < jlim && (unsigned)ti.x < (unsigned)len_l ? base_l + ti.x : -1;
    const int m0 = quad_bcast<0>(gt);                                            // row 0
    const int pv = __builtin_amdgcn_mov_dpp(gt, 0x90, 0xf, 0xf, false);          // row r-1: [0,0,1,2]
    const bool eqm = gt >= 0 && gt == m0;
    const bool eqp = gt >= 0 && row_l >= 1 && gt == pv;
    const bool start = gt >= 0 && !eqm && !(row_l >= 2 && eqp);
    const uint64_t bm = (uint64_t)__ballot(eqm);
    const uint64_t bp = (uint64_t)__ballot(eqp);
    const uint64_t bs = (uint64_t)__ballot(start);
    if (start) {
      // the run: row_l and the following rows that repeat its token
      const uint32_t np = (uint32_t)(bp >> (4 * slot_l)) & 0xfu;
      const int run = __builtin_ctz(~(np >> (row_l + 1)));
      const uint32_t bits = ((1u << (row_l + 1 + run)) - 1u) & ~((1u << row_l) - 1u);
      const int at = qcount + __popcll(bs & ((1ull << lane) - 1ull));
      qtok[at] = gt;
      qbits[at] = bits;
    }
    qcount += __popcll(bs);
    return Tile{m0, (uint32_t)(bm >> (4 * slot_l)) & 0xfu};
  };

  // Invalid slots load zeros (their scores are forced to -inf, and their V
  // is 0, multiplied by p = 0).
  const uint32_t k_row_bytes = (uint32_t)(2 * p.k_row_stride);   // < 2^32 (host check)
  const uint32_t v_row_bytes = (uint32_t)(2 * p.v_row_stride);
  const bool v_like_k = v_row_bytes == k_row_bytes;
  // FP8 records: kvh's record of row 0 (k_row_stride counts 2-byte units)
  const uint8_t* kwb = FP8 ? reinterpret_cast<const uint8_t*>(p.k) + team_kv * k_row_bytes + kvh * 656
                           : reinterpret_cast<const uint8_t*>(kw);
  const uint8_t* kbn = kwb + 16 * n;   // this lane's 16 bytes of a 256-byte half row
  const uint8_t* vbn = reinterpret_cast<const uint8_t*>(vw) + 16 * n;
  // BUF: K and V rows as windows of row-strided records from the same bases
  // (the launcher checks that strides and windows fit the descriptors).
  const rows_rsrc_t rk = rows_rsrc(kwb, k_row_bytes);
  const rows_rsrc_t rv = rows_rsrc(vw, v_row_bytes);
  // Issues a tile's loads; returns the ownership bits of slots 4g..4g+3
  // (0 for an invalid slot): slot 4g+i contributes to column n of tile c iff
  // bit col_sh[c] of own[i] is set.
  auto load_data = [&](Data& td, const Tile& tl, int own[4]) {
    const bool ok = tl.tok >= 0 && (tl.bits & team_bits);
    if constexpr (BUF) {
      // The index lane's row (kNoRow when invalid) and bits reach the
      // sixteen lanes of group g by row broadcast; an invalid slot owns no
      // column.
      int rw[4];
      row_bcast4(ok ? tl.tok : kNoRow, rw);
      row_bcast4(ok ? (int)tl.bits : 0, own);
      if constexpr (FP8) {
        // as below: latent half rows, one rope chunk, the slot's scales
        const int ir = n >> 2, is = n & 3;
        auto pick = [](const int a[4], int i) { return i == 0 ? a[0] : i == 1 ? a[1] : i == 2 ? a[2] : a[3]; };
        if constexpr (FP8DIRECT) {   // codes of chunks n and 16 + n, 8 bytes each
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const u32x2_t a = ld_row8(rk, rw[i], 256 * split + 8 * n);
            const u32x2_t b = ld_row8(rk, rw[i], 256 * split + 128 + 8 * n);
            td.kd[i] = (u32x4_t){a[0], a[1], b[0], b[1]};
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) td.kd[i] = ld_row16(rk, rw[i], 256 * split + 16 * n);
        }
        td.kd[4] = ld_row16(rk, pick(rw, ir), 528 + 64 * split + 16 * is);
        td.kd[5] = ld_row16(rk, pick(rw, is), 512);
      } else if constexpr (VDIRECT) {
        auto pick = [](const int a[4], int i) { return i == 0 ? a[0] : i == 1 ? a[1] : i == 2 ? a[2] : a[3]; };
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int h = 0; h < VCH; ++h)
            td.kd[VCH * i + h] = ld_row16(rk, rw[i], 2 * split * MAIN + 256 * h + 16 * n);
        td.kd[4 * VCH] = ld_row16(rk, pick(rw, n >> 2), 2 * (DV + split * ROPE) + 16 * (n & 3));
      } else if constexpr (VKLDS) {
#pragma unroll
        for (int q = 0; q < KSTEPS; ++q) {
          const int i0 = (16 * q) / CPR;
          const int c = 16 * q + n;
          const bool nx = i0 < 3 && c >= CPR * (i0 + 1);
          const int ch = c - CPR * (nx ? i0 + 1 : i0);
          const int d = ch < MAIN / 8 ? split * MAIN + 8 * ch : DV + split * ROPE + 8 * (ch - MAIN / 8);
          td.kd[q] = ld_row16(rk, nx ? rw[i0 < 3 ? i0 + 1 : 3] : rw[i0], 2 * d);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int h = 0; h < KCH; ++h) td.kd[KCH * i + h] = ld_row16(rk, rw[i], 16 * n + 256 * h);
#pragma unroll
          for (int h = 0; h < VCH; ++h) td.vd[VCH * i + h] = ld_row16(rv, rw[i], 16 * n + 256 * h);
        }
      }
      return;
    }
    int64_t koff;
    if constexpr (DECODE)   // record (t & mask) of page t >> shift (page stride < 2^32)
      koff = ok ? (int64_t)((uint64_t)((uint32_t)tl.tok >> p.page_shift) * (uint32_t)p.page_stride +
                            ((uint32_t)tl.tok & ((1u << p.page_shift) - 1u)) * 656u)
                : -1;
    else
      koff = ok ? (int64_t)((uint64_t)(uint32_t)tl.tok * k_row_bytes) : -1;
    int khi[4];
    row_bcast4((int)(koff >> 32), khi);
    row_bcast4(ok ? (int)tl.bits : 0, own);
    if constexpr (FP8) {
      // Per slot 4g+i: the wave's 256 latent bytes, sixteen lanes per row.
      // Per lane: one rope chunk (slot 4g + n/4, chunk n%4 of the wave's 64
      // rope bytes) and the 16 scale bytes of slot 4g + n%4.
      int klo[4];
      row_bcast4((int)koff, klo);
      const int ir = n >> 2, is = n & 3;
      auto pick = [](const int a[4], int i) { return i == 0 ? a[0] : i == 1 ? a[1] : i == 2 ? a[2] : a[3]; };
      auto rec = [&](int lo, int hi) { return hi >= 0 ? kwb + join64(lo, hi) : kZeroRow; };
#pragma unroll
      for (int i = 0; i < 4; ++i) td.kd[i] = ld16(rec(klo[i], khi[i]) + 256 * split + 16 * n);
      td.kd[4] = ld16(rec(pick(klo, ir), pick(khi, ir)) + 528 + 64 * split + 16 * is);
      td.kd[5] = ld16(rec(pick(klo, is), pick(khi, is)) + 512);
      return;
    }
    if constexpr (VKLDS) {
      // Lane group g gathers its own slots 4g..4g+3 (their offsets arrive by
      // row broadcast): load q of lane n takes chunk c = 16q + n of the
      // group's 4 * CPR chunks, i.e. chunk c % CPR of slot 4g + c / CPR, so
      // sixteen lanes read 256 consecutive bytes of a row, and the sixteen
      // chunks of one load span at most two slots (CPR > 16).
      static_assert(CPR > 16 && 4 * CPR == 16 * KSTEPS, "MLA slice chunks");
      int klo[4];
      row_bcast4((int)koff, klo);
#pragma unroll
      for (int q = 0; q < KSTEPS; ++q) {
        const int i0 = (16 * q) / CPR;              // the load's first slot
        const int c = 16 * q + n;
        const bool nx = i0 < 3 && c >= CPR * (i0 + 1);   // this lane is in the next slot
        const int lo = nx ? klo[i0 < 3 ? i0 + 1 : 3] : klo[i0];
        const int hi = nx ? khi[i0 < 3 ? i0 + 1 : 3] : khi[i0];
        const int ch = c - CPR * (nx ? i0 + 1 : i0);
        const int d = ch < MAIN / 8 ? split * MAIN + 8 * ch : DV + split * ROPE + 8 * (ch - MAIN / 8);
        td.kd[q] = ld16((hi >= 0 ? kwb + join64(lo, hi) : kZeroRow) + 2 * d);
      }
      return;
    }
    int klo[4], vlo[4], vhi[4];
    row_bcast4((int)koff, klo);
    if (v_like_k) {   // V rows at K's byte offsets (from their own base)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vlo[i] = klo[i];
        vhi[i] = khi[i];
      }
    } else {
      const int64_t voff = ok ? (int64_t)((uint64_t)(uint32_t)tl.tok * v_row_bytes) : -1;
      row_bcast4((int)voff, vlo);
      row_bcast4((int)(voff >> 32), vhi);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // K and V rows of slot 4g+i, bytes 256h + 16m: sixteen lanes per row
      const bool ok = khi[i] >= 0;
      const uint8_t* kp = ok ? kbn + join64(klo[i], khi[i]) : kZeroRow + 16 * n;
      const uint8_t* vp = ok ? vbn + join64(vlo[i], vhi[i]) : kZeroRow + 16 * n;
#pragma unroll
      for (int h = 0; h < KCH; ++h) td.kd[KCH * i + h] = ld16(kp + 256 * h);
#pragma unroll
      for (int h = 0; h < VCH; ++h) td.vd[VCH * i + h] = ld16(vp + 256 * h);
    }
  };

  // Reference max (log2 domain) and this lane's share of the sum. The max
  // starts at -FLT_MAX, not -inf: it stays finite, so a column that has seen
  // no valid score yet needs no special case (its masked scores give
  // exp2(-inf) = 0, and the first valid score moves the max and scales the
  // empty state by exp2(-FLT_MAX - m) = 0).
  float m_run[C], l_run[C];
  f32x4_t acc[C][MTILES];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    m_run[c] = -__FLT_MAX__;
    l_run[c] = 0.f;
#pragma unroll
    for (int mt = 0; mt < MTILES; ++mt) acc[c][mt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  }
  const float sc = p.scale_log2e;

  int par = 0;
  uint8_t* lk = klds + wv * TT::KLDS_BYTES;   // this wave's K tile in LDS
  // Byte position of 16-byte chunk c in a staged row. FP8 rows are written
  // as dequantised pairs (lane n writes chunks 2n and 2n + 1), so their 32
  // latent chunks are rotated within blocks of 8 (chunk c of block b sits at
  // (c + b) mod 8): the pair writes, the V reads (chunk 16h + n of lane n)
  // and the A-operand reads all stay free of bank conflicts.
  auto cpos = [](int c) {
    return 16 * (FP8 && !FP8DIRECT && c < 32 ? (c & ~7) | ((c + (c >> 3)) & 7) : c);
  };
  auto compute = [&](const Data& td, const int own[4]) {
    u32x4_t vdq[FP8DIRECT ? 8 : 1];   // FP8DIRECT: the dequantised latent chunks n, 16 + n (V)
    // Stage the gathered rows in LDS, in the A-operand order.
    if constexpr (FP8) {
      // Dequantise: latent chunk n of slot 4g+i (values 16n .. 16n+15 of the
      // wave's slice, block 2 split + n/8) times its block scale, rounded to
      // bf16, becomes slice chunks 2n and 2n+1; the rope chunk is bf16
      // already. The scales of slot 4g+i sit in quad lane i.
      int s0[4], s1[4];
      quad_bcast4((int)td.kd[5][2 * split], s0);
      quad_bcast4((int)td.kd[5][2 * split + 1], s1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (FP8DIRECT) {
          // words 0-1: codes of chunk n (block 2 split), words 2-3: chunk 16 + n
          const float sa = __builtin_bit_cast(float, s0[i]), sb = __builtin_bit_cast(float, s1[i]);
          uint32_t b[8];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float sc = w < 2 ? sa : sb;
            const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)td.kd[i][w], false);
            const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)td.kd[i][w], true);
            b[2 * w] = pack_bf16x2(lo[0] * sc, lo[1] * sc);
            b[2 * w + 1] = pack_bf16x2(hi[0] * sc, hi[1] * sc);
          }
          vdq[2 * i] = (u32x4_t){b[0], b[1], b[2], b[3]};
          vdq[2 * i + 1] = (u32x4_t){b[4], b[5], b[6], b[7]};
          uint8_t* row = lk + (4 * g + i) * KROW;
          *reinterpret_cast<u32x4_t*>(row + 16 * n) = vdq[2 * i];
          *reinterpret_cast<u32x4_t*>(row + 16 * (16 + n)) = vdq[2 * i + 1];
          continue;
        }
        const float sc = __builtin_bit_cast(float, (n >> 3) ? s1[i] : s0[i]);
        uint32_t b[8];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)td.kd[i][w], false);
          const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)td.kd[i][w], true);
          b[2 * w] = pack_bf16x2(lo[0] * sc, lo[1] * sc);
          b[2 * w + 1] = pack_bf16x2(hi[0] * sc, hi[1] * sc);
        }
        uint8_t* row = lk + (4 * g + i) * KROW;
        *reinterpret_cast<u32x4_t*>(row + cpos(2 * n)) = (u32x4_t){b[0], b[1], b[2], b[3]};
        *reinterpret_cast<u32x4_t*>(row + cpos(2 * n + 1)) = (u32x4_t){b[4], b[5], b[6], b[7]};
      }
      *reinterpret_cast<u32x4_t*>(lk + (4 * g + (n >> 2)) * KROW + 16 * (MAIN / 8 + (n & 3))) = td.kd[4];
    } else if constexpr (VDIRECT) {
      // latent chunk 16h + n of slot 4g+i, rope chunk n % 4 of slot 4g + n/4
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < VCH; ++h)
          *reinterpret_cast<u32x4_t*>(lk + (4 * g + i) * KROW + 16 * (16 * h + n)) = td.kd[VCH * i + h];
      *reinterpret_cast<u32x4_t*>(lk + (4 * g + (n >> 2)) * KROW + 16 * (MAIN / 8 + (n & 3))) =
          td.kd[4 * VCH];
    } else if constexpr (VKLDS) {
      // chunk c = 16q + n of group g's slots (the gather's order)
#pragma unroll
      for (int q = 0; q < KSTEPS; ++q) {
        const int i0 = (16 * q) / CPR;
        const int c = 16 * q + n;
        const int i = i0 < 3 && c >= CPR * (i0 + 1) ? i0 + 1 : i0;
        *reinterpret_cast<u32x4_t*>(lk + (4 * g + i) * KROW + 16 * (c - CPR * i)) = td.kd[q];
      }
    } else {
      // write slot 4g+i, bytes 256h + 16m; read slot m, bytes 64s + 16g. The
      // pitch KROW = 16 (mod 256) keeps both sides bank-conflict free.
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < KCH; ++h)
          *reinterpret_cast<u32x4_t*>(lk + (4 * g + i) * KROW + 256 * h + 16 * n) = td.kd[KCH * i + h];
    }
    f32x4_t st[C];
#pragma unroll
    for (int c = 0; c < C; ++c) st[c] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const u32x4_t a = *reinterpret_cast<const u32x4_t*>(lk + n * KROW + cpos(4 * s + g));
#pragma unroll
      for (int c = 0; c < C; ++c) st[c] = mfma_16x16x32(a, qop[c][s], st[c]);
    }
    if (WSPLIT > 1) {
      // partial S^T of the other half of d; both waves form half0 + half1
      constexpr int WGW = TT::WG_WAVES;
#pragma unroll
      for (int c = 0; c < C; ++c) xch[((par * WGW + wv) * C + c) * 64 + lane] = st[c];
      __syncthreads();
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const f32x4_t o = xch[((par * WGW + (wv ^ 1)) * C + c) * 64 + lane];
        st[c] = split == 0 ? st[c] + o : o + st[c];
      }
      par ^= 1;
    }
    i16x4_t pop[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      // Masked raw scores; scaling commutes with the max (sc > 0 and
      // rounding is monotonic), and each probability takes one fma.
      float s2[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) s2[i] = keep_if_bit(st[c][i], own[i], col_sh[c]);
      // The reference max moves only when some score of the column passes
      // it by more than kSlack. Each lane tests its own four scores first
      // (rounding is monotonic, so some lane passes iff the column's max
      // does); the cross-lane max runs only when some lane of the wave
      // passes, which after a column's first tiles is rare.
      const float mx = max4(s2[0], s2[1], s2[2], s2[3]);
      const float m_lim = m_run[c] + kSlack;
      if (__builtin_amdgcn_ballot_w64(mx * sc > m_lim)) {
        const float cm = rows_max4(mx) * sc;
        const float m_new = cm > m_lim ? cm : m_run[c];
        // rescale where the column's reference max moved (alpha == 1
        // elsewhere)
        const float alpha = fast_exp2(m_run[c] - m_new);
        l_run[c] *= alpha;
#pragma unroll
        for (int mt = 0; mt < MTILES; ++mt) acc[c][mt] *= alpha;
        m_run[c] = m_new;
      }
      float pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(fmaf(s2[i], sc, -m_run[c]));
      l_run[c] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
      pop[c] = __builtin_bit_cast(i16x4_t,
                                  (u32x2_t){pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])});
    }
    u32x4_t vv[4 * VCH];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < VCH; ++h)
        vv[VCH * i + h] = FP8DIRECT ? vdq[FP8DIRECT ? VCH * i + h : 0]
                          : VDIRECT ? td.kd[VCH * i + h]
                          : VKLDS ? *reinterpret_cast<const u32x4_t*>(lk + (4 * g + i) * KROW + cpos(16 * h + n))
                                  : td.vd[VCH * i + h];
#pragma unroll
    for (int mt = 0; mt < MTILES; ++mt) {
      const int h = mt >> 3, e = mt & 7;
      const i16x4_t a = gather_col4(vv[h], vv[VCH + h], vv[2 * VCH + h], vv[3 * VCH + h], e);
#pragma unroll
      for (int c = 0; c < C; ++c) acc[c][mt] = mfma_16x16x16(a, pop[c], acc[c][mt]);
    }
  };

  Data db;   // every load_data call writes all of it

  // Gathers and consumes queued tokens, 16 at a time (all when flushing).
  auto run_queue = [&](bool flush) {
    while (qcount >= 16 || (flush && qcount > 0)) {
      const bool have = slot_l < qcount;
      const Tile tl{have ? qtok[slot_l] : -1, have ? qbits[slot_l] : 0u};
      int own[4];
      load_data(db, tl, own);
      compute(db, own);
      // move the remaining entries down (in-order LDS: reads first)
      const int rem = qcount > 16 ? qcount - 16 : 0;
      const bool mv = lane < rem;
      const int vt = mv ? qtok[16 + lane] : 0;
      const uint32_t vb = mv ? qbits[16 + lane] : 0u;
      if (mv) {
        qtok[lane] = vt;
        qbits[lane] = vb;
      }
      qcount = rem;
    }
  };

  if (MEMBER && member) {
    // The union of the two rows' sets, ascending: lane l takes bitmap word
    // cw + l of a chunk and appends its tokens (with their rows' bits) at
    // its prefix-sum offset; lanes past the queue's room wait for the next
    // chunk. Whole tiles of 16 are consumed from the queue head; the rest
    // (fewer than 16) move to the front before the next chunk.
    int cw = 0;
    while (cw < member_words || qcount > 0) {
      if (cw < member_words) {
        const int w = cw + lane;
        const uint32_t m0 = w < member_words ? bmp[w] : 0u;
        const uint32_t m1 = w < member_words ? bmp[kMemberWords + w] : 0u;
        const uint32_t u = m0 | m1;
        const uint32_t cnt = __popc(u);
        const uint32_t incl = wave_scan64(cnt);
        const bool fits = (int)incl <= QCAP - qcount && w < member_words;
        const uint64_t fb = (uint64_t)__ballot(fits);
        const int taken = fb == ~0ull ? 64 : __builtin_ctzll(~fb);   // a prefix of the lanes
        if (lane < taken) {
          int at = qcount + (int)(incl - cnt);
          uint32_t v = u;
          const int tok0 = member_base + 32 * w;
          while (v) {
            const int b = __builtin_ctz(v);
            qtok[at] = tok0 + b;
            qbits[at] = ((m0 >> b) & 1u) | (((m1 >> b) & 1u) << 1);
            ++at;
            v &= v - 1u;
          }
        }
        qcount += __builtin_amdgcn_readlane((int)incl, taken - 1);
        cw += taken;
      }
      const bool last = cw >= member_words;
      int head = 0;
      while (qcount - head >= 16 || (last && qcount - head > 0)) {
        const bool have = slot_l < qcount - head;
        const Tile tl{have ? qtok[head + slot_l] : -1, have ? qbits[head + slot_l] : 0u};
        int own[4];
        load_data(db, tl, own);
        compute(db, own);
        head += 16;
      }
      const int rem = qcount > head ? qcount - head : 0;
      if (head > 0 && rem > 0) {
        const int vt = lane < rem ? qtok[head + lane] : 0;
        const uint32_t vb = lane < rem ? qbits[head + lane] : 0u;
        if (lane < rem) {
          qtok[lane] = vt;
          qbits[lane] = vb;
        }
      }
      qcount = rem;
    }
  }
  // Main tiles: the next tile's indices load while this one is gathered and
  // consumed (loads retire in issue order, so they are issued first).
  Idx ib[2];
  if (!(MEMBER && member) && ntiles > 0) load_idx(ib[0], tile_first * TILE);
  for (int tile = 0; tile < (MEMBER && member ? 0 : ntiles); tile += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int cur = tile + u;
      if (cur >= ntiles) break;
      // (after the last tile this reads entry 0 and is never used)
      load_idx(ib[u ^ 1], (tile_first + (cur + 1) * tile_step) * TILE);
      __builtin_amdgcn_sched_barrier(0);
      Tile tl;
      if constexpr (UNION) {
        const bool in = ib[u].j < jlim;
        tl.tok = in && (unsigned)ib[u].x < (unsigned)len_l ? ib[u].x : -1;
        tl.bits = in ? ib[u].b : 0u;
      } else {
        tl = resolve(ib[u]);
      }
      // A tile with nothing to gather for this team is skipped: its scores
      // would all be -inf, which leaves the softmax state and O unchanged.
      // Every wave of the team sees the same tile, so all take the branch.
      // (The three-tile shape keeps the straight path: the branch costs it
      // more register spills than the tiles it could skip.)
      if (C == 3 || __ballot(tl.tok >= 0 && (tl.bits & team_bits)) != 0) {
        int own[4];
        load_data(db, tl, own);
        __builtin_amdgcn_sched_barrier(0);
        compute(db, own);
      }
      // per-token modes: queue tiles whenever 16 queued tokens wait (so the
      // queue never holds more than 63), and a last one for the rest
      if constexpr (!UNION) run_queue(false);
    }
  }
  if constexpr (!UNION) run_queue(true);

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ---------------------
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const float l = rows_sum4(l_run[c]);
    bool live;
    int t, head;
    column(c, live, t, head);
    if (live) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      float* orow = p.out + (int64_t)t * p.out_row_stride + (int64_t)head * DV;
      // decode: a range with no valid slot leaves its O unwritten (the merge
      // gives it weight 0 from its LSE)
      if (!DECODE || l > 0.f) {
#pragma unroll
        for (int h = 0; h < VCH; ++h) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int d0 = 128 * (VCH * split + h) + 32 * g + 8 * i;
            const f32x4_t lo = {acc[c][8 * h + 0][i], acc[c][8 * h + 1][i], acc[c][8 * h + 2][i],
                                acc[c][8 * h + 3][i]};
            const f32x4_t hi = {acc[c][8 * h + 4][i], acc[c][8 * h + 5][i], acc[c][8 * h + 6][i],
                                acc[c][8 * h + 7][i]};
            st16(orow + d0, lo * inv);
            st16(orow + d0 + 4, hi * inv);
          }
        }
      }
      if (g == 0 && split == 0)
        p.lse[(int64_t)t * p.lse_row_stride + head] =
            l > 0.f ? (m_run[c] + fast_log2(l)) * kLn2 : -INFINITY;
    }
  }
}

// Whether every K and V row a launch can name is reachable through a row
// buffer descriptor from the teams' bases: both strides fit the descriptor's
// field and the launch's KV rows span at most 2 GiB at the larger stride.
__device__ __forceinline__ bool rows_fit_rsrc(const AttnParams& p) {
  const uint64_t kb = 2 * (uint64_t)p.k_row_stride, vb = 2 * (uint64_t)p.v_row_stride;
  const int64_t rows = p.cu_kv ? p.cu_kv[p.num_reqs] : (int64_t)p.kv_len;
  const uint64_t stride = kb > vb ? kb : vb;
  return kb <= kMaxRowStride && vb <= kMaxRowStride && rows >= 0 &&
         (uint64_t)rows * stride <= (1ull << 31);
}

// WSPLIT = 1: four independent one-wave teams per workgroup. WSPLIT = 2:
// one team per workgroup, its two halves exchanging partial scores.
template <int DQK, int DV, bool V_IN_K, int MODE, int C, int WSPLIT, bool FP8, int WAVES>
__global__ void __attribute__((amdgpu_flat_work_group_size(64, 256),
                               amdgpu_waves_per_eu(WAVES, WAVES)))
attn_kernel(AttnParams p) {
  using TT = AttnTile<DQK, DV, V_IN_K, MODE, C, WSPLIT, FP8>;
  __shared__ f32x4_t xch[WSPLIT > 1 ? 2 * TT::WG_WAVES * C * 64 : 1];
  __shared__ __attribute__((aligned(16))) uint8_t klds[TT::WG_WAVES * TT::KLDS_BYTES];
  constexpr int QCAP = MODE == kRowsMember ? kMemberQueueCap : kQueueCap;
  __shared__ int32_t qtok[MODE == kUnion ? 1 : TT::WG_WAVES * QCAP];
  __shared__ uint32_t qbits[MODE == kUnion ? 1 : TT::WG_WAVES * QCAP];
  __shared__ uint32_t bmap[MODE == kRowsMember ? TT::TEAMS_PER_WG * (2 * kMemberWords + 2) : 1];
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int team = WSPLIT == 1 ? bid * 4 + w : bid;
  const int split = WSPLIT == 1 ? 0 : w;
  if constexpr (MODE == kDecode)
    attn_team<DQK, DV, V_IN_K, MODE, C, WSPLIT, FP8, false>(p, team, split, xch, klds, qtok, qbits, bmap);
  else if (rows_fit_rsrc(p))
    attn_team<DQK, DV, V_IN_K, MODE, C, WSPLIT, FP8, true>(p, team, split, xch, klds, qtok, qbits, bmap);
  else
    attn_team<DQK, DV, V_IN_K, MODE, C, WSPLIT, FP8, false>(p, team, split, xch, klds, qtok, qbits, bmap);
}

// Workgroups and threads per workgroup for a launch; false when one launch
// cannot hold them (at most 2^32 - 1 threads along x).
template <int WSPLIT>
inline bool attn_grid(const AttnParams& p, int mode, dim3* grid, dim3* block) {
  const int64_t teams =
      mode == kUnion ? (int64_t)p.num_groups * p.teams_per_group * p.num_kv_heads
                     : ((int64_t)p.num_rows + p.rows_per_team - 1) / p.rows_per_team * p.num_kv_heads;
  const int64_t blocks = WSPLIT == 1 ? (teams + 3) / 4 : teams;
  const int64_t threads = WSPLIT == 1 ? 256 : 64 * WSPLIT;
  if (blocks * threads > (int64_t)UINT32_MAX) return false;
  *grid = dim3((unsigned)blocks);
  *block = dim3((unsigned)threads);
  return true;
}

}  // namespace sa
