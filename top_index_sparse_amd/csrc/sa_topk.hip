// Indexer top-k selection (sglang PR 37275, "Motivation": the indexer
// selects 2051 token slots per query row; rows whose visible context is
// shorter select fewer). Row t keeps the k largest of its first n_t scores,
// equal scores going to the lower position, and writes the kept positions in
// ascending order; a row with n_t <= k writes 0 .. n_t - 1 and pads with -1.
//
// gfx950 design: one 1024-thread workgroup per row, two resident per CU.
//   Keys. A score's bits map to a uint32 key whose unsigned order is the
//   float order (-0 is folded onto +0 first, so the two tie).
//   Sampled selection (rows of 4097 .. 32768 positions, k <= 4096, the
//   row's raw bits held in registers). A 1024-element strided sample of
//   the row gives a lower bound on its k-th largest key: the 11-bit bin
//   holding the sample's r-th largest, r the expected rank plus four
//   standard deviations. One compare per element (the raw bits compared as
//   signed integers when the bound is above +0) sends every element at or
//   above the bound to an LDS list, compacted by wave ballots; the exact
//   selection then runs on that list alone: levels of 11 bits over the
//   keys relative to the bound, until the threshold bin is either needed
//   whole or small enough (at most 64) for one wave to rank its members by
//   key and position. A list that misses the k-th largest or overflows
//   sends the row to the full path below, so the result never depends on
//   the sample. Against the full path it takes no histogram atomics for
//   the row's elements, and about a third of their instructions.
//   Full path. Level 0: an LDS histogram of the keys' top 13 bits (8192
//   bins, wide enough that scores crowding a few exponents still spread
//   their atomics) and a block-wide scan from the top bin down find the bin
//   b0 that holds the k-th largest key.
//   Classes. Every element is then above b0 (kept, into an LDS bitmap by
//   position), in b0 (a candidate) or below (dropped). Candidates, usually a
//   few hundred, are appended to an LDS list straight from the registers;
//   levels 1 and 2 (11 and 8 more bits) run on that list alone and mark each
//   candidate kept or tied in two more bitmaps.
//   Output. Thread j owns bitmap words (positions 32 words at a time, in
//   order): one block-wide scan of the owners' (kept, tied) counts gives
//   every owner its first output slot, and it writes its positions in
//   order, so neighbouring threads write neighbouring slots. An element goes
//   to (kept before it) + min(tied before it, still needed), and a tie is
//   kept while fewer than that many ties precede it.
//   Rows of up to 32768 positions keep their keys in registers from the
//   single read to the classes; rows up to 65536 read the scores twice. A
//   read issues all of its chunks (or a group of them) before it converts
//   the first to keys, so the chunks' loads are in flight together. When the candidates overflow their list
//   (scores crowding one bin), levels 1 and 2 and the marking read the row
//   again instead. Longer rows take a generic kernel, one workgroup per row,
//   that runs every level over the row, reads it again for each pass, and
//   orders the output with per-wave ballots and a scan of (chunk, wave)
//   totals.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 8192;     // level 0 digit: the key's top 13 bits
constexpr int kBatch = 8;       // 4096-position chunks per output batch
constexpr int kCand = 2048;     // candidate list capacity (a few hundred in practice)

__device__ __forceinline__ uint32_t score_key(uint32_t u) {
  if (u == 0x80000000u) u = 0u;   // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// LDS shared by both paths.
struct TopkLds {
  uint32_t hist[kBins];
  uint32_t red[kWaves];
  uint32_t found[2];
  uint32_t wsel[kBatch * kWaves + 1];   // output: (chunk, wave) totals, then bases
  uint32_t wtie[kBatch * kWaves + 1];
};

// OR of lanes 8j .. 8j+7 in lane 8j+7 (groups of 8 lie inside a DPP row).
__device__ __forceinline__ uint32_t or8_into_top(uint32_t v) {
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);   // row_shr:4
  return v;
}

static_assert(kWaves == 16, "the per-wave totals are scanned as one row of 16 lanes");

// Exclusive prefix over the block of one value per thread; *total gets the
// block's sum. Two barriers.
__device__ __forceinline__ uint32_t block_exclusive_scan(int tid, uint32_t v, uint32_t* red,
                                                         uint32_t* total) {
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t x = wave_scan64(v);
  if (lane == 63) red[wv] = x;
  __syncthreads();
  const uint32_t r = row_scan16(red[lane & 15]);   // lane w: waves 0..w
  __syncthreads();
  *total = (uint32_t)__builtin_amdgcn_readlane((int)r, kWaves - 1);
  const uint32_t before = (uint32_t)__builtin_amdgcn_readlane((int)r, wv > 0 ? wv - 1 : 0);
  return (wv > 0 ? before : 0u) + x - v;
}

// Prefix over the wave's lanes below this one, and the wave's total, of a
// count in 0..7 (three ballots; no cross-lane data movement).
__device__ __forceinline__ void wave_prefix3(uint32_t v, uint32_t* before, uint32_t* total) {
  uint32_t b = 0, t = 0;
#pragma unroll
  for (int bit = 0; bit < 3; ++bit) {
    const uint64_t m = __ballot((v >> bit) & 1u);
    b += __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))
         << bit;
    t += (uint32_t)__popcll(m) << bit;
  }
  *before = b;
  *total = t;
}

// After a histogram of nb bins: the bin holding the need-th largest counted
// key (scanning from the top bin down) and how many of that bin are still
// needed. *whole: the bin is needed entirely. Ends with hist reusable.
__device__ __forceinline__ void find_bin(TopkLds& L, int tid, int nb, uint32_t* need, uint32_t* bin,
                                         bool* whole) {
  const int per = nb >= kThreads ? nb / kThreads : 1;
  const int top = nb - 1 - per * tid;
  uint32_t mine = 0;
  for (int j = 0; j < per; ++j) mine += top - j >= 0 ? L.hist[top - j] : 0u;
  uint32_t tot;
  uint32_t above = block_exclusive_scan(tid, mine, L.red, &tot);
  if (above < *need && *need <= above + mine) {
    for (int j = 0; j < per; ++j) {
      const uint32_t h = L.hist[top - j];
      if (*need <= above + h) {
        L.found[0] = (uint32_t)(top - j);
        L.found[1] = *need - above;
        break;
      }
      above += h;
    }
  }
  __syncthreads();
  *bin = L.found[0] & (uint32_t)(nb - 1);   // exactly one thread found it
  *need = L.found[1];
  *whole = L.hist[*bin] == *need;
  __syncthreads();
}

// Output pass over chunks [0, nchunks) in position order. cls(i, &s, &t)
// gives this thread's 4 elements of chunk i as kept / tied flags (bit c).
// need: ties still to keep.
template <typename Cls>
__device__ __forceinline__ void write_output(TopkLds& L, int nchunks, uint32_t need, int k,
                                             int32_t* out, Cls&& cls) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint32_t carry_sel = 0, carry_tie = 0;   // totals of earlier batches
  for (int b0 = 0; b0 < nchunks; b0 += kBatch) {
    const int nb = nchunks - b0 < kBatch ? nchunks - b0 : kBatch;
    uint32_t lane_pre[kBatch], fsel[kBatch], ftie[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      lane_pre[j] = 0;
      fsel[j] = 0;
      ftie[j] = 0;
      if (j < nb) {
        cls(b0 + j, &fsel[j], &ftie[j]);
        uint32_t sb, st, tb, tt;
        wave_prefix3(__popc(fsel[j]), &sb, &st);
        wave_prefix3(__popc(ftie[j]), &tb, &tt);
        lane_pre[j] = (sb << 16) | tb;   // each at most 63 * 4
        if (lane == 0) {
          L.wsel[j * kWaves + wv] = st;
          L.wtie[j * kWaves + wv] = tt;
        }
      }
    }
    __syncthreads();
    // exclusive scans of the (chunk, wave) totals in position order: wave 0
    // scans the kept counts, wave 1 the tied ones
    if (wv < 2) {
      uint32_t* w = wv == 0 ? L.wsel : L.wtie;
      const uint32_t carry = wv == 0 ? carry_sel : carry_tie;
      const int e = 2 * lane;   // entries e, e+1 of kBatch * kWaves = 128
      const uint32_t a = e < nb * kWaves ? w[e] : 0u;
      const uint32_t b = e + 1 < nb * kWaves ? w[e + 1] : 0u;
      uint32_t x = a + b;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
      }
      const uint32_t ex = x - a - b;
      w[e] = carry + ex;
      w[e + 1] = carry + ex + a;
      if (lane == 63) w[kBatch * kWaves] = carry + x;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (j < nb && (fsel[j] | ftie[j])) {
        uint32_t kept = L.wsel[j * kWaves + wv] + (lane_pre[j] >> 16);
        uint32_t tied = L.wtie[j * kWaves + wv] + (lane_pre[j] & 0xffffu);
        const int pos = 4 * ((b0 + j) * kThreads + tid);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          // (the counts give exactly k writes; o < k keeps every store in the row)
          const uint32_t o = kept + (tied < need ? tied : need);
          const bool w = ((fsel[j] >> c) & 1u) || (((ftie[j] >> c) & 1u) && tied < need);
          if (w && o < (uint32_t)k) out[o] = pos + c;
          kept += (fsel[j] >> c) & 1u;
          tied += (ftie[j] >> c) & 1u;
        }
      }
    }
    carry_sel = L.wsel[kBatch * kWaves];
    carry_tie = L.wtie[kBatch * kWaves];
    __syncthreads();   // the totals are rewritten by the next batch
  }
}

// The raw score bits of this thread's positions 4 (i kThreads + tid) .. +3
// of chunk i. Loads only, and no use of their values, so that the loads of
// several chunks are all in flight before the first wait (a key computed
// inside the branch would make each load wait for itself). vlen: how many
// positions from the row's start may be read with 16-byte loads (the row's
// storage, kv_len, when the row is 16-byte aligned; else 0). A chunk inside
// that span is read with one 16-byte load per thread, the thread whose four
// positions straddle n included (keys4 masks what lies past n); other
// chunks read one score at a time, positions past n reading the row's last
// score. Positions of threads wholly past n get 0xffffffff, whose key is 0.
__device__ __forceinline__ void load4_raw(int tid, const float* row, int n, int vlen, int i,
                                          uint32_t r[4]) {
  const int base = 4 * i * kThreads;
  const int pos = base + 4 * tid;
  // (two independent uniform tests rather than if / else: at an if / else
  // join the compiler may give one side's load addresses the registers the
  // other side loads into, and then waits for older loads in flight)
  const bool wide = base < n && base + 4 * kThreads <= vlen;
  const bool narrow = !wide && base < n;
#pragma unroll
  for (int c = 0; c < 4; ++c) r[c] = 0xffffffffu;
  if (wide && pos < n) {
    const float4 v = *reinterpret_cast<const float4*>(row + pos);
    r[0] = __float_as_uint(v.x);
    r[1] = __float_as_uint(v.y);
    r[2] = __float_as_uint(v.z);
    r[3] = __float_as_uint(v.w);
  }
  if (narrow) {
#pragma unroll
    for (int c = 0; c < 4; ++c) r[c] = __float_as_uint(row[pos + c < n ? pos + c : n - 1]);
  }
}

// Keys of chunk i's positions from their raw bits, in place; 0 past the row
// (no score maps to 0).
__device__ __forceinline__ void keys4(int tid, int n, int i, uint32_t k4[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) k4[c] = score_key(k4[c]);
  const int base = 4 * i * kThreads;
  if (base < n && base + 4 * kThreads > n) {   // the chunk straddles the row's end (uniform)
    const int pos = base + 4 * tid;
#pragma unroll
    for (int c = 0; c < 4; ++c) k4[c] = pos + c < n ? k4[c] : 0u;
  }
}

__device__ __forceinline__ void load4_keys(int tid, const float* row, int n, int vlen, int i,
                                           uint32_t k4[4]) {
  load4_raw(tid, row, n, vlen, i, k4);
  keys4(tid, n, i, k4);
}

// Generic path, any row length: every level and the output re-read the
// row's scores (0 keys = past the row; no score maps to 0).
__device__ __forceinline__ void select_generic(TopkLds& L, const float* row, int n, int vlen, int k,
                               int32_t* out) {
  const int tid = threadIdx.x;
  const int nchunks = (n + 4 * kThreads - 1) / (4 * kThreads);
  uint32_t prefix = 0;
  int shift = 32;
  uint32_t need = (uint32_t)k;
#pragma unroll 1
  for (int level = 0; level < 3; ++level) {
    const int bits = level == 0 ? 13 : (level == 1 ? 11 : 8);
    const int sh = level == 0 ? 19 : (level == 1 ? 8 : 0);
    const int nb = 1 << bits;
    for (int b = tid; b < nb; b += kThreads) L.hist[b] = 0u;
    __syncthreads();
    for (int i = 0; i < nchunks; ++i) {
      uint32_t k4[4];
      load4_keys(tid, row, n, vlen, i, k4);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t kk = k4[c];
        if (kk != 0u && (shift == 32 || (kk >> shift) == prefix))
          atomicAdd(&L.hist[(kk >> sh) & (uint32_t)(nb - 1)], 1u);
      }
    }
    __syncthreads();
    uint32_t bin;
    bool whole;
    find_bin(L, tid, nb, &need, &bin, &whole);
    prefix = (shift == 32 ? 0u : prefix << bits) | bin;
    shift = sh;
    if (whole) break;
  }
  write_output(L, nchunks, need, k, out, [&](int i, uint32_t* fs, uint32_t* ft) {
    uint32_t k4[4];
    load4_keys(tid, row, n, vlen, i, k4);
    uint32_t s = 0, t = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t pk = k4[c] >> shift;
      s |= (uint32_t)(k4[c] != 0u && pk > prefix) << c;
      t |= (uint32_t)(k4[c] != 0u && pk == prefix) << c;
    }
    *fs = s;
    *ft = t;
  });
}

// Exclusive prefixes over the block of two values per thread; *t1, *t2
// get the block's sums. Two barriers; red holds 2 * kWaves words.
__device__ __forceinline__ void block_exclusive_scan2(int tid, uint32_t v1, uint32_t v2,
                                                      uint32_t* red,
                                                      uint32_t* e1, uint32_t* e2, uint32_t* t1,
                                                      uint32_t* t2) {
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t x1 = wave_scan64(v1), x2 = wave_scan64(v2);
  if (lane == 63) {
    red[wv] = x1;
    red[kWaves + wv] = x2;
  }
  __syncthreads();
  const uint32_t r1 = row_scan16(red[lane & 15]), r2 = row_scan16(red[kWaves + (lane & 15)]);
  __syncthreads();
  const int prev = wv > 0 ? wv - 1 : 0;
  const uint32_t b1 = (uint32_t)__builtin_amdgcn_readlane((int)r1, prev);
  const uint32_t b2 = (uint32_t)__builtin_amdgcn_readlane((int)r2, prev);
  *e1 = (wv > 0 ? b1 : 0u) + x1 - v1;
  *e2 = (wv > 0 ? b2 : 0u) + x2 - v2;
  *t1 = (uint32_t)__builtin_amdgcn_readlane((int)r1, kWaves - 1);
  *t2 = (uint32_t)__builtin_amdgcn_readlane((int)r2, kWaves - 1);
}

// Fast path for rows of at most kThreads * PER positions. Position bitmaps
// in LDS (bit j of word w = position 32 w + j): kept by level 0 (above the
// threshold bin, or all of a bin needed whole), and the candidates (keys in
// that bin) kept or tied after levels 1 and 2.
template <int PER>
struct FastLds : TopkLds {
  static constexpr int kWords = PER * kThreads / 32;
  uint32_t amap[kWords];
  uint32_t selb[kWords];
  uint32_t tieb[kWords];
  uint32_t red2[2 * kWaves];
  uint32_t ncand;
  uint32_t ckey[kCand];
  int32_t cpos[kCand];
};

// ---- sampled selection (rows held in registers, k <= kSampleMaxK) -------------
// A row's k-th largest key is bracketed from below by a threshold read off a
// sample of the row: every element at or above it goes to a candidate list
// (one compare per element, no atomics), and the exact selection runs on
// that list alone. The threshold is the bin (the key's top 11 bits) holding
// the sample's r-th largest key, r the expected rank of the row's k-th
// largest in the sample plus four standard deviations; whenever the list
// turns out to miss the k-th largest (fewer than k candidates) or to
// overflow, the row takes the full path instead, so the result never
// depends on the sample.
constexpr int kLevelBins = 2048;   // 11 bits per level
constexpr int kSCap = 6144;        // candidate list capacity (C1topk: about 1.6 k)
constexpr int kSampleMaxK = 4096;
constexpr int kSmall = 64;         // a bin this small is ranked by one wave

template <int PER>
struct SampledLds {
  static constexpr int kWords = PER * kThreads / 32;
  // (the list first: its stores' constant offsets fold into the instruction)
  uint32_t craw[kSCap];           // candidates: raw score bits
  uint32_t cpos[kSCap];           // and positions
  uint32_t hist[2][kLevelBins];   // [0]: the sample; then the levels alternate [1], [0], [1]
  uint32_t selb[kWords];          // kept, by position
  uint32_t tieb[kWords];          // tied at the final threshold, by position
  uint32_t red2[2 * kWaves];
  uint32_t ncand;
  uint32_t hi;                    // the row's largest key (above +0; else the largest key there is)
  uint32_t found[4];
  uint32_t nsmall;                // a threshold bin of at most kSmall candidates, ranked whole
  uint32_t skey[kSmall];
  uint32_t spos[kSmall];
  uint32_t smax, scount;          // the sample's largest key and its count
};

// Largest value over the wave's lanes (the DPP steps of wave_scan64 with max;
// lane 63 ends with it), in every lane.
__device__ __forceinline__ uint32_t wave_max64(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true));   // row_shr:1
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true));   // row_shr:2
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true));   // row_shr:4
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true));   // row_shr:8
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false));  // row_bcast:15
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// One wave: over nb bins of h (a power of two, at most 2048), with need
// = need_of(total count), the bin holding the need-th largest counted from
// the top bin down. found: the bin, how many of it are needed, whether that
// is all of it, and its count. Lane l sums bins [nb - per (l+1), nb - per l); the lane
// holding the need-th then has its bins spread over the wave.
template <int UNROLL, typename NeedOf>
__device__ __forceinline__ void wave_find(const uint32_t* h, int nb, NeedOf need_of, uint32_t* found) {
  const int lane = threadIdx.x & 63;
  const int per = nb >= 64 ? nb >> 6 : 1;
  const int top = nb - per * lane;
  uint32_t s = 0;
  if (top > 0) {
    if (per >= 4) {
      // UNROLL reads in flight (one where the row's keys still hold 32 registers)
#pragma unroll UNROLL
      for (int j = 0; j < per; j += 4) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(h + top - per + j);
        s += (v[0] + v[1]) + (v[2] + v[3]);
      }
    } else {
      for (int j = 0; j < per; ++j) s += h[top - 1 - j];
    }
  }
  const uint32_t incl = wave_scan64(s);
  const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  uint32_t need = need_of(total);   // 1 <= need <= total
  need = need < total ? need : total;   // (so that both searches below find a lane)
  const int L = __builtin_ctzll(__ballot(incl >= need));
  const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)incl, L) -
                         (uint32_t)__builtin_amdgcn_readlane((int)s, L);
  const int topL = nb - per * L;
  const uint32_t c = lane < per ? h[topL - 1 - lane] : 0u;
  const uint32_t incl2 = wave_scan64(c);
  const int M = __builtin_ctzll(__ballot(lane < per && above + incl2 >= need));
  const uint32_t cM = (uint32_t)__builtin_amdgcn_readlane((int)c, M);
  const uint32_t before = above + (uint32_t)__builtin_amdgcn_readlane((int)incl2, M) - cM;
  if (lane == 0) {
    found[0] = (uint32_t)(topL - 1 - M);
    found[1] = need - before;
    found[2] = cM == need - before;
    found[3] = cM;
  }
}

// The sampled selection of a row of n > k positions whose raw score bits
// sit in kreg, 0xffffffff at every position past the row (no score has
// those bits). Marks the kept positions in
// S.selb and the ties at the final threshold in S.tieb, sets *tie_need,
// and returns true; when the row needs the full path, runs full() once S
// is free for reuse and returns false. (full() is called here rather than
// by the caller so that no path out of the sampled selection still holds
// the row's registers.)
template <int PER, typename Full>
__device__ __forceinline__ bool sampled_select(SampledLds<PER>& S, int n, uint32_t k,
                                               const uint32_t* kreg, uint32_t* tie_need,
                                               Full&& full) {
  constexpr int NCH = PER / 4;
  constexpr int NWORDS = SampledLds<PER>::kWords;
  constexpr int E = kSCap / kThreads;   // list entries per thread
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t* flat = &S.hist[0][0];
  for (int b = tid; b < 2 * kLevelBins; b += kThreads) flat[b] = 0u;
  for (int w = tid; w < NWORDS; w += kThreads) S.selb[w] = S.tieb[w] = 0u;
  if (tid == 0) {
    S.ncand = 0u;
    S.hi = 0u;
    S.nsmall = 0u;
    S.smax = 0u;
    S.scount = 0u;
  }
  // sample: position 4 (c kThreads + tid) of chunk c = tid mod NCH
  const int cs = tid & (NCH - 1);
  // (each value passes through an empty asm, so the selects stay selects
  // rather than becoming an indexed read that would move kreg to memory)
  uint32_t sraw = kreg[0];
#pragma unroll
  for (int i = 1; i < NCH; ++i) {
    uint32_t v = kreg[4 * i];
    asm("" : "+v"(v));
    sraw = cs == i ? v : sraw;
  }
  const uint32_t skey = 4 * (cs * kThreads + tid) < n ? score_key(sraw) : 0u;
  __syncthreads();
  if (skey) atomicAdd(&S.hist[0][skey >> 21], 1u);
  {
    const uint32_t wmax = wave_max64(skey);
    const uint32_t wcnt = (uint32_t)__popcll(__builtin_amdgcn_ballot_w64(skey != 0u));
    if (lane == 0) {
      atomicMax(&S.smax, wmax);
      atomicAdd(&S.scount, wcnt);
    }
  }
  __syncthreads();
  if (wv == 0) {
    const float pk = (float)k / (float)n;
    auto need_of = [&](uint32_t ns) {
      const float mean = (float)ns * pk;
      const uint32_t r = (uint32_t)ceilf(mean + 4.f * sqrtf(mean * (1.f - pk)) + 4.f);
      return r < ns ? r : ns;
    };
    // The bin sought is usually a few below the sample's largest: lane l
    // takes bin top - l, and one scan finds it among those 64; otherwise
    // the search over all 2048 bins.
    const int topb = (int)(S.smax >> 21);
    const uint32_t total = S.scount;
    uint32_t need = need_of(total);
    need = need < total ? need : total;
    const int b = topb - lane;
    const uint32_t c = b >= 0 ? S.hist[0][b & (kLevelBins - 1)] : 0u;
    const uint32_t incl = wave_scan64(c);
    const uint64_t hit = __builtin_amdgcn_ballot_w64(incl >= need);
    if (hit) {   // uniform
      const int M = __builtin_ctzll(hit);
      const uint32_t cM = (uint32_t)__builtin_amdgcn_readlane((int)c, M);
      const uint32_t before = (uint32_t)__builtin_amdgcn_readlane((int)incl, M) - cM;
      if (lane == 0) {
        S.found[0] = (uint32_t)(topb - M);
        S.found[1] = need - before;
        S.found[2] = cM == need - before;
        S.found[3] = cM;
      }
    } else {
      wave_find<1>(S.hist[0], kLevelBins, need_of, S.found);
    }
  }
  __syncthreads();
  uint32_t tk = S.found[0] << 21;
  tk = tk ? tk : 1u;   // (0 keys are past the row)
  for (int b = tid; b < kLevelBins; b += kThreads) S.hist[0][b] = 0u;   // for the second level

  // ---- candidates: every element with key >= tk --------------------------
  // Above +0 the key order of the raw bits is their signed order, so one
  // compare decides; otherwise the key is formed first.
  // A bound on the largest key of the row comes out of the same pass: above
  // +0 the largest raw bits read as signed (the row's largest key itself);
  // otherwise the largest key there is (at most one more level).
  uint32_t top = 0xffffffffu;
  auto filter = [&](auto above_zero) {
    const int32_t tr = (int32_t)(tk ^ 0x80000000u);
    int32_t mraw = -1;
#pragma unroll
    for (int g = 0; g < NCH / 2; ++g) {   // two chunks per list allocation
      bool in[8];
      uint64_t bal[8];
      uint32_t tot = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t raw = kreg[8 * g + j];
        if constexpr (decltype(above_zero)::value) {
          in[j] = (int32_t)raw >= tr;
          mraw = max(mraw, (int32_t)raw);
        } else {
          in[j] = score_key(raw) >= tk;
        }
        bal[j] = __builtin_amdgcn_ballot_w64(in[j]);
        tot += (uint32_t)__popcll(bal[j]);
      }
      if (tot) {   // wave-uniform
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&S.ncand, tot);
        base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
        if (base + tot <= (uint32_t)kSCap) {   // else the list overflows: the full path
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if (in[j]) {
              // (the wave's base stays scalar: one shift-add forms the address)
              const uint32_t below = __builtin_amdgcn_mbcnt_hi(
                  (uint32_t)(bal[j] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal[j], 0u));
              S.craw[base + below] = kreg[8 * g + j];
              S.cpos[base + below] = (uint32_t)(4 * ((2 * g + (j >> 2)) * kThreads + tid) + (j & 3));
            }
            base += (uint32_t)__popcll(bal[j]);
          }
        }
      }
    }
    if constexpr (decltype(above_zero)::value) top = mraw < 0 ? 0u : (uint32_t)mraw | 0x80000000u;
  };
  if (tk > 0x80000000u) filter(std::true_type{});
  else filter(std::false_type{});
  top = wave_max64(top);
  if (lane == 0) atomicMax(&S.hi, top);
  __syncthreads();
  const uint32_t nc = S.ncand;
  if (nc < k || nc > (uint32_t)kSCap) {   // uniform
    __syncthreads();   // every thread has read ncand before the memory is reused
    full();
    return false;
  }

  // ---- exact selection on the list: keys relative to tk, 11 bits a level -----
  const uint32_t hi = S.hi - tk;   // (S.hi >= tk: the row's largest key is a candidate)
  uint32_t rk[E];
  int32_t rp[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t c = (uint32_t)(tid + e * kThreads);
    rk[e] = 0u;
    rp[e] = -1;
    if (c < nc) {
      rk[e] = score_key(S.craw[c]) - tk;
      rp[e] = (int32_t)S.cpos[c];
    }
  }
  const int nbits = hi ? 32 - __builtin_clz(hi) : 0;   // every relative key is below 2^nbits
  int sp = nbits;                                      // bits at and above sp: the prefix P
  int s = nbits > 11 ? nbits - 11 : 0;
  uint32_t P = 0, need = k;
  int hb = 1;
  while (true) {
    const int nb = 1 << (sp - s);
    uint32_t* h = S.hist[hb];
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (rp[e] >= 0 && (sp >= 32 || (rk[e] >> sp) == P))
        atomicAdd(&h[(rk[e] >> s) & (uint32_t)(nb - 1)], 1u);
    __syncthreads();
    if (wv == 0) wave_find<4>(h, nb, [&](uint32_t) { return need; }, S.found);
    __syncthreads();
    const uint32_t bin = S.found[0];
    need = S.found[1];
    const bool whole = S.found[2] != 0u;
    const uint32_t cnt = S.found[3];
    for (int b = tid; b < nb; b += kThreads) h[b] = 0u;   // (read only before the barrier)
    P = (sp >= 32 ? 0u : P << (sp - s)) | bin;
    sp = s;
    if (whole || s == 0) break;
    if (cnt <= (uint32_t)kSmall) {   // uniform
      // Everything above the bin is kept; the bin's cnt candidates are ranked
      // by one wave (larger key first, then lower position) and the first
      // `need` of them kept: no further level.
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (rp[e] >= 0) {
          const uint32_t pk = rk[e] >> sp;
          if (pk > P) {
            atomicOr(&S.selb[rp[e] >> 5], 1u << (rp[e] & 31));
          } else if (pk == P) {
            const uint32_t at = atomicAdd(&S.nsmall, 1u);   // < cnt <= kSmall
            S.skey[at] = rk[e];
            S.spos[at] = (uint32_t)rp[e];
          }
        }
      }
      __syncthreads();
      if (wv == 0) {
        const uint32_t key = lane < (int)cnt ? S.skey[lane] : 0u;
        const uint32_t pos = lane < (int)cnt ? S.spos[lane] : 0u;
        uint32_t rank = 0;
        for (int j = 0; j < (int)cnt; ++j) {
          const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)key, j);
          const uint32_t pj = (uint32_t)__builtin_amdgcn_readlane((int)pos, j);
          rank += (kj > key || (kj == key && pj < pos)) ? 1u : 0u;
        }
        if (lane < (int)cnt && rank < need) atomicOr(&S.selb[pos >> 5], 1u << (pos & 31));
      }
      *tie_need = 0;
      __syncthreads();
      return true;
    }
    s = s > 11 ? s - 11 : 0;
    hb ^= 1;
  }
  // kept above the final prefix, tied at it
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (rp[e] >= 0) {
      const uint32_t pk = sp >= 32 ? 0u : rk[e] >> sp;
      const uint32_t bit = 1u << (rp[e] & 31);
      if (pk > P) atomicOr(&S.selb[rp[e] >> 5], bit);
      else if (pk == P) atomicOr(&S.tieb[rp[e] >> 5], bit);
    }
  }
  *tie_need = need;
  __syncthreads();
  return true;
}

// Every row's visible length and, when it exceeds k, the selection.
__device__ __forceinline__ int row_length(const TopkParams& p, int t) {
  int n = p.kv_len;
  if (p.row_len) {
    const int r = p.row_len[t];
    n = r < 0 ? 0 : (r < n ? r : n);
  }
  return n;
}

// One workgroup per row. REG: the row's scores are read once into
// registers, all chunks requested before the first is used.
// Two rows per CU: 8 waves per SIMD, which bounds both register files.
template <int PER, bool REG, bool SAMPLED = false>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
topk_fast_kernel(TopkParams p) {
  // SAMPLED (rows in registers, k <= kSampleMaxK): the sampled selection
  // first, the full path only where it gives up; the two share the memory
  static_assert(!SAMPLED || REG, "the sampled selection reads the row from registers");
  union Lds {
    FastLds<PER> f;
    typename std::conditional<SAMPLED, SampledLds<PER>, TopkLds>::type s;
  };
  __shared__ Lds U;
  FastLds<PER>& L = U.f;
  constexpr int NCH = PER / 4;                      // 4096-position chunks
  // chunks per group: re-read groups are loaded whole before their first use
  constexpr int GCH = REG ? (NCH < 8 ? NCH : 8) : 4;
  static_assert(NCH % GCH == 0, "whole groups");
  constexpr int GUNROLL = REG ? NCH / GCH : 1;   // re-read groups stay a loop
  constexpr int NWORDS = FastLds<PER>::kWords;      // bitmap words
  constexpr int WPT = NWORDS >= kThreads ? NWORDS / kThreads : 1;   // words per owner
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int n = row_length(p, t);
  int32_t* out = p.idx + (int64_t)t * p.idx_row_stride;
  if (n <= p.k) {   // every visible position, then padding
    for (int j = tid; j < p.k; j += kThreads) out[j] = j < n ? j : -1;
    return;
  }
  const float* row = p.scores + (int64_t)t * p.score_row_stride;
  // 16-byte loads over the row's storage when the row is aligned for them
  const int vlen = (reinterpret_cast<uintptr_t>(row) & 15u) == 0 ? p.kv_len : 0;
  uint32_t kreg[REG ? PER : 1];
  if constexpr (REG) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) load4_raw(tid, row, n, vlen, i, &kreg[4 * i]);
  }
  // chunk group g's keys: REG, from the registers; else read now, the
  // group's chunks issued before their first use
  uint32_t kg[REG ? 1 : 4 * GCH];
  auto group_keys = [&](int g) {
    if constexpr (!REG) {
#pragma unroll
      for (int i8 = 0; i8 < GCH; ++i8) load4_raw(tid, row, n, vlen, GCH * g + i8, &kg[4 * i8]);
#pragma unroll
      for (int i8 = 0; i8 < GCH; ++i8) keys4(tid, n, GCH * g + i8, &kg[4 * i8]);
    }
  };
  auto keys = [&](int i, uint32_t k4[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) k4[c] = REG ? kreg[4 * i + c] : kg[4 * (i % GCH) + c];
  };
  uint32_t tie_need = 0;
  auto full_path = [&]() {
  if constexpr (SAMPLED) {
    // (keeps the key conversion below from being hoisted above the sampled
    // selection, where raw bits and keys would hold registers together)
#pragma unroll
    for (int i = 0; i < PER; ++i) asm volatile("" : "+v"(kreg[i]));
  }
  uint32_t need = (uint32_t)p.k, b0 = 0;
  bool whole0 = true;

  // ---- level 0 --------------------------------------------------------------
  for (int b = tid; b < kBins; b += kThreads) L.hist[b] = 0u;
  for (int w = tid; w < NWORDS; w += kThreads) L.selb[w] = L.tieb[w] = 0u;   // (amap: below)
  if (tid == 0) L.ncand = 0u;
  if constexpr (REG) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) keys4(tid, n, i, &kreg[4 * i]);
  }
  __syncthreads();
  // Past-the-row keys (0) are not counted: one bin taking thousands of
  // same-address atomics would serialise them.
#pragma unroll GUNROLL
  for (int g = 0; g < NCH / GCH; ++g) {
    group_keys(g);
#pragma unroll
    for (int i8 = 0; i8 < GCH; ++i8) {
      const int i = GCH * g + i8;
      uint32_t k4[4];
      keys(i, k4);
      if ((i + 1) * 4 * kThreads <= n) {   // the whole chunk is inside the row
#pragma unroll
        for (int c = 0; c < 4; ++c) atomicAdd(&L.hist[k4[c] >> 19], 1u);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (k4[c] != 0u) atomicAdd(&L.hist[k4[c] >> 19], 1u);
      }
    }
    if (!REG) __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  find_bin(L, tid, kBins, &need, &b0, &whole0);

  // ---- classes: kept into the bitmap, candidates into a list ----------------
  // chunk i covers positions 4 (i kThreads + tid) .. +3: one nibble of word
  // (i kThreads + tid) / 8, shared with the 7 neighbouring lanes; the eight
  // nibbles are ORed across lanes and the top lane writes the word (every
  // word once, so the bitmap needs no clearing). A chunk group's candidates
  // are appended to the list with one wave scan and one LDS atomic per wave;
  // the list is unordered (levels 1 and 2 count, the marks go by position).
#pragma unroll GUNROLL
  for (int g = 0; g < NCH / GCH; ++g) {
    group_keys(g);
    uint32_t cmask = 0;   // bit 4 i8 + c: candidate position c of chunk GCH g + i8
#pragma unroll
    for (int i8 = 0; i8 < GCH; ++i8) {
      const int i = GCH * g + i8;
      uint32_t k4[4];
      keys(i, k4);
      uint32_t a = 0, cm = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t d = k4[c] >> 19;   // (0 keys fall below b0)
        a |= (uint32_t)(d > b0 || (whole0 && d == b0)) << c;
        cm |= (uint32_t)(!whole0 && d == b0) << c;
      }
      const int pos0 = 4 * (i * kThreads + tid);
      const uint32_t word = or8_into_top(a << (pos0 & 31));
      if ((tid & 7) == 7) L.amap[pos0 >> 5] = word;
      cmask |= cm << (4 * i8);
      // (materialised per chunk: the compare masks would otherwise stay in
      // scalar registers until the group ends, 64 of them for eight chunks,
      // enough to keep a second workgroup off the CU)
      __asm__ volatile("" : "+v"(cmask));
    }
    if (!whole0) {
      const uint32_t cnt = (uint32_t)__popc(cmask);
      const uint32_t incl = wave_scan64(cnt);
      const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      if (total) {   // wave-uniform
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&L.ncand, total);
        uint32_t at = (uint32_t)__builtin_amdgcn_readlane((int)base, 0) + incl - cnt;
#pragma unroll
        for (int i8 = 0; i8 < GCH; ++i8) {
          const uint32_t nib = (cmask >> (4 * i8)) & 0xfu;
          if (nib) {
            const int i = GCH * g + i8;
            uint32_t k4[4];
            keys(i, k4);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              if ((nib >> c) & 1u) {
                if (at < (uint32_t)kCand) {
                  L.ckey[at] = k4[c];
                  L.cpos[at] = 4 * (i * kThreads + tid) + c;
                }
                ++at;
              }
            }
          }
        }
      }
    }
    if (!REG) __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();

  // ---- levels 1 and 2 on the candidates (or, on overflow, the row) ---------
  if (!whole0) {
    const uint32_t nc = L.ncand;
    const bool spill = nc > (uint32_t)kCand;   // candidates overflow their list
    uint32_t prefix = b0;
    int shift = 19;
#pragma unroll 1
    for (int level = 1; level < 3; ++level) {
      const int bits = level == 1 ? 11 : 8;
      const int sh = level == 1 ? 8 : 0;
      const int nb = 1 << bits;
      for (int b = tid; b < nb; b += kThreads) L.hist[b] = 0u;
      __syncthreads();
      if (!spill) {
        for (uint32_t c = tid; c < nc; c += kThreads) {
          const uint32_t kk = L.ckey[c];
          if ((kk >> shift) == prefix) atomicAdd(&L.hist[(kk >> sh) & (uint32_t)(nb - 1)], 1u);
        }
      } else {
#pragma unroll 1
        for (int i = 0; i < NCH; ++i) {
          uint32_t k4[4];
          load4_keys(tid, row, n, vlen, i, k4);
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (k4[c] != 0u && (k4[c] >> shift) == prefix)
              atomicAdd(&L.hist[(k4[c] >> sh) & (uint32_t)(nb - 1)], 1u);
        }
      }
      __syncthreads();
      uint32_t bin;
      bool whole;
      find_bin(L, tid, nb, &need, &bin, &whole);
      prefix = (prefix << bits) | bin;
      shift = sh;
      if (whole) break;
    }
    // mark the candidates: kept above the threshold prefix, tied at it
    auto mark = [&](uint32_t kk, int pos) {
      const uint32_t pk = kk >> shift;
      if (pk > prefix) atomicOr(&L.selb[pos >> 5], 1u << (pos & 31));
      else if (pk == prefix) atomicOr(&L.tieb[pos >> 5], 1u << (pos & 31));
    };
    if (!spill) {
      for (uint32_t c = tid; c < nc; c += kThreads) mark(L.ckey[c], L.cpos[c]);
    } else {
#pragma unroll 1
      for (int i = 0; i < NCH; ++i) {
        uint32_t k4[4];
        load4_keys(tid, row, n, vlen, i, k4);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (k4[c] != 0u && (k4[c] >> 19) == b0) mark(k4[c], 4 * (i * kThreads + tid) + c);
      }
    }
    tie_need = need;
    __syncthreads();
  }

  };   // full path
  bool sampled = false;
  if constexpr (SAMPLED) {
    // the chunk that reaches the row's end: its positions past n (a 16-byte
    // read may cover them) become 0xffffffff, like the chunks wholly past it
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      if (4 * i * kThreads < n && 4 * (i + 1) * kThreads > n) {   // uniform
#pragma unroll
        for (int c = 0; c < 4; ++c)
          kreg[4 * i + c] = 4 * (i * kThreads + tid) + c < n ? kreg[4 * i + c] : 0xffffffffu;
      }
    }
    sampled = sampled_select<PER>(U.s, n, (uint32_t)p.k, kreg, &tie_need, full_path);
  }
  else full_path();

  // ---- output from the bitmaps, in position order ----------------------------
  // An element goes to (kept before it) + min(tied before it, tie_need); a
  // tie is kept while fewer than tie_need ties precede it.
  uint32_t ksel[WPT], ktie[WPT], ns = 0, nt = 0;
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int w = tid * WPT + j;
    uint32_t sw = 0, tw = 0;
    if (w < NWORDS) {
      sw = L.amap[w] | L.selb[w];
      tw = L.tieb[w];
      if constexpr (SAMPLED) {
        if (sampled) {
          sw = U.s.selb[w];
          tw = U.s.tieb[w];
        }
      }
    }
    ksel[j] = sw;
    ktie[j] = tw;
    ns += __popc(ksel[j]);
    nt += __popc(ktie[j]);
  }
  uint32_t kept, tied, ts, tt;
  uint32_t* red2 = L.red2;
  if constexpr (SAMPLED) {
    if (sampled) red2 = U.s.red2;
  }
  block_exclusive_scan2(tid, ns, nt, red2, &kept, &tied, &ts, &tt);
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int w = tid * WPT + j;
    uint32_t m = ksel[j] | ktie[j];
    while (m) {
      const int b = __builtin_ctz(m);
      m &= m - 1u;
      // (the counts give exactly k writes; o < k keeps every store in the row)
      const uint32_t o = kept + (tied < tie_need ? tied : tie_need);
      if ((ksel[j] >> b) & 1u) {
        if (o < (uint32_t)p.k) out[o] = 32 * w + b;
        ++kept;
      } else {
        if (tied < tie_need && o < (uint32_t)p.k) out[o] = 32 * w + b;
        ++tied;
      }
    }
  }
}

__global__ void __launch_bounds__(kThreads) topk_generic_kernel(TopkParams p) {
  __shared__ TopkLds L;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = row_length(p, t);
  int32_t* out = p.idx + (int64_t)t * p.idx_row_stride;
  if (n <= p.k) {
    for (int j = tid; j < p.k; j += kThreads) out[j] = j < n ? j : -1;
    return;
  }
  const float* row = p.scores + (int64_t)t * p.score_row_stride;
  select_generic(L, row, n, (reinterpret_cast<uintptr_t>(row) & 15u) == 0 ? p.kv_len : 0, p.k,
                 out);
}

}  // namespace

hipError_t launch_topk(const TopkParams& p, hipStream_t stream) {
  const int kv = p.kv_len;
  const dim3 grid((unsigned)p.num_rows), block(kThreads);
  const bool sampled = p.k <= kSampleMaxK;
  if (kv <= 4 * kThreads)
    hipLaunchKernelGGL((topk_fast_kernel<4, true>), grid, block, 0, stream, p);
  else if (kv <= 16 * kThreads && sampled)
    hipLaunchKernelGGL((topk_fast_kernel<16, true, true>), grid, block, 0, stream, p);
  else if (kv <= 16 * kThreads)
    hipLaunchKernelGGL((topk_fast_kernel<16, true>), grid, block, 0, stream, p);
  else if (kv <= 32 * kThreads && sampled)
    hipLaunchKernelGGL((topk_fast_kernel<32, true, true>), grid, block, 0, stream, p);
  else if (kv <= 32 * kThreads)
    hipLaunchKernelGGL((topk_fast_kernel<32, true>), grid, block, 0, stream, p);
  else if (kv <= 64 * kThreads)
    hipLaunchKernelGGL((topk_fast_kernel<64, false>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(topk_generic_kernel, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa
