// Per-token sparse GQA prefill, head dim 256, for gfx950.
//
// What it computes (sglang PR 37275, "Motivation" and the mechanism note
// under it; PR 32779, "Motivation"): one program per query row and KV head;
// the KV group's query heads are padded into one 16-row matrix tile; the row
// streams its own selected K/V slots; the online softmax lives in registers;
// no split partials reach HBM.
//
// gfx950 design. One wavefront owns one (row, KV head); four independent
// wavefronts (four consecutive rows) form a workgroup, with no barrier and
// no LDS. The work of a 16-slot tile is three MFMA chains whose operand
// layouts are chosen so that every gathered byte goes straight from global
// memory into the register where the matrix core wants it:
//
//   S^T[slot, head] = K_tile(16 x 256) . Q^T(256 x 16)     8 x mfma 16x16x32
//     lane (g = l/16, m = l%16) loads 8 x 16 B of K row idx[slot m] at
//     d = 32s + 8g: four lanes cover 64 contiguous bytes per instruction.
//   P^T = exp2(S^T - m): the S^T accumulator (lane (g, n) holds slots
//     4g..4g+3 of head n) is already the B operand of the next product.
//   O^T[d, head] += V^T(16 x 16 slots) . P^T(16 x 16)     16 x mfma 16x16x16
//     lane (g, m) loads V rows idx[slot 4g+i] (i < 4) at bytes 16m and
//     256+16m: one instruction covers 256 contiguous bytes of four rows.
//     M-tile mt, row m of the A operand stands for d = 128(mt/8) + 8m + mt%8,
//     which is element mt%8 of chunk mt/8 the lane already holds, so V needs
//     no transpose through LDS.
//   Every O^T accumulator of lane (g, n) belongs to head n, whose running
//   max and sum the lane holds after two cross-lane max steps per tile.
//
// Two tiles of K/V (32 KB per wavefront) are in flight while one is being
// consumed; indices are fetched one tile further ahead. Invalid slots
// (outside [0, kv_len), beyond topk or topk_len) issue no memory traffic and
// are masked to -inf before the softmax.
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int D = 256;
constexpr int KSTEPS = D / 32;  // k-steps of the S^T product
constexpr int MTILES = D / 16;  // 16-wide d blocks of O^T
constexpr int TILE = 16;        // slots per tile

#ifndef SA_GQA_NBUF
#define SA_GQA_NBUF 1
#endif
#ifndef SA_GQA_WAVES
#define SA_GQA_WAVES 2
#endif
constexpr int kNbuf = SA_GQA_NBUF;    // K/V tiles in flight per wavefront
constexpr int kWaves = SA_GQA_WAVES;  // wavefronts per SIMD the registers allow

struct TileIdx {
  int xk;                       // slot m's index (K operand rows)
  int xv[4];                    // slots 4g..4g+3 (V operand, softmax columns)
};

struct TileData {
  u32x4_t kd[KSTEPS];
  u32x4_t vd[8];                // vd[2i + h]: slot 4g+i, d = 128h + 8m .. +7
  uint32_t vmask;               // bit i: slot 4g+i is valid
};

template <bool RAGGED, int NBUF, int WAVES>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(WAVES, WAVES)))
gqa_d256_kernel(AttnParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int n = lane & 15;

  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int quads = (p.num_rows + 3) >> 2;
  const int kvh = bid / quads;
  const int t = (bid - kvh * quads) * 4 + wave;
  if (t >= p.num_rows) return;

  int64_t kv_base = 0;
  int kv_len = p.kv_len;
  if (RAGGED) {
    int lo = 0, hi = p.num_reqs - 1;  // last request whose first row is <= t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.cu_q[mid] <= t) lo = mid; else hi = mid - 1;
    }
    kv_base = p.cu_kv[lo];
    kv_len = (int)(p.cu_kv[lo + 1] - kv_base);
  }

  int jmax = p.topk;
  if (p.topk_len) {
    const int tl = p.topk_len[t];
    jmax = tl < 0 ? 0 : (tl < jmax ? tl : jmax);
  }
  if (kv_len <= 0) jmax = 0;
  const int ntiles = (jmax + TILE - 1) / TILE;

  const int32_t* irow = p.idx + (int64_t)t * p.idx_row_stride;
  const uint16_t* kbase = p.k + kv_base * p.k_row_stride + kvh * D + 8 * g;
  const uint16_t* vbase = p.v + kv_base * p.v_row_stride + kvh * D + 8 * n;

  // Q^T operand: lane (g, n) holds head n, d = 32s + 8g .. +7.
  u32x4_t qop[KSTEPS];
  {
    const bool live = n < p.group;
    const uint16_t* qp = p.q + (int64_t)t * p.q_row_stride + (int64_t)(kvh * p.group + n) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qop[s] = live ? ld16(qp + 32 * s) : (u32x4_t){0, 0, 0, 0};
  }

  auto load_idx = [&](TileIdx& ti, int j0) {
    const int jk = j0 + n;
    ti.xk = jk < jmax ? irow[jk] : -1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int jv = j0 + 4 * g + i;
      ti.xv[i] = jv < jmax ? irow[jv] : -1;
    }
  };

  auto load_data = [&](TileData& td, const TileIdx& ti) {
    const bool kok = (unsigned)ti.xk < (unsigned)kv_len;
    const uint16_t* kp = kbase + (int64_t)(kok ? ti.xk : 0) * p.k_row_stride;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) td.kd[s] = (u32x4_t){0, 0, 0, 0};
    if (kok) {
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) td.kd[s] = ld16(kp + 32 * s);
    }
    uint32_t mask = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = (unsigned)ti.xv[i] < (unsigned)kv_len;
      mask |= (uint32_t)ok << i;
      const uint16_t* vp = vbase + (int64_t)(ok ? ti.xv[i] : 0) * p.v_row_stride;
      td.vd[2 * i] = (u32x4_t){0, 0, 0, 0};
      td.vd[2 * i + 1] = (u32x4_t){0, 0, 0, 0};
      if (ok) {
        td.vd[2 * i] = ld16(vp);
        td.vd[2 * i + 1] = ld16(vp + 128);
      }
    }
    td.vmask = mask;
  };

  float m_run = -INFINITY;  // running max of head n (log2 domain)
  float l_run = 0.f;        // this lane's share of the running sum
  f32x4_t acc[MTILES];
#pragma unroll
  for (int mt = 0; mt < MTILES; ++mt) acc[mt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  const float c = p.scale_log2e;

  auto compute = [&](const TileData& td) {
    f32x4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) st = mfma_16x16x32(td.kd[s], qop[s], st);
    float s2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s2[i] = ((td.vmask >> i) & 1u) ? st[i] * c : -INFINITY;
    float mx = fmaxf(fmaxf(s2[0], s2[1]), fmaxf(s2[2], s2[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(s2[i] - m_use);
    l_run = l_run * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    m_run = m_new;
#pragma unroll
    for (int mt = 0; mt < MTILES; ++mt) acc[mt] *= alpha;
    const i16x4_t pop =
        __builtin_bit_cast(i16x4_t, (u32x2_t){pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])});
#pragma unroll
    for (int mt = 0; mt < MTILES; ++mt) {
      const int h = mt >> 3, e = mt & 7;
      const i16x4_t a = gather_col4(td.vd[h], td.vd[2 + h], td.vd[4 + h], td.vd[6 + h], e);
      acc[mt] = mfma_16x16x16(a, pop, acc[mt]);
    }
  };

  // Software pipeline over NBUF register buffers: before tile `cur` is
  // consumed, the data loads of tile cur+NBUF-1 and the index loads of tile
  // cur+NBUF are issued.
  TileIdx ib[NBUF];
  TileData db[NBUF];
#pragma unroll
  for (int u = 0; u < NBUF; ++u)
    if (u < ntiles) load_idx(ib[u], u * TILE);
#pragma unroll
  for (int u = 0; u + 1 < NBUF; ++u)
    if (u < ntiles) load_data(db[u], ib[u]);
  for (int tile = 0; tile < ntiles; tile += NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      const int cur = tile + u;
      if (cur >= ntiles) break;
      const int nb = (u + NBUF - 1) % NBUF;
      if (cur + NBUF - 1 < ntiles) {
        load_data(db[nb], ib[nb]);
        if (cur + NBUF < ntiles) load_idx(ib[u], (cur + NBUF) * TILE);
      }
      compute(db[u]);
    }
  }

  float l = l_run + __shfl_xor(l_run, 16);
  l += __shfl_xor(l, 32);
  if (n < p.group) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int head = kvh * p.group + n;
    float* orow = p.out + (int64_t)t * p.out_row_stride + (int64_t)head * D;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 128 * h + 32 * g + 8 * i;
        const f32x4_t lo = {acc[8 * h + 0][i], acc[8 * h + 1][i], acc[8 * h + 2][i], acc[8 * h + 3][i]};
        const f32x4_t hi = {acc[8 * h + 4][i], acc[8 * h + 5][i], acc[8 * h + 6][i], acc[8 * h + 7][i]};
        st16(orow + d0, lo * inv);
        st16(orow + d0 + 4, hi * inv);
      }
    }
    if (g == 0)
      p.lse[(int64_t)t * p.num_q_heads + head] = l > 0.f ? (m_run + fast_log2(l)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_gqa_d256(const AttnParams& p, bool ragged, hipStream_t stream) {
  const int quads = (p.num_rows + 3) / 4;
  const dim3 grid((unsigned)(quads * p.num_kv_heads)), block(256);
  if (ragged)
    hipLaunchKernelGGL((gqa_d256_kernel<true, kNbuf, kWaves>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((gqa_d256_kernel<false, kNbuf, kWaves>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa
