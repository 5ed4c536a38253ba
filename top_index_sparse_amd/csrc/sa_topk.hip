// Indexer top-k selection (sglang PR 37275, "Motivation": the indexer
// selects 2051 token slots per query row; rows whose visible context is
// shorter select fewer). Row t keeps the k largest of its first n_t scores,
// equal scores going to the lower position, and writes the kept positions in
// ascending order; a row with n_t <= k writes 0 .. n_t - 1 and pads with -1.
//
// gfx950 design: one 1024-thread workgroup per row.
//   Keys. A score's bits map to a uint32 key whose unsigned order is the
//   float order (-0 is folded onto +0 first, so the two tie). Rows of at
//   most 32768 positions keep their keys in registers after one read (up to
//   32 per thread; 64 would spill at 1024 threads); longer rows read the
//   scores again for every pass.
//   Threshold. A radix select over the key's top 11, next 11 and last 10
//   bits: an LDS histogram of the keys that share the prefix found so far,
//   then a block-wide scan from the top bin down finds the bin holding the
//   k-th largest key. It stops early when that whole bin is kept.
//   Output. The row is walked in position order, 4096 positions at a time
//   (4 consecutive per thread): a block-wide scan of (kept, tied) counts
//   gives every thread its output offset, and tied keys are kept while
//   their rank among the row's ties is below the number still needed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;

__device__ __forceinline__ uint32_t score_key(uint32_t u) {
  if (u == 0x80000000u) u = 0u;   // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix over the block of one value per thread; *total gets the
// block's sum. Two barriers; red holds kWaves words.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* red,
                                                         uint32_t* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) red[wv] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t s = red[w];
    before += w < wv ? s : 0u;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// PER > 0: keys held in registers (n <= kThreads * PER); PER == 0: re-read.
template <int PER>
__global__ void __launch_bounds__(kThreads) topk_kernel(TopkParams p) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t red[kWaves];
  __shared__ uint32_t found[2];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  int n = p.kv_len;
  if (p.row_len) {
    const int r = p.row_len[t];
    n = r < 0 ? 0 : (r < n ? r : n);
  }
  int32_t* out = p.idx + (int64_t)t * p.idx_row_stride;
  if (n <= p.k) {   // every visible position, then padding
    for (int j = tid; j < p.k; j += kThreads) out[j] = j < n ? j : -1;
    return;
  }
  const float* row = p.scores + (int64_t)t * p.score_row_stride;
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;   // 16-byte loads
  const int nchunks = PER > 0 ? PER / 4 : (n + 4 * kThreads - 1) / (4 * kThreads);

  // keys of chunk i: positions 4 (i kThreads + tid) .. +3; 0 = past the row
  // (no score maps to 0: only NaN bit patterns would)
  auto load4 = [&](int i, uint32_t k4[4]) {
    const int pos = 4 * (i * kThreads + tid);
    if (vec && pos + 3 < n) {
      const float4 v = *reinterpret_cast<const float4*>(row + pos);
      k4[0] = score_key(__float_as_uint(v.x));
      k4[1] = score_key(__float_as_uint(v.y));
      k4[2] = score_key(__float_as_uint(v.z));
      k4[3] = score_key(__float_as_uint(v.w));
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) k4[c] = pos + c < n ? score_key(__float_as_uint(row[pos + c])) : 0u;
    }
  };
  uint32_t kreg[PER > 0 ? PER : 1];
  if constexpr (PER > 0) {
#pragma unroll
    for (int i = 0; i < PER / 4; ++i) load4(i, &kreg[4 * i]);
  }
  auto chunk = [&](int i, uint32_t k4[4]) {
    if constexpr (PER > 0) {
#pragma unroll
      for (int c = 0; c < 4; ++c) k4[c] = kreg[4 * i + c];
    } else {
      load4(i, k4);
    }
  };
  // every chunk in order (unrolled when the keys are registers)
  auto for_chunks = [&](auto&& body) {
    if constexpr (PER > 0) {
#pragma unroll
      for (int i = 0; i < PER / 4; ++i) body(i);
    } else {
      for (int i = 0; i < nchunks; ++i) body(i);
    }
  };

  // ---- threshold: prefix of the k-th largest key ------------------------
  uint32_t prefix = 0;   // bins found so far
  int shift = 32;        // keys are compared as key >> shift against prefix
  uint32_t need = (uint32_t)p.k;
#pragma unroll 1
  for (int level = 0; level < 3; ++level) {
    const int sh = level == 0 ? 21 : (level == 1 ? 10 : 0);
    const uint32_t mask = level == 2 ? 0x3ffu : 0x7ffu;
    hist[tid] = 0u;
    hist[tid + kThreads] = 0u;
    __syncthreads();
    for_chunks([&](int i) {
      uint32_t k4[4];
      chunk(i, k4);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t kk = k4[c];
        if (kk != 0u && (shift == 32 || (kk >> shift) == prefix))
          atomicAdd(&hist[(kk >> sh) & mask], 1u);
      }
    });
    __syncthreads();
    // bins 2047 - 2 tid and 2046 - 2 tid, scanned from the top bin down
    const uint32_t ha = hist[kBins - 1 - 2 * tid], hb = hist[kBins - 2 - 2 * tid];
    uint32_t tot;
    const uint32_t above = block_exclusive_scan(ha + hb, red, &tot);
    if (above < need && need <= above + ha) {
      found[0] = kBins - 1 - 2 * tid;
      found[1] = need - above;
    } else if (above + ha < need && need <= above + ha + hb) {
      found[0] = kBins - 2 - 2 * tid;
      found[1] = need - above - ha;
    }
    __syncthreads();
    const uint32_t bin = found[0] & (kBins - 1);   // exactly one thread found it
    need = found[1];
    prefix = (shift == 32 ? 0u : prefix << (level == 2 ? 10 : 11)) | bin;
    shift = sh;
    const bool whole = hist[bin] == need;   // the bin is kept entirely
    __syncthreads();                        // hist and found are reused
    if (whole) break;
  }

  // ---- output in position order ------------------------------------------
  uint32_t written = 0, ties_before = 0;
  for_chunks([&](int i) {
    uint32_t k4[4];
    chunk(i, k4);
    uint32_t nsel = 0, ntie = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t pk = k4[c] >> shift;
      nsel += k4[c] != 0u && pk > prefix;
      ntie += k4[c] != 0u && pk == prefix;
    }
    uint32_t tot;
    const uint32_t pre = block_exclusive_scan((nsel << 16) | ntie, red, &tot);
    const uint32_t quota = need > ties_before ? need - ties_before : 0u;
    uint32_t tie_rank = pre & 0xffffu;
    uint32_t o = written + (pre >> 16) + (tie_rank < quota ? tie_rank : quota);
    const int pos = 4 * (i * kThreads + tid);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t pk = k4[c] >> shift;
      if (k4[c] == 0u) continue;
      // (the counts give exactly k writes; o < k keeps every store in the row)
      if (pk > prefix) {
        if (o < (uint32_t)p.k) out[o] = pos + c;
        ++o;
      } else if (pk == prefix) {
        if (tie_rank < quota) {
          if (o < (uint32_t)p.k) out[o] = pos + c;
          ++o;
        }
        ++tie_rank;
      }
    }
    const uint32_t tsel = tot >> 16, ttie = tot & 0xffffu;
    written += tsel + (ttie < quota ? ttie : quota);
    ties_before += ttie;
  });
}

}  // namespace

hipError_t launch_topk(const TopkParams& p, hipStream_t stream) {
  const int kv = p.kv_len;
  const dim3 grid((unsigned)p.num_rows), block(kThreads);
  if (kv <= 4 * kThreads)
    hipLaunchKernelGGL(topk_kernel<4>, grid, block, 0, stream, p);
  else if (kv <= 16 * kThreads)
    hipLaunchKernelGGL(topk_kernel<16>, grid, block, 0, stream, p);
  else if (kv <= 32 * kThreads)
    hipLaunchKernelGGL(topk_kernel<32>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(topk_kernel<0>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa
