// Sparse MLA decode over the split pool (sglang PR 32320: the decode kernel
// that reads the 64-token pages the page split writes).
//
// Decode has one query row per request, so one team per request would leave
// most of the chip idle. Each request's slots are therefore cut into ranges
// of whole 16-slot tiles, one two-wave team per (request, range) in the kDecode
// mode of attn_kernel: it gathers the range's FP8 records straight from the
// pages, and writes the range's normalised O and its LSE. The merge then
// weighs range s of (b, h) by exp(lse_s - LSE) with
// LSE = log sum_s exp(lse_s), which is the softmax over the union of the
// ranges; a range without a valid slot has lse_s = -inf, weight 0, and its
// O is neither written nor read. Range s takes the request's slot tiles
// s, s + S, s + 2S, ..., so valid slots that come first in a request's list
// (as decode indices often do: the newest tokens, then -1) spread over all
// its ranges.
#include "sa_attn_kernel.h"

namespace sa {

namespace {

constexpr int kCombineThreads = 128;   // two waves; 4 of the 512 output columns each
constexpr int kCombineChunk = 256;     // ranges compacted per pass
constexpr float kLog2e = 1.4426950408889634f;

// max (sum) over the block's two waves; every thread gets the result
template <bool MAX>
__device__ __forceinline__ float block_reduce(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float w = __shfl_xor(v, o);
    v = MAX ? fmaxf(v, w) : v + w;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = MAX ? fmaxf(red[0], red[1]) : red[0] + red[1];
  __syncthreads();
  return v;
}

// One workgroup per (request, head). The ranges' LSEs are read in parallel;
// the ranges that wrote an O are compacted into a list (in chunks), whose O
// rows are then read four at a time.
__global__ void __launch_bounds__(kCombineThreads) decode_combine_kernel(DecodeCombineParams c) {
  __shared__ float red[kCombineThreads / 64];
  __shared__ int list_s[kCombineChunk];
  __shared__ float list_w[kCombineChunk];
  __shared__ int list_n;
  const int tid = threadIdx.x, lane = tid & 63;
  const int H = c.num_q_heads;
  const int b = blockIdx.x / H;
  const int h = blockIdx.x - b * H;
  const int S = c.splits;
  const float* pl = c.part_lse + (int64_t)b * S * H + h;   // range s at pl[s * H]
  float* orow = c.out + (int64_t)b * c.out_row_stride + (int64_t)h * 512 + 4 * tid;

  float mx = -INFINITY;
  for (int s = tid; s < S; s += kCombineThreads) mx = fmaxf(mx, pl[(int64_t)s * H]);
  mx = block_reduce<true>(mx, red);
  if (mx == -INFINITY) {   // no valid slot in any range
    st16(orow, (f32x4_t){0.f, 0.f, 0.f, 0.f});
    if (tid == 0) c.lse[(int64_t)b * H + h] = -INFINITY;
    return;
  }
  float dn = 0.f;
  for (int s = tid; s < S; s += kCombineThreads) {
    const float ls = pl[(int64_t)s * H];
    dn += ls == -INFINITY ? 0.f : exp2f((ls - mx) * kLog2e);
  }
  dn = block_reduce<false>(dn, red);
  const float inv = 1.f / dn;

  const float* po = c.part_out + ((int64_t)b * S * H + h) * 512 + 4 * tid;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < S; c0 += kCombineChunk) {
    const int c1 = S < c0 + kCombineChunk ? S : c0 + kCombineChunk;
    if (tid < 64) {
      int n = 0;
      for (int s0 = c0; s0 < c1; s0 += 64) {
        const int s = s0 + lane;
        const float ls = s < c1 ? pl[(int64_t)s * H] : -INFINITY;
        const bool nz = ls != -INFINITY;
        const uint64_t m = (uint64_t)__ballot(nz);
        if (nz) {
          const int at = n + __popcll(m & ((1ull << lane) - 1ull));
          list_s[at] = s;
          list_w[at] = exp2f((ls - mx) * kLog2e) * inv;
        }
        n += __popcll(m);
      }
      if (lane == 0) list_n = n;
    }
    __syncthreads();
    const int n = list_n;
    for (int i = 0; i < n; i += 4) {
      f32x4_t o[4];
      float w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = i + k < n ? i + k : i;
        w[k] = i + k < n ? list_w[j] : 0.f;
        o[k] = *reinterpret_cast<const f32x4_t*>(po + (int64_t)list_s[j] * H * 512);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) acc += w[k] * o[k];
    }
    __syncthreads();   // the list is rewritten by the next chunk
  }
  st16(orow, acc);
  if (tid == 0) c.lse[(int64_t)b * H + h] = mx + logf(dn);
}

}  // namespace

hipError_t launch_decode_mla576_fp8(AttnParams p, const DecodeCombineParams& c,
                                    hipStream_t stream) {
  p.rows_per_team = 1;
  // one team per (request, range); more than 16 heads run as 16-head
  // slices, each writing its heads' columns of the partial results
  for (int h0 = 0; h0 < p.group; h0 += 16) {
    AttnParams ps = p;
    ps.group = ps.num_q_heads = p.group - h0 < 16 ? p.group - h0 : 16;
    ps.q = p.q + (int64_t)h0 * 576;
    ps.out = p.out + (int64_t)h0 * 512;
    ps.lse = p.lse + h0;
    dim3 grid, block;
    if (!attn_grid<2>(ps, kRows, &grid, &block)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_kernel<576, 512, true, kDecode, 1, 2, true, 2>), grid, block, 0,
                       stream, ps);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t blocks = (int64_t)c.batch * c.num_q_heads;
  if (blocks * kCombineThreads > (int64_t)UINT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)blocks),
                     dim3(kCombineThreads), 0, stream, c);
  return hipGetLastError();
}

}  // namespace sa
