// Sparse MLA decode over the split pool (sglang PR 32320: the decode kernel
// that reads the 64-token pages the page split writes).
//
// Decode has one query row per request, so one team per request would leave
// most of the chip idle. Each request's slots are therefore cut into ranges
// of dec_split_len, one two-wave team per (request, range) in the kDecode
// mode of attn_kernel: it gathers the range's FP8 records straight from the
// pages, and writes the range's normalised O and its LSE. The merge then
// weighs range s of (b, h) by exp(lse_s - LSE) with
// LSE = log sum_s exp(lse_s), which is the softmax over the union of the
// ranges; a range without a valid slot has lse_s = -inf, weight 0, and its
// O is neither written nor read.
#include "sa_attn_kernel.h"

namespace sa {

namespace {

constexpr int kCombineThreads = 128;   // 4 of the 512 output columns each
constexpr float kLog2e = 1.4426950408889634f;

__global__ void __launch_bounds__(kCombineThreads) decode_combine_kernel(DecodeCombineParams c) {
  const int H = c.num_q_heads;
  const int b = blockIdx.x / H;
  const int h = blockIdx.x - b * H;
  const int S = c.splits;
  const float* pl = c.part_lse + (int64_t)b * S * H + h;   // range s at pl[s * H]
  float m = -INFINITY;
  for (int s = 0; s < S; ++s) m = fmaxf(m, pl[(int64_t)s * H]);
  float lse = -INFINITY;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (m != -INFINITY) {
    float den = 0.f;
    for (int s = 0; s < S; ++s) den += exp2f((pl[(int64_t)s * H] - m) * kLog2e);
    lse = m + logf(den);
    const float* po = c.part_out + ((int64_t)b * S * H + h) * 512 + 4 * threadIdx.x;
    for (int s = 0; s < S; ++s) {
      const float ls = pl[(int64_t)s * H];
      if (ls == -INFINITY) continue;
      const float w = exp2f((ls - lse) * kLog2e);
      const f32x4_t o = *reinterpret_cast<const f32x4_t*>(po + (int64_t)s * H * 512);
      acc += w * o;
    }
  }
  st16(c.out + (int64_t)b * c.out_row_stride + (int64_t)h * 512 + 4 * threadIdx.x, acc);
  if (threadIdx.x == 0) c.lse[(int64_t)b * H + h] = lse;
}

}  // namespace

hipError_t launch_decode_mla576_fp8(AttnParams p, const DecodeCombineParams& c,
                                    hipStream_t stream) {
  p.rows_per_team = 1;
  dim3 grid, block;
  attn_grid<2>(p, kRows, &grid, &block);   // one team per (request, range)
  hipLaunchKernelGGL((attn_kernel<576, 512, true, kDecode, 1, 2, true, 2>), grid, block, 0, stream,
                     p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)(c.batch * c.num_q_heads)),
                     dim3(kCombineThreads), 0, stream, c);
  return hipGetLastError();
}

}  // namespace sa
