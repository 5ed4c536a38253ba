// Sparse GQA prefill kernels, head dim 256 (K and V separate, group <= 16):
// per-token, ragged chunk prefill and union instantiations of attn_kernel.
#include "sa_attn_kernel.h"

#ifndef SA_GQA_NBUF
#define SA_GQA_NBUF 1
#endif
#ifndef SA_GQA_WAVES
#define SA_GQA_WAVES 2
#endif

namespace sa {

// One K/V tile in flight per wavefront at two wavefronts per SIMD measured
// faster on the 8192 x 2051 workload than two to four tiles at one wavefront.
constexpr int kGqaNbuf = SA_GQA_NBUF;
constexpr int kGqaWaves = SA_GQA_WAVES;

hipError_t launch_attn_gqa256(const AttnParams& p, int mode, hipStream_t stream) {
  const int64_t waves = mode == kUnion
      ? (int64_t)p.num_groups * p.waves_per_group * p.num_kv_heads
      : (int64_t)((p.num_rows + 3) / 4) * 4 * p.num_kv_heads;
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  switch (mode) {
    case kPerToken:
      hipLaunchKernelGGL((attn_kernel<256, 256, false, kPerToken, kGqaNbuf, kGqaWaves>), grid,
                         block, 0, stream, p);
      break;
    case kRagged:
      hipLaunchKernelGGL((attn_kernel<256, 256, false, kRagged, kGqaNbuf, kGqaWaves>), grid,
                         block, 0, stream, p);
      break;
    default:
      hipLaunchKernelGGL((attn_kernel<256, 256, false, kUnion, kGqaNbuf, kGqaWaves>), grid,
                         block, 0, stream, p);
      break;
  }
  return hipGetLastError();
}

}  // namespace sa
