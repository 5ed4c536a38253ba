// Sparse GQA prefill kernels, head dim 256 (K and V separate, group <= 16):
// per-token, ragged chunk prefill and union instantiations of attn_kernel.
#include "sa_attn_kernel.h"

#ifndef SA_GQA_NBUF
#define SA_GQA_NBUF 1
#endif
#ifndef SA_GQA_WAVES
#define SA_GQA_WAVES 2
#endif
#ifndef SA_GQA_WSPLIT
#define SA_GQA_WSPLIT 1
#endif

namespace sa {

constexpr int kGqaNbuf = SA_GQA_NBUF;      // K/V tiles in flight per wavefront
constexpr int kGqaWaves = SA_GQA_WAVES;    // wavefronts per SIMD the registers allow
constexpr int kGqaWsplit = SA_GQA_WSPLIT;  // wavefronts sharing one 16-column tile

hipError_t launch_attn_gqa256(const AttnParams& p, int mode, hipStream_t stream) {
  dim3 grid, block;
  attn_grid<kGqaWsplit>(p, mode, &grid, &block);
  switch (mode) {
    case kPerToken:
      hipLaunchKernelGGL((attn_kernel<256, 256, false, kPerToken, kGqaNbuf, kGqaWsplit, kGqaWaves>),
                         grid, block, 0, stream, p);
      break;
    case kRagged:
      hipLaunchKernelGGL((attn_kernel<256, 256, false, kRagged, kGqaNbuf, kGqaWsplit, kGqaWaves>),
                         grid, block, 0, stream, p);
      break;
    case kPaired:
      hipLaunchKernelGGL((attn_kernel<256, 256, false, kPaired, 1, kGqaWsplit, kGqaWaves>),
                         grid, block, 0, stream, p);
      break;
    case kPairedRagged:
      hipLaunchKernelGGL((attn_kernel<256, 256, false, kPairedRagged, 1, kGqaWsplit, kGqaWaves>),
                         grid, block, 0, stream, p);
      break;
    default:
      hipLaunchKernelGGL((attn_kernel<256, 256, false, kUnion, kGqaNbuf, kGqaWsplit, kGqaWaves>),
                         grid, block, 0, stream, p);
      break;
  }
  return hipGetLastError();
}

}  // namespace sa
