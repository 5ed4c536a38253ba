// Sparse MLA prefill kernels: 576-wide latent rows (512 latent + 64 rope)
// whose first 512 columns serve as V, group <= 16 query heads per latent
// row: per-token, ragged and union instantiations of attn_kernel.
#include "sa_attn_kernel.h"

#ifndef SA_MLA_NBUF
#define SA_MLA_NBUF 1
#endif
#ifndef SA_MLA_WAVES
#define SA_MLA_WAVES 2
#endif
#ifndef SA_MLA_WSPLIT
#define SA_MLA_WSPLIT 2
#endif

namespace sa {

constexpr int kMlaNbuf = SA_MLA_NBUF;      // K/V tiles in flight per wavefront
constexpr int kMlaWaves = SA_MLA_WAVES;    // wavefronts per SIMD the registers allow
constexpr int kMlaWsplit = SA_MLA_WSPLIT;  // wavefronts sharing one 16-column tile

hipError_t launch_attn_mla576(const AttnParams& p, int mode, hipStream_t stream) {
  dim3 grid, block;
  attn_grid<kMlaWsplit>(p, mode, &grid, &block);
  switch (mode) {
    case kPerToken:
      hipLaunchKernelGGL((attn_kernel<576, 512, true, kPerToken, kMlaNbuf, kMlaWsplit, kMlaWaves>),
                         grid, block, 0, stream, p);
      break;
    case kRagged:
      hipLaunchKernelGGL((attn_kernel<576, 512, true, kRagged, kMlaNbuf, kMlaWsplit, kMlaWaves>),
                         grid, block, 0, stream, p);
      break;
    case kPaired:
      hipLaunchKernelGGL((attn_kernel<576, 512, true, kPaired, 1, kMlaWsplit, kMlaWaves>),
                         grid, block, 0, stream, p);
      break;
    case kPairedRagged:
      hipLaunchKernelGGL((attn_kernel<576, 512, true, kPairedRagged, 1, kMlaWsplit, kMlaWaves>),
                         grid, block, 0, stream, p);
      break;
    default:
      hipLaunchKernelGGL((attn_kernel<576, 512, true, kUnion, kMlaNbuf, kMlaWsplit, kMlaWaves>),
                         grid, block, 0, stream, p);
      break;
  }
  return hipGetLastError();
}

}  // namespace sa
