// Sparse MLA prefill kernels: 576-wide latent rows (512 latent + 64 rope)
// whose first 512 columns serve as V, group <= 16 query heads per latent
// row: per-token, ragged and union instantiations of attn_kernel.
#include "sa_attn_kernel.h"

#ifndef SA_MLA_NBUF
#define SA_MLA_NBUF 1
#endif
#ifndef SA_MLA_WAVES
#define SA_MLA_WAVES 1
#endif

namespace sa {

constexpr int kMlaNbuf = SA_MLA_NBUF;
constexpr int kMlaWaves = SA_MLA_WAVES;

hipError_t launch_attn_mla576(const AttnParams& p, int mode, hipStream_t stream) {
  const int64_t waves = mode == kUnion
      ? (int64_t)p.num_groups * p.waves_per_group * p.num_kv_heads
      : (int64_t)((p.num_rows + 3) / 4) * 4 * p.num_kv_heads;
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  switch (mode) {
    case kPerToken:
      hipLaunchKernelGGL((attn_kernel<576, 512, true, kPerToken, kMlaNbuf, kMlaWaves>), grid,
                         block, 0, stream, p);
      break;
    case kRagged:
      hipLaunchKernelGGL((attn_kernel<576, 512, true, kRagged, kMlaNbuf, kMlaWaves>), grid,
                         block, 0, stream, p);
      break;
    default:
      hipLaunchKernelGGL((attn_kernel<576, 512, true, kUnion, kMlaNbuf, kMlaWaves>), grid,
                         block, 0, stream, p);
      break;
  }
  return hipGetLastError();
}

}  // namespace sa
