// Sparse MLA prefill kernels: 576-wide latent rows (512 latent + 64 rope)
// whose first 512 columns serve as V, group <= 16 query heads per latent
// row: per-token (one request or ragged requests) and union instantiations
// of attn_kernel. A team is one 16-column tile on two wavefronts (each half
// of the latent columns), which keeps a wave's registers within budget.
#include "sa_attn_kernel.h"

namespace sa {

namespace {

template <bool FP8>
hipError_t launch(AttnParams p, int union_mode, hipStream_t stream) {
  dim3 grid, block;
  const int r = 16 / p.group;   // rows of one 16-column tile
  if (union_mode) {
    p.rows_per_team = r < p.G ? r : p.G;
    p.teams_per_group = (p.G + p.rows_per_team - 1) / p.rows_per_team;
    if (!attn_grid<2>(p, kUnion, &grid, &block)) return hipErrorInvalidConfiguration;
    // FP8 union teams fit three waves per SIMD (168 VGPRs, 2 spilled), which
    // hides more of their per-tile latency (C3 FP8 union G=2 0.56 -> 0.49
    // ms); the bf16 union and per-token teams lose more to spills there
    hipLaunchKernelGGL((attn_kernel<576, 512, true, kUnion, 1, 2, FP8, FP8 ? 3 : 2>), grid, block, 0,
                       stream, p);
  } else {
    p.rows_per_team = r < 4 ? r : 4;
    if (!attn_grid<2>(p, kRows, &grid, &block)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_kernel<576, 512, true, kRows, 1, 2, FP8, 2>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_mla576(AttnParams p, int union_mode, hipStream_t stream) {
  return launch<false>(p, union_mode, stream);
}

// K rows as 656-byte FP8 records, dequantised while they are staged.
hipError_t launch_attn_mla576_fp8(AttnParams p, int union_mode, hipStream_t stream) {
  return launch<true>(p, union_mode, stream);
}

}  // namespace sa
