// Sparse MLA prefill kernels: 576-wide latent rows (512 latent + 64 rope)
// whose first 512 columns serve as V, up to 32 query heads per latent row:
// per-token (one request or ragged requests) and union instantiations of
// attn_kernel. A team is one 16-column tile on two wavefronts (each half of
// the latent columns), which keeps a wave's registers within budget.
#include "sa_attn_kernel.h"

namespace sa {

namespace {

template <bool FP8>
hipError_t launch_slice(AttnParams p, int union_mode, hipStream_t stream) {
  dim3 grid, block;
  const int r = 16 / p.group;   // rows of one 16-column tile
  if (union_mode) {
    p.rows_per_team = r < p.G ? r : p.G;
    p.teams_per_group = (p.G + p.rows_per_team - 1) / p.rows_per_team;
    if (!attn_grid<2>(p, kUnion, &grid, &block)) return hipErrorInvalidConfiguration;
    // FP8 union teams fit three waves per SIMD (168 VGPRs; 8 spilled, saved
    // before the tile loop and reloaded after it), which hides more of their
    // per-tile latency (C3 FP8 union G=2 0.48 -> 0.42 ms); the bf16 union and
    // per-token teams lose more to spills there
    hipLaunchKernelGGL((attn_kernel<576, 512, true, kUnion, 1, 2, FP8, FP8 ? 3 : 2>), grid, block, 0,
                       stream, p);
  } else {
    p.rows_per_team = r < 4 ? r : 4;
    if (!attn_grid<2>(p, kRows, &grid, &block)) return hipErrorInvalidConfiguration;
    // two-row teams (5-8 heads) match their rows by membership
    if (p.rows_per_team == 2)
      hipLaunchKernelGGL((attn_kernel<576, 512, true, kRowsMember, 1, 2, FP8, 2>), grid, block, 0,
                         stream, p);
    else
      hipLaunchKernelGGL((attn_kernel<576, 512, true, kRows, 1, 2, FP8, 2>), grid, block, 0, stream,
                         p);
  }
  return hipGetLastError();
}

// A row of more than 16 heads (one latent KV head) runs as slices of at most
// 16 heads, each a launch of its own over the q, out and lse columns of its
// heads; each slice gathers the rows again.
template <bool FP8>
hipError_t launch(const AttnParams& p, int union_mode, hipStream_t stream) {
  if (p.group <= 16) return launch_slice<FP8>(p, union_mode, stream);
  for (int h0 = 0; h0 < p.group; h0 += 16) {
    AttnParams ps = p;
    ps.group = ps.num_q_heads = p.group - h0 < 16 ? p.group - h0 : 16;
    ps.q = p.q + (int64_t)h0 * 576;
    ps.out = p.out + (int64_t)h0 * 512;
    ps.lse = p.lse + h0;
    const hipError_t e = launch_slice<FP8>(ps, union_mode, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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
