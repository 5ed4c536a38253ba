// Sparse GQA prefill kernels, head dim 256 (K and V separate, group <= 32):
// per-token (one request or ragged requests) and union instantiations of
// attn_kernel, for three team shapes.
#include "sa_attn_kernel.h"

namespace sa {

namespace {

// Waves per SIMD: two everywhere (the register budget of the products),
// except the two-tile union team, which fits three (168 VGPRs, no spills);
// the third wave hides more of its per-tile latency (C2 union G=2 1.76 ->
// 1.45 ms), where the per-token shapes lose more to spills than they gain.
template <int MODE, int C, int WSPLIT>
hipError_t launch(const AttnParams& p, hipStream_t stream) {
  constexpr int kWaves = MODE == kUnion && C == 2 ? 3 : 2;
  dim3 grid, block;
  if (!attn_grid<WSPLIT>(p, MODE, &grid, &block)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_kernel<256, 256, false, MODE, C, WSPLIT, false, kWaves>), grid, block, 0,
                     stream, p);
  return hipGetLastError();
}

// One wave with whole K/V rows for 16 columns; two waves, each with half of
// d, for 32 or 48 columns (union teams have at most 32).
template <int MODE>
hipError_t launch_cols(const AttnParams& p, int cols, hipStream_t stream) {
  if (cols <= 16) return launch<MODE, 1, 1>(p, stream);
  if (MODE == kUnion || cols <= 32) return launch<MODE, 2, 2>(p, stream);
  return launch<kRows, 3, 2>(p, stream);
}

}  // namespace

// Team shapes. Per-token: a team serves the consecutive rows that share its
// gathered slot positions: 16 / group rows on one wave for group <= 8 (the
// wave's 16 columns), up to four rows on two waves with three 16-column
// tiles above that. Union: one team per group (G x group <= 32 columns by
// the host).
hipError_t launch_attn_gqa256(AttnParams p, int union_mode, hipStream_t stream) {
  if (union_mode) {
    p.rows_per_team = p.G;
    p.teams_per_group = 1;
    return launch_cols<kUnion>(p, p.G * p.group, stream);
  }
  const int r = p.group <= 8 ? 16 / p.group : 48 / p.group;
  p.rows_per_team = r < 4 ? r : 4;
  // two-row one-wave teams (group 5-8) match their rows by membership
  if (p.rows_per_team == 2 && p.group <= 8) return launch<kRowsMember, 1, 1>(p, stream);
  return launch_cols<kRows>(p, p.rows_per_team * p.group, stream);
}

}  // namespace sa
