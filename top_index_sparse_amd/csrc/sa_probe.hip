// Measurement aid (no part of the attention path): the K/V row gathers of
// the head-dim-256 per-token kernels without their arithmetic, to measure
// what the gather stream alone sustains. A wavefront walks one index row in
// tiles of 16 slots; lane (g, m) reads 16 bytes at offset 256 h + 16 m of
// the K and V rows of slots 4g .. 4g+3 (h = 0, 1), through the same row
// buffer descriptors (absent rows read zeros), and folds them into a
// checksum so nothing is dropped.
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kRowBytes = 512;   // 256 bf16

// LDS: 64 KB per four-wave workgroup caps a CU at eight waves (the attention
// kernels' occupancy); without it registers alone decide.
template <bool LDS8>
__global__ void __launch_bounds__(256) gather_probe_kernel(GatherProbeParams p) {
  __shared__ uint32_t pad[LDS8 ? 16384 : 1];
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, m = lane & 15;
  const int row = bid * 4 + wv;
  if (row >= p.num_rows) return;
  const rows_rsrc_t rk = rows_rsrc(p.k, kRowBytes), rv = rows_rsrc(p.v, kRowBytes);
  const int32_t* ir = p.idx + (int64_t)row * p.topk;
  // Indices are loaded a tile ahead, clamped to the row, and checked only
  // where they are used (a check at the load would wait for it at once).
  auto ld_index = [&](int j) { return ir[j < p.topk ? j : p.topk - 1]; };
  u32x4_t acc = {0u, 0u, 0u, 0u};
  int tn[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) tn[i] = ld_index(4 * g + i);
  for (int j0 = 0; j0 < p.topk; j0 += 16) {
    int tok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + 4 * g + i;
      tok[i] = (j < p.topk && (unsigned)tn[i] < (unsigned)p.kv_len) ? tn[i] : kNoRow;
      tn[i] = ld_index(j + 16);
    }
    u32x4_t kd[8], vd[8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        kd[2 * i + h] = ld_row16(rk, tok[i], 256 * h + 16 * m);
        vd[2 * i + h] = ld_row16(rv, tok[i], 256 * h + 16 * m);
      }
#pragma unroll
    for (int q = 0; q < 8; ++q) acc ^= kd[q] ^ vd[q];
  }
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (LDS8 && p.topk < 0) {   // never: keeps the allocation
    pad[threadIdx.x] = x;
    __syncthreads();
    x = pad[threadIdx.x ^ 1];
  }
  p.out[(int64_t)row * 64 + lane] = x;
}

}  // namespace

hipError_t launch_gather_probe(const GatherProbeParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((p.num_rows + 3) / 4)), block(256);
  if (p.eight_waves)
    hipLaunchKernelGGL(gather_probe_kernel<true>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(gather_probe_kernel<false>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa
