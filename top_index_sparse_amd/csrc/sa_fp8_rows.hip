// FP8 MLA records to bf16 rows (sglang PR 32779, "Accuracy Tests" (c): the
// kernel measured there reads rows dequantised to bf16 before it runs). A
// step that gathers each pool record many times (every query row of a
// prefill chunk selects most of its neighbours' tokens) can convert each
// touched record once and run the bf16 kernels over the converted rows,
// instead of dequantising a record in every team that gathers it.
//
// One wavefront per (token, KV head): lane l converts latent values
// 8l .. 8l+7 (block l / 16) with the same instructions the attention
// kernels use while staging (fp32 convert, fp32 multiply by the block
// scale, nearest-even bf16 pack), so both paths see identical bf16 values;
// lanes 0-7 copy the 128 rope bytes.
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kWaves = 4;   // rows per workgroup

__global__ void __launch_bounds__(64 * kWaves) fp8_rows_kernel(Fp8RowsParams p) {
  const int64_t r = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (r >= p.rows) return;
  const int64_t t = r / p.num_kv_heads;
  const int h = (int)(r - t * p.num_kv_heads);
  if (p.mask && p.mask[t] == 0) return;
  const int lane = threadIdx.x & 63;
  const uint8_t* rec = p.pool + t * p.pool_row_stride + (int64_t)h * 656;
  uint16_t* row = p.out + t * p.out_row_stride + (int64_t)h * 576;
  const u32x2_t codes = *reinterpret_cast<const u32x2_t*>(rec + 8 * lane);
  const float sc = *reinterpret_cast<const float*>(rec + 512 + 4 * (lane >> 4));
  const uint32_t c0 = codes[0], c1 = codes[1];
  const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)c0, false);
  const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)c0, true);
  const f32x2_t c = __builtin_amdgcn_cvt_pk_f32_fp8((int)c1, false);
  const f32x2_t d = __builtin_amdgcn_cvt_pk_f32_fp8((int)c1, true);
  const u32x4_t v = {pack_bf16x2(a[0] * sc, a[1] * sc), pack_bf16x2(b[0] * sc, b[1] * sc),
                     pack_bf16x2(c[0] * sc, c[1] * sc), pack_bf16x2(d[0] * sc, d[1] * sc)};
  *reinterpret_cast<u32x4_t*>(row + 8 * lane) = v;
  if (lane < 8)
    *reinterpret_cast<u32x4_t*>(row + 512 + 8 * lane) =
        *reinterpret_cast<const u32x4_t*>(rec + 528 + 16 * lane);
}

}  // namespace

hipError_t launch_fp8_records_to_bf16(const Fp8RowsParams& p, hipStream_t stream) {
  const int64_t blocks = (p.rows + kWaves - 1) / kWaves;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fp8_rows_kernel, dim3((unsigned)blocks), dim3(64 * kWaves), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa
