// Decode-pool page mark and masked page split (sglang PR 32320,
// "Modifications"): the pool keeps pages of src_page_tokens tokens; the
// decode kernel reads pages of dst_page_tokens. The mark pass flags every
// source page that a valid token index of the step falls in; the split pass
// runs a fixed grid of one workgroup per destination page and returns at once
// when its source page is unflagged: untouched pages cost one flag read, and
// the launch shape never depends on the data (no host read, graph safe).
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kThreads = 256;

// Clears the mask (a fill kernel rather than a memset node, so that a
// captured graph replays it like any other kernel).
__global__ void __launch_bounds__(kThreads) page_clear_kernel(int8_t* mask, int32_t n) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) mask[i] = 0;
}

// Sixteen indices per thread (four 16-byte loads in flight where the array
// is 16-byte aligned): same-value stores of 1, no atomics needed. A store is skipped
// when the byte already reads 1, so that many indices into few pages (a
// prefill step's rows over one-token pages) do not all write the same lines.
// page_shift >= 0: src_page_tokens is 1 << page_shift.
constexpr int kMarkPerThread = 16;

__global__ void __launch_bounds__(kThreads) page_mark_kernel(const int32_t* idx, int64_t num_idx,
                                                             int64_t pool_tokens,
                                                             int32_t src_page_tokens,
                                                             int32_t page_shift, bool vec16,
                                                             int8_t* mask) {
  const int64_t i0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kMarkPerThread;
  if (i0 >= num_idx) return;
  int32_t t[kMarkPerThread];
  if (vec16 && i0 + kMarkPerThread <= num_idx) {
    u32x4_t v[kMarkPerThread / 4];
#pragma unroll
    for (int q = 0; q < kMarkPerThread / 4; ++q) v[q] = ld16(idx + i0 + 4 * q);
#pragma unroll
    for (int j = 0; j < kMarkPerThread; ++j) t[j] = (int32_t)v[j / 4][j % 4];
  } else {
#pragma unroll
    for (int j = 0; j < kMarkPerThread; ++j) t[j] = i0 + j < num_idx ? idx[i0 + j] : -1;
  }
#pragma unroll
  for (int j = 0; j < kMarkPerThread; ++j) {
    if (t[j] >= 0 && (int64_t)t[j] < pool_tokens) {
      int8_t* m = mask + (page_shift >= 0 ? t[j] >> page_shift : t[j] / src_page_tokens);
      if (*m == 0) *m = 1;
    }
  }
}

// Copies n bytes; sixteen 16-byte loads per thread are issued before their
// stores, so a 64-row destination page (10.25 chunks per thread) costs one
// memory round trip.
// Both sides are streamed (non-temporal): the pool pages are read once and
// the destination is not read back by this kernel.
template <bool VEC16>
__device__ __forceinline__ void copy_bytes(uint8_t* __restrict__ dst, const uint8_t* __restrict__ src,
                                           int64_t n) {
  if (VEC16) {
    constexpr int U = 16;
    const int64_t nv = n >> 4;
    const u32x4_t* s = reinterpret_cast<const u32x4_t*>(src);
    u32x4_t* d = reinterpret_cast<u32x4_t*>(dst);
    for (int64_t i = threadIdx.x; i < nv; i += U * kThreads) {
      u32x4_t v[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i + u * kThreads < nv) v[u] = __builtin_nontemporal_load(&s[i + u * kThreads]);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i + u * kThreads < nv) __builtin_nontemporal_store(v[u], &d[i + u * kThreads]);
    }
  } else {
    for (int64_t i = threadIdx.x; i < n; i += kThreads) dst[i] = src[i];
  }
}

// Workgroup (p, s) writes destination page p*ratio + s.
template <bool VEC16>
__global__ void __launch_bounds__(kThreads) page_split_kernel(PageParams p) {
  const int ratio = p.src_page_tokens / p.dst_page_tokens;
  const int page = blockIdx.x / ratio;
  const int sub = blockIdx.x - page * ratio;
  if (p.mask && p.mask[page] == 0) return;
  const uint8_t* src = p.src + (int64_t)page * p.src_page_stride;
  uint8_t* dst = p.dst + (int64_t)blockIdx.x * p.dst_page_stride;
  const int64_t rows = (int64_t)p.dst_page_tokens * p.row_bytes;
  const int64_t scales = (int64_t)p.dst_page_tokens * p.scale_bytes;
  copy_bytes<VEC16>(dst, src + sub * rows, rows);
  copy_bytes<VEC16>(dst + rows,
                    src + (int64_t)p.src_page_tokens * p.row_bytes + sub * scales, scales);
}

}  // namespace

hipError_t launch_page_mark(const int32_t* idx, int64_t num_idx, int32_t num_src_pages,
                            int32_t src_page_tokens, int8_t* mask, hipStream_t stream) {
  hipLaunchKernelGGL(page_clear_kernel, dim3((unsigned)((num_src_pages + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, mask, num_src_pages);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || num_idx == 0) return e;
  const int32_t shift = (src_page_tokens & (src_page_tokens - 1)) == 0
                            ? __builtin_ctz((uint32_t)src_page_tokens) : -1;
  const bool vec16 = (reinterpret_cast<uintptr_t>(idx) & 15) == 0;
  const int64_t per_block = (int64_t)kThreads * kMarkPerThread;
  hipLaunchKernelGGL(page_mark_kernel, dim3((unsigned)((num_idx + per_block - 1) / per_block)),
                     dim3(kThreads), 0, stream, idx, num_idx,
                     (int64_t)num_src_pages * src_page_tokens, src_page_tokens, shift, vec16,
                     mask);
  return hipGetLastError();
}

hipError_t launch_page_split(const PageParams& p, hipStream_t stream) {
  const int ratio = p.src_page_tokens / p.dst_page_tokens;
  const dim3 grid((unsigned)((int64_t)p.num_src_pages * ratio)), block(kThreads);
  const int64_t rows = (int64_t)p.dst_page_tokens * p.row_bytes;
  const int64_t scales = (int64_t)p.dst_page_tokens * p.scale_bytes;
  const int64_t scale0 = (int64_t)p.src_page_tokens * p.row_bytes;
  const bool vec = ((reinterpret_cast<uintptr_t>(p.src) | reinterpret_cast<uintptr_t>(p.dst)) & 15) == 0 &&
                   ((p.src_page_stride | p.dst_page_stride | rows | scales | scale0) & 15) == 0;
  if (vec)
    hipLaunchKernelGGL(page_split_kernel<true>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(page_split_kernel<false>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa
