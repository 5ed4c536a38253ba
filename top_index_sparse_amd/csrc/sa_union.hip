// Union-of-G index sets on the device (sglang PR 32779, "Modifications",
// --dsa-triton-union): each row's selected indices are sorted on their own,
// then one workgroup per group of G adjacent rows runs a lower_bound of every
// index against the other rows' sorted lists. A row emits an index iff no
// earlier row of the group selected it, and every row that selected it sets
// its ownership bit. Nothing is read back to the host and nothing outlives
// the call.
//
// Output layout (bit-exact, deterministic): union_idx[g] lists row 0's
// distinct valid indices ascending, then row 1's new ones ascending, ...,
// then -1; union_bits[g][r] has bit j set iff row j of the group selected
// union_idx[g][r]; union_len[g] counts the listed indices.
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kSortThreads = 256;
constexpr int kMergeThreads = 256;
constexpr int kItems = 8;           // consecutive list entries per merge thread
constexpr int32_t kEmpty = 0x7fffffff;

// Sort kernel: one workgroup per row; bitonic sort of topk_pad keys in LDS.
// Invalid indices (outside [0, kv_len)) become kEmpty and sort last.
__global__ void __launch_bounds__(kSortThreads) union_sort_kernel(UnionBuildParams p) {
  extern __shared__ int32_t keys[];
  const int t = blockIdx.x;
  const int N = p.topk_pad;
  const int32_t* row = p.idx + (int64_t)t * p.idx_row_stride;
  for (int i = threadIdx.x; i < N; i += kSortThreads) {
    const int32_t x = i < p.topk ? row[i] : -1;
    keys[i] = (unsigned)x < (unsigned)p.kv_len ? x : kEmpty;
  }
  __syncthreads();
  for (int k = 2; k <= N; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < (N >> 1); i += kSortThreads) {
        // i-th compare-exchange pair of this stage: lo has bit j clear
        const int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1));
        const int hi = lo | j;
        const bool ascending = (lo & k) == 0;
        const int32_t a = keys[lo], b = keys[hi];
        if ((a > b) == ascending) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  int32_t* out = p.sorted + (int64_t)t * N;
  for (int i = threadIdx.x; i < N; i += kSortThreads) out[i] = keys[i];
}

// First position in the sorted list s[0..n) whose key is >= x.
__device__ __forceinline__ int lower_bound(const int32_t* s, int n, int32_t x) {
  int lo = 0;
  while (n > 0) {
    const int half = n >> 1;
    if (s[lo + half] < x) {
      lo += half + 1;
      n -= half + 1;
    } else {
      n = half;
    }
  }
  return lo;
}

// Merge kernel: one workgroup per group. The group's lists are walked in
// the output order (row-major, ascending within a row); a block-wide scan
// of the emit flags gives every emitted index its output slot.
__global__ void __launch_bounds__(kMergeThreads) union_merge_kernel(UnionBuildParams p) {
  __shared__ int32_t warp_sums[kMergeThreads / 64];
  __shared__ int32_t carry_s;
  const int gi = blockIdx.x;
  const int N = p.topk_pad;
  const int first = gi * p.G;
  int members = p.num_rows - first;
  if (members > p.G) members = p.G;
  const int32_t* lists = p.sorted + (int64_t)first * N;
  const int64_t width = (int64_t)p.G * p.topk;
  int32_t* uidx = p.union_idx + (int64_t)gi * p.union_stride;
  uint8_t* ubits = p.union_bits + (int64_t)gi * p.union_stride;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) carry_s = 0;
  __syncthreads();

  const int total_items = members * N;
  const int chunk = kMergeThreads * kItems;
  for (int base = 0; base < total_items; base += chunk) {
    int32_t xs[kItems];
    uint32_t bits[kItems];
    int count = 0;
    const int start = base + threadIdx.x * kItems;
#pragma unroll
    for (int e = 0; e < kItems; ++e) {
      const int pos = start + e;
      xs[e] = kEmpty;
      bits[e] = 0;
      if (pos < total_items) {
        const int j = pos / N, k = pos - j * N;
        const int32_t* s = lists + (int64_t)j * N;
        const int32_t x = s[k];
        const bool live = x != kEmpty && (k == 0 || s[k - 1] != x);
        if (live) {
          uint32_t b = 1u << j;
          bool earlier = false;
          for (int jj = 0; jj < members; ++jj) {
            if (jj == j) continue;
            const int32_t* o = lists + (int64_t)jj * N;
            const int at = lower_bound(o, N, x);
            if (at < N && o[at] == x) {
              b |= 1u << jj;
              earlier |= jj < j;
            }
          }
          if (!earlier) {
            xs[e] = x;
            bits[e] = b;
            ++count;
          }
        }
      }
    }
    // block-wide exclusive scan of the per-thread counts
    int incl = count;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    if (lane == 63) warp_sums[wave] = incl;
    __syncthreads();
    int wave_base = 0, chunk_total = 0;
#pragma unroll
    for (int w = 0; w < kMergeThreads / 64; ++w) {
      if (w < wave) wave_base += warp_sums[w];
      chunk_total += warp_sums[w];
    }
    int out = carry_s + wave_base + incl - count;
#pragma unroll
    for (int e = 0; e < kItems; ++e) {
      if (bits[e]) {
        uidx[out] = xs[e];
        ubits[out] = (uint8_t)bits[e];
        ++out;
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) carry_s += chunk_total;
    __syncthreads();
  }
  const int len = carry_s;
  for (int64_t r = len + threadIdx.x; r < width; r += kMergeThreads) {
    uidx[r] = -1;
    ubits[r] = 0;
  }
  if (threadIdx.x == 0) p.union_len[gi] = len;
}

}  // namespace

hipError_t launch_union_build(const UnionBuildParams& p, hipStream_t stream) {
  const size_t lds = (size_t)p.topk_pad * sizeof(int32_t);
  hipLaunchKernelGGL(union_sort_kernel, dim3((unsigned)p.num_rows), dim3(kSortThreads), lds,
                     stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned groups = (unsigned)((p.num_rows + p.G - 1) / p.G);
  hipLaunchKernelGGL(union_merge_kernel, dim3(groups), dim3(kMergeThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa
