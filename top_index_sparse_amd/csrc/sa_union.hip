// Union-of-G index sets on the device (sglang PR 32779, "Modifications",
// --dsa-triton-union). For each group of G neighbouring rows the output
// lists every distinct valid index once, under the lowest member row that
// selected it, with one ownership bit per member row that selected it. Two
// builders below produce the same bytes; neither reads anything back to the
// host or keeps state between calls.
//
// Output layout (bit-exact, deterministic): union_idx[g] lists row 0's
// distinct valid indices ascending, then row 1's new ones ascending, ...,
// then -1; union_bits[g][r] has bit j set iff row j of the group selected
// union_idx[g][r]; union_len[g] counts the listed indices.
//
// gfx950 design.
//   Bitmap (when the group's planes fit 64 KB of LDS, G x kv_len <= 2^19):
//   one workgroup per group keeps one bit plane per member over [0, kv_len)
//   in LDS, marks each member's valid indices with atomic ORs, then scans
//   the words in order. A token belongs to the bucket of its lowest owning
//   member; each thread counts its word range per bucket, a block-wide scan
//   turns the counts into output positions, and a second pass over the same
//   words writes every token ascending within its bucket, with the OR of
//   the planes as its bits. That is the output layout below, reached with
//   O(G k + G kv_len / 32) work and no sort.
//   Otherwise, sort and merge:
//   Sort: one wavefront per row holds the row's N = 64R keys in registers
//   (lane l owns keys lR .. lR+R-1). A bitonic network runs its
//   compare-exchanges between registers of one lane when the partner
//   distance is below R and between lanes by shuffles otherwise, so the
//   sort needs no barrier. The coalesced load reaches that blocked layout
//   through a wave-private LDS buffer.
//   Merge: one workgroup per group stages the members' sorted lists in LDS
//   (global memory when they exceed 64 KB); each thread takes 8 consecutive
//   keys of one list, binary-searches the first in every other list and
//   walks forward for the rest. A block-wide scan of the emit flags gives
//   every emitted key its output slot.
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kMergeThreads = 256;
constexpr int kItems = 8;             // consecutive list entries per merge thread
constexpr int32_t kEmpty = 0x7fffffff;
constexpr int kMergeLdsMax = 65536;   // bytes of sorted lists staged in LDS

template <int R>
__global__ void __launch_bounds__(64) union_sort_kernel(UnionBuildParams p) {
  constexpr int N = 64 * R;
  static_assert(R >= 4 && (R & (R - 1)) == 0, "keys per lane");
  __shared__ __attribute__((aligned(16))) int32_t sh[N];
  const int lane = threadIdx.x;
  const int t = blockIdx.x;
  const int32_t* row = p.idx + (int64_t)t * p.idx_row_stride;
  // Invalid indices (outside [0, kv_len)) become kEmpty and sort last.
#pragma unroll 8
  for (int r = 0; r < R; ++r) {
    const int e = r * 64 + lane;
    const int32_t x = e < p.topk ? row[e] : -1;
    sh[e] = (unsigned)x < (unsigned)p.kv_len ? x : kEmpty;
  }
  int32_t key[R];
#pragma unroll
  for (int r = 0; r < R; r += 4) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(sh + lane * R + r);
    key[r] = (int32_t)v[0];
    key[r + 1] = (int32_t)v[1];
    key[r + 2] = (int32_t)v[2];
    key[r + 3] = (int32_t)v[3];
  }
  for (int k = 2; k <= N; k <<= 1) {
    // partner element e ^ j lives in lane ^ (j / R), same register
    for (int j = k >> 1; j >= R; j >>= 1) {
      const int d = j / R;
      const bool lower = (lane & d) == 0;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int32_t o = __shfl_xor(key[r], d);
        const bool asc = ((lane * R + r) & k) == 0;
        key[r] = (asc == lower) ? min(key[r], o) : max(key[r], o);
      }
    }
    // partner in the same lane: registers r and r + j
#pragma unroll
    for (int j = R / 2; j >= 1; j >>= 1) {
      if (j < k) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (r & j) continue;
          const bool asc = ((lane * R + r) & k) == 0;
          const int32_t a = key[r], b = key[r + j];
          const int32_t lo = min(a, b), hi = max(a, b);
          key[r] = asc ? lo : hi;
          key[r + j] = asc ? hi : lo;
        }
      }
    }
  }
  int32_t* out = p.sorted + (int64_t)t * N + lane * R;
#pragma unroll
  for (int r = 0; r < R; r += 4)
    *reinterpret_cast<u32x4_t*>(out + r) =
        (u32x4_t){(uint32_t)key[r], (uint32_t)key[r + 1], (uint32_t)key[r + 2], (uint32_t)key[r + 3]};
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

// One workgroup per group. The group's lists are walked in the output order
// (row-major, ascending within a row).
template <bool LDS>
__global__ void __launch_bounds__(kMergeThreads) union_merge_kernel(UnionBuildParams p) {
  extern __shared__ __attribute__((aligned(16))) int32_t staged[];
  __shared__ int32_t warp_sums[kMergeThreads / 64];
  __shared__ int32_t carry_s;
  const int gi = blockIdx.x;
  const int N = p.topk_pad;
  const int first = gi * p.G;
  int members = p.num_rows - first;
  if (members > p.G) members = p.G;
  const int32_t* src = p.sorted + (int64_t)first * N;
  const int total_items = members * N;
  const int32_t* lists = src;
  if (LDS) {
    for (int i = threadIdx.x * 4; i < total_items; i += kMergeThreads * 4)
      *reinterpret_cast<u32x4_t*>(staged + i) = *reinterpret_cast<const u32x4_t*>(src + i);
    lists = staged;
  }
  const int64_t width = (int64_t)p.G * p.topk;
  int32_t* uidx = p.union_idx + (int64_t)gi * p.union_stride;
  uint8_t* ubits = p.union_bits + (int64_t)gi * p.union_stride;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) carry_s = 0;
  __syncthreads();

  const int chunk = kMergeThreads * kItems;
  for (int base = 0; base < total_items; base += chunk) {
    int32_t xs[kItems];
    uint32_t bits[kItems];
    const int start = base + threadIdx.x * kItems;   // all items in one list (N % 8 == 0)
    const int j = start / N;
    const int k0 = start - j * N;
    const int32_t* s = lists + (int64_t)j * N;
    bool live[kItems];
#pragma unroll
    for (int e = 0; e < kItems; ++e) {
      xs[e] = kEmpty;
      bits[e] = 0;
      live[e] = false;
      if (start + e < total_items) {
        const int32_t x = s[k0 + e];
        live[e] = x != kEmpty && (k0 + e == 0 || s[k0 + e - 1] != x);
        xs[e] = x;
        bits[e] = 1u << j;
      }
    }
    bool earlier[kItems];
#pragma unroll
    for (int e = 0; e < kItems; ++e) earlier[e] = false;
    if (start < total_items) {
      for (int jj = 0; jj < members; ++jj) {
        if (jj == j) continue;
        const int32_t* o = lists + (int64_t)jj * N;
        int at = lower_bound(o, N, xs[0]);
#pragma unroll
        for (int e = 0; e < kItems; ++e) {
          while (at < N && o[at] < xs[e]) ++at;     // keys ascend within the thread
          if (live[e] && at < N && o[at] == xs[e]) {
            bits[e] |= 1u << jj;
            earlier[e] |= jj < j;
          }
        }
      }
    }
    int count = 0;
#pragma unroll
    for (int e = 0; e < kItems; ++e) {
      live[e] = live[e] && !earlier[e];
      count += live[e];
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
      if (live[e]) {
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
  for (int64_t r = len + threadIdx.x; p.fill_tail && r < width; r += kMergeThreads) {
    uidx[r] = -1;
    ubits[r] = 0;
  }
  if (threadIdx.x == 0) p.union_len[gi] = len;
}

constexpr int kBitmapThreads = 256;
constexpr int kMaxMembers = 8;
constexpr int kStagedReqs = 256;   // ragged build: requests whose group starts go to LDS
constexpr int kRaggedPlaneBytes = 16384;

// Block-wide exclusive scan of per-thread counts (thread order), for every
// bucket at once; returns each bucket's total in tot.
template <int M>
__device__ __forceinline__ void scan_buckets(const int cnt[M], int excl[M], int tot[M],
                                             int32_t (*wave_tot)[M]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    int incl = cnt[j];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    excl[j] = incl - cnt[j];
    if (lane == 63) wave_tot[wave][j] = incl;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < M; ++j) {
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kBitmapThreads / 64; ++w) {
      const int t = wave_tot[w][j];
      if (w < wave) before += t;
      total += t;
    }
    excl[j] += before;
    tot[j] = total;
  }
  __syncthreads();   // wave_tot is reused by the next scan
}

// One workgroup per group. The token range [0, kv_len) is covered in chunks
// of 32 * plane_words tokens (one chunk whenever the planes fit); with more
// than one chunk a first pass counts every bucket so that the second can
// place each chunk's tokens after the earlier chunks'.
// M: member capacity (2, 4 or 8, at least G), the size of the per-member
// registers and scans.
template <bool RAGGED, int M>
__global__ void __launch_bounds__(kBitmapThreads) union_bitmap_kernel(UnionBuildParams p) {
  extern __shared__ uint32_t planes[];   // [members][plane_words]
  __shared__ int32_t wave_tot[kBitmapThreads / 64][M];
  const int gi = blockIdx.x;
  const int tid = threadIdx.x;
  int first, members, kv_len;
  if (RAGGED) {
    // the group's request: a binary search of the first group ids, staged
    // in LDS (one round trip instead of one per search step)
    __shared__ int32_t gs[kStagedReqs + 1];
    const int32_t* starts = p.gstart;
    if (p.num_reqs <= kStagedReqs) {
      for (int r = tid; r <= p.num_reqs; r += kBitmapThreads) gs[r] = p.gstart[r];
      __syncthreads();
      starts = gs;
    }
    int64_t kv_base;
    if (!ragged_group(starts, p.cu_q, p.cu_kv, p.num_reqs, p.G, gi, first, members, kv_base,
                      kv_len))
      return;
  } else {
    first = gi * p.G;
    members = p.G;
    kv_len = p.kv_len;
  }
  if (members > p.num_rows - first) members = p.num_rows - first;   // rows that exist
  if (members < 0) members = 0;

  int32_t* uidx = p.union_idx + (int64_t)gi * p.union_stride;
  uint8_t* ubits = p.union_bits + (int64_t)gi * p.union_stride;
  const int cap = 32 * p.plane_words;
  const int nchunks = kv_len > 0 ? (kv_len + cap - 1) / cap : 0;

  // Clears the planes, then marks every member's indices in [c0, c0 + 32 W).
  // A batch reads KB indices of every member before it marks any, so about
  // eight loads per thread are in flight instead of one.
  constexpr int KB = M >= 8 ? 1 : 8 / M;
  auto mark = [&](int c0, int W) {
    for (int i = tid; i < members * W; i += kBitmapThreads) planes[i] = 0u;
    __syncthreads();
    for (int e0 = 0; e0 < p.topk; e0 += KB * kBitmapThreads) {
      int32_t x[M][KB];
#pragma unroll
      for (int j = 0; j < M; ++j) {
        const int32_t* row = p.idx + (int64_t)(first + (j < members ? j : 0)) * p.idx_row_stride;
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          const int e = e0 + tid + u * kBitmapThreads;
          x[j][u] = j < members && e < p.topk ? row[e] : -1;
        }
      }
#pragma unroll
      for (int j = 0; j < M; ++j) {
        uint32_t* plane = planes + j * W;
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          const uint32_t o = (uint32_t)(x[j][u] - c0);
          if ((unsigned)x[j][u] < (unsigned)kv_len && o < (uint32_t)(32 * W))
            atomicOr(&plane[o >> 5], 1u << (o & 31));
        }
      }
    }
    __syncthreads();
  };
  // Wave v owns the contiguous words [wb, we) of a chunk and reads them 64 at
  // a time, lane l taking word wb + 64 r + l in round r: a round's tokens of
  // one bucket then go to consecutive list positions (the bucket of a token
  // is its lowest owning member). count: this lane's tokens per bucket.
  const int lane = tid & 63, wave = tid >> 6;
  auto wave_words = [&](int W, int& wb, int& we) {
    const int per = (W + kBitmapThreads / 64 - 1) / (kBitmapThreads / 64);
    wb = min(W, wave * per);
    we = min(W, wb + per);
  };
  auto count = [&](int W, int cnt[M]) {
#pragma unroll
    for (int j = 0; j < M; ++j) cnt[j] = 0;
    int wb, we;
    wave_words(W, wb, we);
    for (int w = wb + lane; w < we; w += 64) {
      uint32_t seen = 0u;
#pragma unroll
      for (int j = 0; j < M; ++j) {
        if (j < members) {
          const uint32_t b = planes[j * W + w];
          cnt[j] += __popc(b & ~seen);
          seen |= b;
        }
      }
    }
  };
  auto words = [&](int c) { const int left = (kv_len - c * cap + 31) >> 5; return left < p.plane_words ? left : p.plane_words; };

  int total[M];
#pragma unroll
  for (int j = 0; j < M; ++j) total[j] = 0;
  if (nchunks > 1) {
    for (int c = 0; c < nchunks; ++c) {
      const int W = words(c);
      int cnt[M], excl[M], tot[M];
      mark(c * cap, W);
      count(W, cnt);
      scan_buckets<M>(cnt, excl, tot, wave_tot);
#pragma unroll
      for (int j = 0; j < M; ++j) total[j] += tot[j];
    }
  }
  int base[M], carry[M];
  int len = 0;
#pragma unroll
  for (int j = 0; j < M; ++j) carry[j] = 0;
  for (int c = 0; c < nchunks; ++c) {
    const int W = words(c);
    const int c0 = c * cap;
    int cnt[M], excl[M], tot[M];
    mark(c0, W);
    count(W, cnt);
    scan_buckets<M>(cnt, excl, tot, wave_tot);
    if (nchunks == 1) {
#pragma unroll
      for (int j = 0; j < M; ++j) total[j] = tot[j];
    }
    // bucket j starts after every token of buckets < j
    int acc = 0;
#pragma unroll
    for (int j = 0; j < M; ++j) {
      base[j] = acc;
      acc += total[j];
    }
    len = acc;
    // this wave's first position per bucket (lane 0's exclusive prefix: the
    // tokens of the earlier waves), advanced round by round
    int at0[M];
#pragma unroll
    for (int j = 0; j < M; ++j) at0[j] = base[j] + carry[j] + __builtin_amdgcn_readlane(excl[j], 0);
    int wb, we;
    wave_words(W, wb, we);
    for (int r0 = wb; r0 < we; r0 += 64) {
      const int w = r0 + lane;
      uint32_t b[M];
#pragma unroll
      for (int j = 0; j < M; ++j) b[j] = j < members && w < we ? planes[j * W + w] : 0u;
      uint32_t seen = 0u;
#pragma unroll
      for (int j = 0; j < M; ++j) {
        uint32_t fresh = b[j] & ~seen;
        seen |= b[j];
        const uint32_t n = (uint32_t)__popc(fresh);
        const uint32_t incl = wave_scan64(n);
        int at = at0[j] + (int)(incl - n);
        at0[j] += __builtin_amdgcn_readlane((int)incl, 63);
        while (fresh) {
          const int bit = __builtin_ctz(fresh);
          fresh &= fresh - 1u;
          uint32_t own = 0u;
#pragma unroll
          for (int jj = 0; jj < M; ++jj) own |= ((b[jj] >> bit) & 1u) << jj;
          uidx[at] = c0 + w * 32 + bit;
          ubits[at] = (uint8_t)own;
          ++at;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < M; ++j) carry[j] += tot[j];
    __syncthreads();   // the planes are cleared for the next chunk
  }
  const int64_t width = (int64_t)p.G * p.topk;
  for (int64_t r = len + tid; p.fill_tail && r < width; r += kBitmapThreads) {
    uidx[r] = -1;
    ubits[r] = 0;
  }
  if (tid == 0) p.union_len[gi] = len;
}

// gstart[r] = sum over r' < r of ceil(q_r' / G), for r = 0 .. num_reqs
// (one workgroup).
__global__ void __launch_bounds__(kBitmapThreads) union_group_starts_kernel(const int32_t* cu_q,
                                                                            int32_t num_reqs,
                                                                            int32_t G,
                                                                            int32_t* gstart) {
  __shared__ int32_t wave_tot[kBitmapThreads / 64];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base <= num_reqs; base += kBitmapThreads) {
    const int r = base + tid;
    int q = r < num_reqs ? cu_q[r + 1] - cu_q[r] : 0;
    if (q < 0) q = 0;
    const int cnt = (q + G - 1) / G;
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kBitmapThreads / 64; ++w) {
      if (w < wave) before += wave_tot[w];
      total += wave_tot[w];
    }
    if (r <= num_reqs) gstart[r] = carry_s + before + incl - cnt;
    __syncthreads();
    if (tid == 0) carry_s += total;
    __syncthreads();
  }
}

template <int R>
void launch_sort(const UnionBuildParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(union_sort_kernel<R>, dim3((unsigned)p.num_rows), dim3(64), 0, stream, p);
}

}  // namespace

hipError_t launch_union_build(const UnionBuildParams& p, hipStream_t stream) {
  const unsigned groups = (unsigned)((p.num_rows + p.G - 1) / p.G);
  const size_t words = ((size_t)p.kv_len + 31) / 32;
  if (p.G <= kMaxMembers && (size_t)p.G * words * sizeof(uint32_t) <= (size_t)kMergeLdsMax) {
    UnionBuildParams q = p;
    q.plane_words = (int32_t)(words > 0 ? words : 1);   // one chunk
    const size_t lds = (size_t)p.G * q.plane_words * sizeof(uint32_t);
    if (p.G <= 2)
      hipLaunchKernelGGL((union_bitmap_kernel<false, 2>), dim3(groups), dim3(kBitmapThreads), lds,
                         stream, q);
    else if (p.G <= 4)
      hipLaunchKernelGGL((union_bitmap_kernel<false, 4>), dim3(groups), dim3(kBitmapThreads), lds,
                         stream, q);
    else
      hipLaunchKernelGGL((union_bitmap_kernel<false, kMaxMembers>), dim3(groups),
                         dim3(kBitmapThreads), lds, stream, q);
    return hipGetLastError();
  }
  switch (p.topk_pad) {
    case 256: launch_sort<4>(p, stream); break;
    case 512: launch_sort<8>(p, stream); break;
    case 1024: launch_sort<16>(p, stream); break;
    case 2048: launch_sort<32>(p, stream); break;
    case 4096: launch_sort<64>(p, stream); break;
    case 8192: launch_sort<128>(p, stream); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lists = (size_t)p.G * p.topk_pad * sizeof(int32_t);
  if (lists <= (size_t)kMergeLdsMax)
    hipLaunchKernelGGL(union_merge_kernel<true>, dim3(groups), dim3(kMergeThreads), lists, stream, p);
  else
    hipLaunchKernelGGL(union_merge_kernel<false>, dim3(groups), dim3(kMergeThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_union_build_ragged(UnionBuildParams p, int32_t* gstart, hipStream_t stream) {
  hipLaunchKernelGGL(union_group_starts_kernel, dim3(1), dim3(kBitmapThreads), 0, stream, p.cu_q,
                     p.num_reqs, p.G, gstart);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  p.gstart = gstart;
  // 16 KB of planes (65536 tokens per chunk at G = 2): small enough for
  // several workgroups per CU; longer contexts take more chunks
  p.plane_words = (int32_t)(kRaggedPlaneBytes / (int)sizeof(uint32_t) / p.G);
  const size_t lds = (size_t)p.G * p.plane_words * sizeof(uint32_t);
  const dim3 grid((unsigned)p.num_groups), block(kBitmapThreads);
  if (p.G <= 2)
    hipLaunchKernelGGL((union_bitmap_kernel<true, 2>), grid, block, lds, stream, p);
  else if (p.G <= 4)
    hipLaunchKernelGGL((union_bitmap_kernel<true, 4>), grid, block, lds, stream, p);
  else
    hipLaunchKernelGGL((union_bitmap_kernel<true, kMaxMembers>), grid, block, lds, stream, p);
  return hipGetLastError();
}

}  // namespace sa
