// Internal interface between the C ABI (sa_api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sparse_attn.h"

namespace sa {

// One attention launch. Pointers are device pointers; strides in elements.
struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;          // == k when V lives in the K row
  const int32_t* idx;
  const int32_t* topk_len;    // nullable
  const int32_t* cu_q;        // ragged only
  const int64_t* cu_kv;       // ragged only
  float* out;
  float* lse;
  int64_t q_row_stride;
  int64_t k_row_stride;
  int64_t v_row_stride;
  int64_t idx_row_stride;
  int64_t out_row_stride;
  int64_t lse_row_stride;     // lse[t * lse_row_stride + head]
  int32_t num_rows;
  int32_t num_reqs;
  int32_t kv_len;             // non-ragged KV length
  int32_t topk;
  int32_t group;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  float scale_log2e;          // sm_scale * log2(e)
  // union mode: prebuilt union sets of G adjacent rows
  const int32_t* union_idx;   // [num_groups][union_stride]
  const uint8_t* union_bits;  // [num_groups][union_stride]
  const int32_t* union_len;   // [num_groups]
  int64_t union_stride;
  int32_t G;
  int32_t num_groups;
  const int32_t* gstart;      // union over ragged requests: first group id per request
  int32_t teams_per_group;    // union: teams serving one group
  // rows one team serves (per-token: consecutive rows; union: group members)
  int32_t rows_per_team;
  // decode over pages: virtual row b * dec_splits + s covers slot tiles
  // s, s + dec_splits, ... of request b; token t is the record at byte
  // (t >> page_shift) * page_stride + (t & mask) * 656
  int32_t dec_splits;
  int32_t page_shift;
  int64_t page_stride;
};

// Merge of the per-range decode results: out[b, h] and lse[b, h] from
// part_out[b * splits + s, h] and part_lse[b * splits + s, h].
struct DecodeCombineParams {
  const float* part_out;      // [batch * splits][num_q_heads][512], normalised
  const float* part_lse;      // [batch * splits][num_q_heads], natural log
  float* out;
  float* lse;
  int64_t out_row_stride;
  int32_t batch;
  int32_t splits;
  int32_t num_q_heads;
};

struct UnionBuildParams {
  const int32_t* idx;
  int64_t idx_row_stride;
  int32_t num_rows;
  int32_t topk;
  int32_t kv_len;
  int32_t G;
  int32_t* sorted;            // workspace [num_rows][topk_pad]
  int32_t topk_pad;           // power of two >= topk
  int32_t* union_idx;         // [groups][union_stride], first G*topk used
  uint8_t* union_bits;        // [groups][union_stride]
  int32_t* union_len;         // [groups]
  int64_t union_stride;
  // ragged groups (chunk prefill): G rows inside each request, request-local
  // indices; group ids [gstart[r], gstart[r+1]) belong to request r
  const int32_t* gstart;      // nullable: one request of kv_len
  const int32_t* cu_q;
  const int64_t* cu_kv;
  int32_t num_reqs;
  int32_t num_groups;         // groups launched (an upper bound when ragged)
  int32_t plane_words;        // 32-token words per member per bit-plane chunk
  int32_t fill_tail;          // write -1 / 0 after union_len up to G * topk
};

// Ragged union groups: ids [gstart[r], gstart[r+1]) belong to request r,
// each covering G consecutive rows of it (the last may be short). False for
// ids past the last group.
__device__ __forceinline__ bool ragged_group(const int32_t* gstart, const int32_t* cu_q,
                                             const int64_t* cu_kv, int num_reqs, int G, int gi,
                                             int& first, int& members, int64_t& kv_base,
                                             int& kv_len) {
  if (gi >= gstart[num_reqs]) return false;
  int lo = 0, hi = num_reqs - 1;   // last request whose first group id is <= gi
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (gstart[mid] <= gi) lo = mid; else hi = mid - 1;
  }
  first = cu_q[lo] + (gi - gstart[lo]) * G;
  const int end = cu_q[lo + 1];
  members = end - first < G ? end - first : G;
  kv_base = cu_kv[lo];
  kv_len = (int)(cu_kv[lo + 1] - cu_kv[lo]);
  return true;
}

struct PageParams {
  const uint8_t* src;
  uint8_t* dst;
  const int8_t* mask;         // nullable
  int64_t src_page_stride;
  int64_t dst_page_stride;
  int32_t num_src_pages;
  int32_t src_page_tokens;
  int32_t dst_page_tokens;
  int32_t row_bytes;
  int32_t scale_bytes;
};

// Indexer top-k: row t keeps the k largest of its first n_t scores
// (n_t = row_len[t] clamped to [0, kv_len], or kv_len), ascending positions.
struct TopkParams {
  const float* scores;        // [num_rows][score_row_stride]
  int64_t score_row_stride;   // floats
  const int32_t* row_len;     // nullable
  int32_t num_rows;
  int32_t kv_len;
  int32_t k;
  int32_t* idx;               // [num_rows][idx_row_stride]
  int64_t idx_row_stride;
};

// union: 0 per-token results (ragged when cu_q is set), 1 union lists. The
// launchers choose the team shape (rows per team, column tiles).
hipError_t launch_attn_gqa256(AttnParams p, int union_mode, hipStream_t stream);
hipError_t launch_attn_mla576(AttnParams p, int union_mode, hipStream_t stream);
hipError_t launch_attn_mla576_fp8(AttnParams p, int union_mode, hipStream_t stream);
// Decode over 64-token pages of FP8 records: the per-range team kernel
// (p.out / p.lse point at the partials), then the combine.
hipError_t launch_decode_mla576_fp8(AttnParams p, const DecodeCombineParams& c,
                                    hipStream_t stream);
hipError_t launch_union_build(const UnionBuildParams& p, hipStream_t stream);
// Ragged: writes gstart[0..num_reqs] from cu_q, then builds every group's
// union over its request's KV range with bit planes.
hipError_t launch_union_build_ragged(UnionBuildParams p, int32_t* gstart, hipStream_t stream);
hipError_t launch_page_mark(const int32_t* idx, int64_t num_idx, int32_t num_src_pages,
                            int32_t src_page_tokens, int8_t* mask, hipStream_t stream);
hipError_t launch_page_split(const PageParams& p, hipStream_t stream);
hipError_t launch_topk(const TopkParams& p, hipStream_t stream);

struct Fp8RowsParams {
  const uint8_t* pool;
  int64_t pool_row_stride;   // bytes
  const int8_t* mask;        // nullable
  uint16_t* out;
  int64_t out_row_stride;    // elements
  int64_t rows;              // num_tokens * num_kv_heads
  int32_t num_kv_heads;
};
hipError_t launch_fp8_records_to_bf16(const Fp8RowsParams& p, hipStream_t stream);

// sa_probe.hip: the gather stream of the head-dim-256 kernels alone
struct GatherProbeParams {
  const void* k;         // [kv_len][256] bf16, 512-byte rows
  const void* v;
  const int32_t* idx;    // [num_rows][topk]
  uint32_t* out;         // [num_rows][64] checksums
  int32_t num_rows, topk, kv_len;
  int32_t eight_waves;   // 1: at most eight waves per CU, like the attention kernels
};
hipError_t launch_gather_probe(const GatherProbeParams& p, hipStream_t stream);

// sa_api.cpp: the decode entry points' common body (counted under `entry`
// on success). Without `scratch` it runs over the caller's `ws`; with it,
// once every argument has passed, over the static scratch of `ws_bytes`
// that scratch() returns (nullptr and a message in msg when the lookup
// fails).
using ScratchFn = void* (*)(char* msg, size_t msg_len);
sa_status decode_paged_ws(const sa_attn_desc* desc, const sa_page_desc* pages, const void* q,
                          const uint8_t* pool, int32_t num_dst_pages, const int32_t* idx,
                          const int32_t* topk_len, int32_t batch, void* ws, size_t ws_bytes,
                          float* out, float* lse, hipStream_t stream, int entry,
                          ScratchFn scratch);
// Clears the calling thread's error text (entry points defined elsewhere).
void api_clear_error();

}  // namespace sa
