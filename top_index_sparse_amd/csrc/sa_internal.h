// Internal interface between the C ABI (sa_api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
  int32_t teams_per_group;    // union: teams serving one group
  // rows one team serves (per-token: consecutive rows; union: group members)
  int32_t rows_per_team;
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
};

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

// union: 0 per-token results (ragged when cu_q is set), 1 union lists. The
// launchers choose the team shape (rows per team, column tiles).
hipError_t launch_attn_gqa256(AttnParams p, int union_mode, hipStream_t stream);
hipError_t launch_attn_mla576(AttnParams p, int union_mode, hipStream_t stream);
hipError_t launch_union_build(const UnionBuildParams& p, hipStream_t stream);
hipError_t launch_page_mark(const int32_t* idx, int64_t num_idx, int32_t num_src_pages,
                            int32_t src_page_tokens, int8_t* mask, hipStream_t stream);
hipError_t launch_page_split(const PageParams& p, hipStream_t stream);

}  // namespace sa
