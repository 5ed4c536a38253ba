// C ABI of the sparse attention library: argument validation, launch
// geometry, status codes, per-thread error text and call counters.
// Nothing here allocates device memory or reads it back.
#include "sparse_attn.h"

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "sa_internal.h"

namespace {

thread_local char g_err[512] = "";
std::atomic<uint64_t> g_calls[SA_ENTRY_COUNT];

sa_status fail(sa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

sa_status ok(sa_entry e, sa_status st = SA_OK) {
  g_calls[e].fetch_add(1, std::memory_order_relaxed);
  return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

enum class Kernel { kNone, kGqa256, kMla576, kMla576Fp8 };

constexpr int64_t kFp8RecordBytes = 656;   // 512 E4M3 + 4 fp32 scales + 64 bf16

// Which built kernel serves this descriptor (no pointer checks).
sa_status check_desc(const sa_attn_desc* d, int32_t G, Kernel* kernel) {
  if (!d) return fail(SA_ERR_NULL, "desc is NULL");
  if (d->kv_dtype != SA_DTYPE_BF16 && d->kv_dtype != SA_DTYPE_FP8_E4M3)
    return fail(SA_ERR_DTYPE, "kv_dtype %d: bf16 K/V, or FP8 MLA records, only", d->kv_dtype);
  const bool fp8 = d->kv_dtype == SA_DTYPE_FP8_E4M3;
  if (d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->num_q_heads % d->num_kv_heads != 0)
    return fail(SA_ERR_SHAPE, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                d->num_q_heads, d->num_kv_heads);
  if (d->topk <= 0) return fail(SA_ERR_SHAPE, "topk %d must be positive", d->topk);
  if (!std::isfinite(d->sm_scale)) return fail(SA_ERR_SHAPE, "sm_scale is not finite");
  if (d->head_dim_qk <= 0 || d->head_dim_v <= 0)
    return fail(SA_ERR_SHAPE, "head dims must be positive");
  if (d->v_in_k && d->head_dim_v > d->head_dim_qk)
    return fail(SA_ERR_SHAPE, "v_in_k needs head_dim_v <= head_dim_qk");
  const int group = d->num_q_heads / d->num_kv_heads;
  if (d->head_dim_qk == 256 && d->head_dim_v == 256 && !d->v_in_k) {
    *kernel = Kernel::kGqa256;
  } else if (d->head_dim_qk == 576 && d->head_dim_v == 512 && d->v_in_k) {
    *kernel = fp8 ? Kernel::kMla576Fp8 : Kernel::kMla576;
  } else {
    return fail(SA_ERR_UNSUPPORTED,
                "head dims (%d, %d, v_in_k=%d) not built; built: (256, 256, 0), (576, 512, 1)",
                d->head_dim_qk, d->head_dim_v, d->v_in_k);
  }
  if (fp8 && *kernel != Kernel::kMla576Fp8)
    return fail(SA_ERR_DTYPE, "FP8 K is accepted as 656-byte MLA records (576/512, v_in_k) only");
  // at most 32 query heads per KV head, the pages' cap; an MLA row of more
  // than 16 heads runs as two 16-head slices over its one latent head
  if (group > 32) return fail(SA_ERR_UNSUPPORTED, "group %d > 32 query heads per KV head", group);
  if (d->v_in_k && group > 16 && d->num_kv_heads != 1)
    return fail(SA_ERR_UNSUPPORTED, "MLA with %d > 16 query heads needs one latent KV head", group);
  const int64_t qrow = (int64_t)d->num_q_heads * d->head_dim_qk;
  const int64_t krow = (int64_t)d->num_kv_heads * d->head_dim_qk;
  const int64_t vrow = (int64_t)d->num_kv_heads * d->head_dim_v;
  const int64_t orow = (int64_t)d->num_q_heads * d->head_dim_v;
  if (d->q_row_stride < qrow || d->q_row_stride % 8)
    return fail(SA_ERR_SHAPE, "q_row_stride %lld: needs >= %lld and a multiple of 8",
                (long long)d->q_row_stride, (long long)qrow);
  // Row byte strides are 32-bit multipliers in the kernels' address math.
  if (fp8) {
    // records: kv_row_stride counts bytes
    const int64_t rec = (int64_t)d->num_kv_heads * kFp8RecordBytes;
    if (d->kv_row_stride < rec || d->kv_row_stride % 16 || d->kv_row_stride >= (int64_t)1 << 32)
      return fail(SA_ERR_SHAPE, "kv_row_stride %lld bytes: needs >= %lld, a multiple of 16, < 2^32",
                  (long long)d->kv_row_stride, (long long)rec);
  } else if (d->kv_row_stride < krow || d->kv_row_stride % 8 || d->kv_row_stride >= (int64_t)1 << 31)
    return fail(SA_ERR_SHAPE, "kv_row_stride %lld: needs >= %lld, a multiple of 8, < 2^31",
                (long long)d->kv_row_stride, (long long)krow);
  if (!d->v_in_k &&
      (d->v_row_stride < vrow || d->v_row_stride % 8 || d->v_row_stride >= (int64_t)1 << 31))
    return fail(SA_ERR_SHAPE, "v_row_stride %lld: needs >= %lld, a multiple of 8, < 2^31",
                (long long)d->v_row_stride, (long long)vrow);
  if (d->idx_row_stride < d->topk)
    return fail(SA_ERR_SHAPE, "idx_row_stride %lld < topk %d", (long long)d->idx_row_stride,
                d->topk);
  if (d->out_row_stride < orow || d->out_row_stride % 4)
    return fail(SA_ERR_SHAPE, "out_row_stride %lld: needs >= %lld and a multiple of 4",
                (long long)d->out_row_stride, (long long)orow);
  if (G < 1 || G > 8) return fail(SA_ERR_SHAPE, "union group size G %d outside 1..8", G);
  if (G > 1 && G * group > 32) return SA_OK_FALLBACK;
  return SA_OK;
}

sa_status check_ptrs(const sa_attn_desc* d, const void* q, const void* k, const void* v,
                     const int32_t* idx, const float* out, const float* lse) {
  if (!q || !k || !idx || !out || !lse || (!d->v_in_k && !v))
    return fail(SA_ERR_NULL, "q, k, v (unless v_in_k), idx, out and lse are required");
  if (!aligned16(q) || !aligned16(k) || (!d->v_in_k && !aligned16(v)) || !aligned16(out))
    return fail(SA_ERR_SHAPE, "q, k, v and out must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(idx) & 3u) || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(SA_ERR_SHAPE, "idx and lse must be 4-byte aligned");
  return SA_OK;
}

sa::AttnParams make_params(const sa_attn_desc* d, const void* q, const void* k, const void* v,
                           const int32_t* idx, float* out, float* lse, int32_t num_rows) {
  sa::AttnParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = d->v_in_k ? p.k : static_cast<const uint16_t*>(v);
  p.idx = idx;
  p.out = out;
  p.lse = lse;
  p.q_row_stride = d->q_row_stride;
  // in 2-byte units (the kernels' byte stride is twice this); FP8 record
  // strides are given in bytes and are even
  const int64_t kstride = d->kv_dtype == SA_DTYPE_FP8_E4M3 ? d->kv_row_stride / 2 : d->kv_row_stride;
  p.k_row_stride = kstride;
  p.v_row_stride = d->v_in_k ? kstride : d->v_row_stride;
  p.idx_row_stride = d->idx_row_stride;
  p.out_row_stride = d->out_row_stride;
  p.lse_row_stride = d->num_q_heads;
  p.num_rows = num_rows;
  p.topk = d->topk;
  p.num_q_heads = d->num_q_heads;
  p.num_kv_heads = d->num_kv_heads;
  p.group = d->num_q_heads / d->num_kv_heads;
  p.scale_log2e = d->sm_scale * 1.4426950408889634f;
  return p;
}

// union_mode: 0 per-token results (ragged when p.cu_q is set), 1 union lists
sa_status launch_attention(Kernel kernel, const sa::AttnParams& p, int union_mode, hipStream_t s) {
  hipError_t e = hipSuccess;
  switch (kernel) {
    case Kernel::kGqa256:
      e = sa::launch_attn_gqa256(p, union_mode, s);
      break;
    case Kernel::kMla576:
      e = sa::launch_attn_mla576(p, union_mode, s);
      break;
    case Kernel::kMla576Fp8:
      e = sa::launch_attn_mla576_fp8(p, union_mode, s);
      break;
    default:
      return fail(SA_ERR_UNSUPPORTED, "no kernel for this head-dim combination");
  }
  // the launchers refuse a grid beyond one launch before calling HIP
  if (e == hipErrorInvalidConfiguration)
    return fail(SA_ERR_SHAPE, "%d rows x %d KV heads exceed one launch", p.num_rows,
                p.num_kv_heads);
  if (e != hipSuccess) return fail(SA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return SA_OK;
}

constexpr int kMaxTopkPad = 8192;  // sort keys held in 32 KB of LDS

int64_t pow2_at_least(int64_t x) {
  int64_t p = 1;
  while (p < x) p <<= 1;
  return p;
}

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Workspace layout shared by union_build and prefill_union.
struct UnionLayout {
  int64_t topk_pad, groups, stride;
  int64_t sorted_off, idx_off, bits_off, len_off, total;
};

bool union_layout(int32_t num_rows, int32_t topk, int32_t G, UnionLayout* L) {
  if (num_rows < 0 || topk <= 0 || G < 1 || G > 8) return false;
  L->topk_pad = pow2_at_least(topk < 256 ? 256 : topk);
  if (L->topk_pad > kMaxTopkPad) return false;
  L->groups = (num_rows + G - 1) / G;
  L->stride = align_up((int64_t)G * topk, 16);
  L->sorted_off = 0;
  L->idx_off = align_up((int64_t)num_rows * L->topk_pad * 4, 256);
  L->bits_off = L->idx_off + align_up(L->groups * L->stride * 4, 256);
  L->len_off = L->bits_off + align_up(L->groups * L->stride, 256);
  L->total = L->len_off + align_up(L->groups * 4, 256);
  return true;
}

// Workspace layout of chunk_prefill_union: per-request first group ids,
// then the union lists of at most ceil(total_q / G) + num_reqs groups.
struct ChunkUnionLayout {
  int64_t groups, stride;
  int64_t gstart_off, idx_off, bits_off, len_off, total;
};

bool chunk_union_layout(int32_t total_q, int32_t num_reqs, int32_t topk, int32_t G,
                        ChunkUnionLayout* L) {
  if (total_q < 0 || num_reqs < 1 || topk <= 0 || G < 1 || G > 8) return false;
  L->groups = ((int64_t)total_q + G - 1) / G + num_reqs;
  if (L->groups > INT32_MAX) return false;
  L->stride = align_up((int64_t)G * topk, 16);
  L->gstart_off = 0;
  L->idx_off = align_up(((int64_t)num_reqs + 1) * 4, 256);
  L->bits_off = L->idx_off + align_up(L->groups * L->stride * 4, 256);
  L->len_off = L->bits_off + align_up(L->groups * L->stride, 256);
  L->total = L->len_off + align_up(L->groups * 4, 256);
  return true;
}

// Slot ranges of a decode launch. Range s of S takes a request's 16-slot
// tiles s, s + S, s + 2S, ... (so a request whose valid slots come first
// still spreads them over its ranges). S aims at kDecodeTeams (request,
// range) teams, one wave per SIMD (a sweep of 256 to 4096 teams measured
// 512 fastest: more ranges only add partial rows to merge), and at most
// kDecodeTilesPerRange tiles per range. Workspace: normalised partial O
// [batch * S][heads][512] fp32, then partial LSE [batch * S][heads] fp32,
// each 256-byte aligned.
constexpr int64_t kDecodeTeams = 512;
constexpr int64_t kDecodeTilesPerRange = 8;

struct DecodeLayout {
  int32_t splits;
  int64_t lse_off, total;
};

bool decode_layout(int32_t batch, int32_t num_q_heads, int32_t topk, DecodeLayout* L) {
  if (batch < 0 || num_q_heads <= 0 || num_q_heads > 32 || topk <= 0) return false;
  const int64_t tiles = ((int64_t)topk + 15) / 16;
  int64_t s = batch > 0 ? (kDecodeTeams + batch - 1) / batch : 1;
  const int64_t s_min = (tiles + kDecodeTilesPerRange - 1) / kDecodeTilesPerRange;
  if (s < s_min) s = s_min;
  if (s > tiles) s = tiles;
  L->splits = (int32_t)s;
  const int64_t rows = (int64_t)batch * L->splits;
  if (rows > INT32_MAX) return false;
  L->lse_off = align_up(rows * num_q_heads * 512 * 4, 256);
  L->total = L->lse_off + align_up(rows * num_q_heads * 4, 256);
  return true;
}

sa::UnionBuildParams build_params(const int32_t* idx, int64_t idx_row_stride, int32_t num_rows,
                                  int32_t topk, int32_t kv_len, int32_t G, const UnionLayout& L,
                                  void* ws) {
  sa::UnionBuildParams b{};
  b.idx = idx;
  b.idx_row_stride = idx_row_stride;
  b.num_rows = num_rows;
  b.topk = topk;
  b.kv_len = kv_len;
  b.G = G;
  b.sorted = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + L.sorted_off);
  b.topk_pad = (int32_t)L.topk_pad;
  return b;
}

}  // namespace

extern "C" {

int sa_validate_attn(const sa_attn_desc* desc, int32_t G) {
  Kernel kernel = Kernel::kNone;
  return check_desc(desc, G, &kernel);
}

const char* sa_last_error(void) { return g_err; }

uint64_t sa_call_count(int32_t entry) {
  if (entry < 0 || entry >= SA_ENTRY_COUNT) return 0;
  return g_calls[entry].load(std::memory_order_relaxed);
}

sa_status sparse_attn_prefill(const sa_attn_desc* desc, const void* q, const void* k,
                              const void* v, const int32_t* idx, const int32_t* topk_len,
                              int32_t num_rows, int32_t kv_len, float* out, float* lse,
                              hipStream_t stream) {
  g_err[0] = 0;
  Kernel kernel = Kernel::kNone;
  sa_status st = check_desc(desc, 1, &kernel);
  if (st != SA_OK) return st;
  if (num_rows < 0 || kv_len < 0)
    return fail(SA_ERR_SHAPE, "num_rows %d and kv_len %d must be >= 0", num_rows, kv_len);
  if (num_rows == 0) return ok(SA_ENTRY_PREFILL);
  st = check_ptrs(desc, q, k, v, idx, out, lse);
  if (st != SA_OK) return st;
  sa::AttnParams p = make_params(desc, q, k, v, idx, out, lse, num_rows);
  p.topk_len = topk_len;
  p.kv_len = kv_len;
  p.num_reqs = 1;
  st = launch_attention(kernel, p, 0, stream);
  return st == SA_OK ? ok(SA_ENTRY_PREFILL) : st;
}

sa_status sparse_attn_chunk_prefill(const sa_attn_desc* desc, const void* q, const void* k,
                                    const void* v, const int32_t* idx,
                                    const int32_t* cu_seqlens_q, const int64_t* cu_seqlens_kv,
                                    int32_t num_reqs, int32_t total_q, float* out, float* lse,
                                    hipStream_t stream) {
  g_err[0] = 0;
  Kernel kernel = Kernel::kNone;
  sa_status st = check_desc(desc, 1, &kernel);
  if (st != SA_OK) return st;
  if (num_reqs < 0 || total_q < 0)
    return fail(SA_ERR_SHAPE, "num_reqs %d and total_q %d must be >= 0", num_reqs, total_q);
  if (total_q == 0 || num_reqs == 0) {
    if (total_q != 0) return fail(SA_ERR_SHAPE, "total_q %d rows but no request", total_q);
    return ok(SA_ENTRY_CHUNK_PREFILL);
  }
  if (!cu_seqlens_q || !cu_seqlens_kv) return fail(SA_ERR_NULL, "cu_seqlens_q/kv are required");
  st = check_ptrs(desc, q, k, v, idx, out, lse);
  if (st != SA_OK) return st;
  sa::AttnParams p = make_params(desc, q, k, v, idx, out, lse, total_q);
  p.cu_q = cu_seqlens_q;
  p.cu_kv = cu_seqlens_kv;
  p.num_reqs = num_reqs;
  st = launch_attention(kernel, p, 0, stream);
  return st == SA_OK ? ok(SA_ENTRY_CHUNK_PREFILL) : st;
}

size_t sparse_attn_union_workspace_bytes(int32_t num_rows, int32_t topk, int32_t G) {
  UnionLayout L;
  if (!union_layout(num_rows, topk, G, &L)) return 0;
  return (size_t)L.total;
}

sa_status sparse_attn_union_build(const int32_t* idx, int64_t idx_row_stride, int32_t num_rows,
                                  int32_t topk, int32_t kv_len, int32_t G, int32_t* union_idx,
                                  uint8_t* union_bits, int32_t* union_len, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  UnionLayout L;
  if (num_rows < 0 || kv_len < 0 || !union_layout(num_rows, topk, G, &L))
    return fail(SA_ERR_SHAPE, "num_rows %d, topk %d (<= %d), G %d (1..8), kv_len %d", num_rows,
                topk, kMaxTopkPad, G, kv_len);
  if (idx_row_stride < topk) return fail(SA_ERR_SHAPE, "idx_row_stride < topk");
  if (num_rows == 0) return ok(SA_ENTRY_UNION_BUILD);
  if (!idx || !union_idx || !union_bits || !union_len)
    return fail(SA_ERR_NULL, "idx and the three outputs are required");
  if (!ws || ws_bytes < (size_t)L.idx_off)
    return fail(SA_ERR_WORKSPACE, "workspace of %zu bytes, %lld needed", ws_bytes,
                (long long)L.idx_off);
  if ((reinterpret_cast<uintptr_t>(ws) & 255) || (reinterpret_cast<uintptr_t>(idx) & 3) ||
      (reinterpret_cast<uintptr_t>(union_idx) & 3) || (reinterpret_cast<uintptr_t>(union_len) & 3))
    return fail(SA_ERR_SHAPE, "ws must be 256-byte aligned; idx and int32 outputs 4-byte aligned");
  sa::UnionBuildParams b = build_params(idx, idx_row_stride, num_rows, topk, kv_len, G, L, ws);
  b.union_idx = union_idx;
  b.union_bits = union_bits;
  b.union_len = union_len;
  b.union_stride = (int64_t)G * topk;
  b.fill_tail = 1;   // the documented -1 / 0 fill after union_len
  const hipError_t e = sa::launch_union_build(b, stream);
  if (e != hipSuccess) return fail(SA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok(SA_ENTRY_UNION_BUILD);
}

sa_status sparse_attn_prefill_union(const sa_attn_desc* desc, const void* q, const void* k,
                                    const void* v, const int32_t* idx, int32_t num_rows,
                                    int32_t kv_len, int32_t G, void* ws, size_t ws_bytes,
                                    float* out, float* lse, hipStream_t stream) {
  g_err[0] = 0;
  Kernel kernel = Kernel::kNone;
  const sa_status legal = check_desc(desc, G, &kernel);
  if (legal != SA_OK && legal != SA_OK_FALLBACK) return legal;
  if (num_rows < 0 || kv_len < 0)
    return fail(SA_ERR_SHAPE, "num_rows %d and kv_len %d must be >= 0", num_rows, kv_len);
  if (num_rows == 0) return ok(SA_ENTRY_PREFILL_UNION, legal);
  sa_status st = check_ptrs(desc, q, k, v, idx, out, lse);
  if (st != SA_OK) return st;
  sa::AttnParams p = make_params(desc, q, k, v, idx, out, lse, num_rows);
  p.kv_len = kv_len;
  p.num_reqs = 1;
  if (legal == SA_OK_FALLBACK) {
    // G * group > 32: the per-token path gives every row its own result
    st = launch_attention(kernel, p, 0, stream);
    return st == SA_OK ? ok(SA_ENTRY_PREFILL_UNION, SA_OK_FALLBACK) : st;
  }
  UnionLayout L;
  if (!union_layout(num_rows, desc->topk, G, &L))
    return fail(SA_ERR_SHAPE, "topk %d above %d", desc->topk, kMaxTopkPad);
  if (!ws || ws_bytes < (size_t)L.total)
    return fail(SA_ERR_WORKSPACE, "workspace of %zu bytes, %lld needed", ws_bytes,
                (long long)L.total);
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(SA_ERR_SHAPE, "ws must be 256-byte aligned");
  char* base = static_cast<char*>(ws);
  sa::UnionBuildParams b =
      build_params(idx, desc->idx_row_stride, num_rows, desc->topk, kv_len, G, L, ws);
  b.union_idx = reinterpret_cast<int32_t*>(base + L.idx_off);
  b.union_bits = reinterpret_cast<uint8_t*>(base + L.bits_off);
  b.union_len = reinterpret_cast<int32_t*>(base + L.len_off);
  b.union_stride = L.stride;
  hipError_t e = sa::launch_union_build(b, stream);
  if (e != hipSuccess) return fail(SA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  p.union_idx = b.union_idx;
  p.union_bits = b.union_bits;
  p.union_len = b.union_len;
  p.union_stride = L.stride;
  p.G = G;
  p.num_groups = (int32_t)L.groups;
  st = launch_attention(kernel, p, 1, stream);
  return st == SA_OK ? ok(SA_ENTRY_PREFILL_UNION) : st;
}

size_t sparse_attn_chunk_union_workspace_bytes(int32_t total_q, int32_t num_reqs, int32_t topk,
                                               int32_t G) {
  ChunkUnionLayout L;
  if (!chunk_union_layout(total_q, num_reqs, topk, G, &L)) return 0;
  return (size_t)L.total;
}

sa_status sparse_attn_chunk_prefill_union(const sa_attn_desc* desc, const void* q, const void* k,
                                          const void* v, const int32_t* idx,
                                          const int32_t* cu_seqlens_q,
                                          const int64_t* cu_seqlens_kv, int32_t num_reqs,
                                          int32_t total_q, int32_t G, void* ws, size_t ws_bytes,
                                          float* out, float* lse, hipStream_t stream) {
  g_err[0] = 0;
  Kernel kernel = Kernel::kNone;
  const sa_status legal = check_desc(desc, G, &kernel);
  if (legal != SA_OK && legal != SA_OK_FALLBACK) return legal;
  if (num_reqs < 0 || total_q < 0)
    return fail(SA_ERR_SHAPE, "num_reqs %d and total_q %d must be >= 0", num_reqs, total_q);
  if (total_q == 0 || num_reqs == 0) {
    if (total_q != 0) return fail(SA_ERR_SHAPE, "total_q %d rows but no request", total_q);
    return ok(SA_ENTRY_CHUNK_PREFILL_UNION, legal);
  }
  if (!cu_seqlens_q || !cu_seqlens_kv) return fail(SA_ERR_NULL, "cu_seqlens_q/kv are required");
  sa_status st = check_ptrs(desc, q, k, v, idx, out, lse);
  if (st != SA_OK) return st;
  sa::AttnParams p = make_params(desc, q, k, v, idx, out, lse, total_q);
  p.cu_q = cu_seqlens_q;
  p.cu_kv = cu_seqlens_kv;
  p.num_reqs = num_reqs;
  if (legal == SA_OK_FALLBACK) {
    // G * group > 32: the per-token path gives every row its own result
    st = launch_attention(kernel, p, 0, stream);
    return st == SA_OK ? ok(SA_ENTRY_CHUNK_PREFILL_UNION, SA_OK_FALLBACK) : st;
  }
  ChunkUnionLayout L;
  if (!chunk_union_layout(total_q, num_reqs, desc->topk, G, &L))
    return fail(SA_ERR_SHAPE, "too many union groups for one launch");
  if (!ws || ws_bytes < (size_t)L.total)
    return fail(SA_ERR_WORKSPACE, "workspace of %zu bytes, %lld needed", ws_bytes,
                (long long)L.total);
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(SA_ERR_SHAPE, "ws must be 256-byte aligned");
  char* base = static_cast<char*>(ws);
  int32_t* gstart = reinterpret_cast<int32_t*>(base + L.gstart_off);
  sa::UnionBuildParams b{};
  b.idx = idx;
  b.idx_row_stride = desc->idx_row_stride;
  b.num_rows = total_q;
  b.topk = desc->topk;
  b.G = G;
  b.union_idx = reinterpret_cast<int32_t*>(base + L.idx_off);
  b.union_bits = reinterpret_cast<uint8_t*>(base + L.bits_off);
  b.union_len = reinterpret_cast<int32_t*>(base + L.len_off);
  b.union_stride = L.stride;
  b.cu_q = cu_seqlens_q;
  b.cu_kv = cu_seqlens_kv;
  b.num_reqs = num_reqs;
  b.num_groups = (int32_t)L.groups;
  hipError_t e = sa::launch_union_build_ragged(b, gstart, stream);
  if (e != hipSuccess) return fail(SA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  p.union_idx = b.union_idx;
  p.union_bits = b.union_bits;
  p.union_len = b.union_len;
  p.union_stride = L.stride;
  p.G = G;
  p.num_groups = (int32_t)L.groups;
  p.gstart = gstart;
  st = launch_attention(kernel, p, 1, stream);
  return st == SA_OK ? ok(SA_ENTRY_CHUNK_PREFILL_UNION) : st;
}

size_t sparse_attn_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t topk) {
  DecodeLayout L;
  if (!decode_layout(batch, num_q_heads, topk, &L)) return 0;
  return (size_t)L.total;
}

}  // extern "C"

namespace sa {

// The decode entry points' common body: validation, then the range teams
// and the merge over the workspace: the caller's `ws`, or, when `scratch`
// is given, the static scratch of `ws_bytes` it returns once every argument
// has passed (nullptr, with a message, when its lookup fails). Counts a
// successful call under `entry`.
sa_status decode_paged_ws(const sa_attn_desc* desc, const sa_page_desc* pages, const void* q,
                          const uint8_t* pool, int32_t num_dst_pages, const int32_t* idx,
                          const int32_t* topk_len, int32_t batch, void* ws, size_t ws_bytes,
                          float* out, float* lse, hipStream_t stream, int entry,
                          ScratchFn scratch) {
  Kernel kernel = Kernel::kNone;
  sa_status st = check_desc(desc, 1, &kernel);
  if (st != SA_OK) return st;
  if (kernel != Kernel::kMla576Fp8)
    return fail(SA_ERR_DTYPE, "decode reads FP8 MLA records: head dims (576, 512), v_in_k, "
                              "kv_dtype SA_DTYPE_FP8_E4M3");
  if (desc->num_kv_heads != 1)
    return fail(SA_ERR_SHAPE, "a page row holds one latent record per token: num_kv_heads %d != 1",
                desc->num_kv_heads);
  if (!pages) return fail(SA_ERR_NULL, "pages is NULL");
  const int32_t ptok = pages->dst_page_tokens;
  if (ptok <= 0 || (ptok & (ptok - 1)) || ptok > (1 << 20))
    return fail(SA_ERR_SHAPE, "dst_page_tokens %d must be a power of two <= 2^20", ptok);
  if (pages->row_bytes != kFp8RecordBytes || desc->kv_row_stride != kFp8RecordBytes)
    return fail(SA_ERR_SHAPE, "token rows are 656-byte records: row_bytes %d, kv_row_stride %lld",
                pages->row_bytes, (long long)desc->kv_row_stride);
  if (pages->scale_bytes < 0) return fail(SA_ERR_SHAPE, "scale_bytes %d < 0", pages->scale_bytes);
  const int64_t page_min = (int64_t)ptok * (pages->row_bytes + pages->scale_bytes);
  if (pages->dst_page_stride < page_min || pages->dst_page_stride % 16 ||
      pages->dst_page_stride >= (int64_t)1 << 32)
    return fail(SA_ERR_SHAPE, "dst_page_stride %lld: needs >= %lld, a multiple of 16, < 2^32",
                (long long)pages->dst_page_stride, (long long)page_min);
  if (num_dst_pages < 0 || batch < 0)
    return fail(SA_ERR_SHAPE, "num_dst_pages %d and batch %d must be >= 0", num_dst_pages, batch);
  if ((int64_t)num_dst_pages * ptok > INT32_MAX)
    return fail(SA_ERR_SHAPE, "pool tokens (%d pages x %d) must stay below 2^31", num_dst_pages,
                ptok);
  DecodeLayout L;
  if (!decode_layout(batch, desc->num_q_heads, desc->topk, &L))
    return fail(SA_ERR_SHAPE, "decode of batch %d x topk %d does not fit one launch", batch,
                desc->topk);
  if (batch == 0) return ok(static_cast<sa_entry>(entry));
  st = check_ptrs(desc, q, pool, nullptr, idx, out, lse);
  if (st != SA_OK) return st;
  if (scratch) {
    if ((size_t)L.total > ws_bytes)
      return fail(SA_ERR_WORKSPACE,
                  "decode of batch %d x %d heads x topk %d needs %lld bytes of partial results; "
                  "the static scratch holds %zu (use sparse_attn_decode_paged with a workspace)",
                  batch, desc->num_q_heads, desc->topk, (long long)L.total, ws_bytes);
    char msg[200] = "";
    ws = scratch(msg, sizeof(msg));
    if (!ws) return fail(SA_ERR_HIP, "%s", msg);
  }
  if (!ws || ws_bytes < (size_t)L.total || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return fail(SA_ERR_WORKSPACE, "ws: needs %lld bytes, 256-byte aligned (got %zu)",
                (long long)L.total, ws_bytes);
  float* part_out = static_cast<float*>(ws);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(ws) + L.lse_off);
  const int32_t rows = batch * L.splits;
  sa::AttnParams p = make_params(desc, q, pool, nullptr, idx, part_out, part_lse, rows);
  p.out_row_stride = (int64_t)desc->num_q_heads * 512;
  p.topk_len = topk_len;
  p.kv_len = num_dst_pages * ptok;
  p.num_reqs = 1;
  p.dec_splits = L.splits;
  int shift = 0;
  while ((1 << shift) < ptok) ++shift;
  p.page_shift = shift;
  p.page_stride = pages->dst_page_stride;
  sa::DecodeCombineParams c{};
  c.part_out = part_out;
  c.part_lse = part_lse;
  c.out = out;
  c.lse = lse;
  c.out_row_stride = desc->out_row_stride;
  c.batch = batch;
  c.splits = L.splits;
  c.num_q_heads = desc->num_q_heads;
  const hipError_t e = sa::launch_decode_mla576_fp8(p, c, stream);
  if (e == hipErrorInvalidConfiguration)
    return fail(SA_ERR_SHAPE, "decode of batch %d does not fit one launch", batch);
  if (e != hipSuccess) return fail(SA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok(static_cast<sa_entry>(entry));
}

void api_clear_error() { g_err[0] = 0; }

}  // namespace sa

extern "C" {

sa_status sparse_attn_decode_paged(const sa_attn_desc* desc, const sa_page_desc* pages,
                                   const void* q, const uint8_t* pool, int32_t num_dst_pages,
                                   const int32_t* idx, const int32_t* topk_len, int32_t batch,
                                   void* ws, size_t ws_bytes, float* out, float* lse,
                                   hipStream_t stream) {
  g_err[0] = 0;
  return sa::decode_paged_ws(desc, pages, q, pool, num_dst_pages, idx, topk_len, batch, ws,
                             ws_bytes, out, lse, stream, SA_ENTRY_DECODE_PAGED, nullptr);
}

sa_status indexer_topk(const float* scores, int64_t score_row_stride, const int32_t* row_len,
                       int32_t num_rows, int32_t kv_len, int32_t k, int32_t* idx,
                       int64_t idx_row_stride, hipStream_t stream) {
  g_err[0] = 0;
  if (num_rows < 0 || kv_len < 0 || k <= 0)
    return fail(SA_ERR_SHAPE, "num_rows %d, kv_len %d must be >= 0 and k %d > 0", num_rows, kv_len, k);
  if (score_row_stride < kv_len)
    return fail(SA_ERR_SHAPE, "score_row_stride %lld < kv_len %d", (long long)score_row_stride,
                kv_len);
  if (idx_row_stride < k)
    return fail(SA_ERR_SHAPE, "idx_row_stride %lld < k %d", (long long)idx_row_stride, k);
  if (num_rows == 0) return ok(SA_ENTRY_INDEXER_TOPK);
  if (!scores || !idx) return fail(SA_ERR_NULL, "scores and idx are required");
  if ((reinterpret_cast<uintptr_t>(scores) & 3u) || (reinterpret_cast<uintptr_t>(idx) & 3u) ||
      (reinterpret_cast<uintptr_t>(row_len) & 3u))
    return fail(SA_ERR_SHAPE, "scores, idx and row_len must be 4-byte aligned");
  sa::TopkParams p{};
  p.scores = scores;
  p.score_row_stride = score_row_stride;
  p.row_len = row_len;
  p.num_rows = num_rows;
  p.kv_len = kv_len;
  p.k = k;
  p.idx = idx;
  p.idx_row_stride = idx_row_stride;
  const hipError_t e = sa::launch_topk(p, stream);
  if (e != hipSuccess) return fail(SA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok(SA_ENTRY_INDEXER_TOPK);
}

sa_status sparse_attn_fp8_records_to_bf16(const uint8_t* pool, int64_t pool_row_stride,
                                          int32_t num_tokens, int32_t num_kv_heads,
                                          const int8_t* mask, void* out, int64_t out_row_stride,
                                          hipStream_t stream) {
  g_err[0] = 0;
  if (num_tokens < 0 || num_kv_heads <= 0)
    return fail(SA_ERR_SHAPE, "num_tokens %d, num_kv_heads %d", num_tokens, num_kv_heads);
  if (pool_row_stride < (int64_t)num_kv_heads * 656 || pool_row_stride % 16)
    return fail(SA_ERR_SHAPE, "pool_row_stride %lld: at least %d bytes and a multiple of 16",
                (long long)pool_row_stride, num_kv_heads * 656);
  if (out_row_stride < (int64_t)num_kv_heads * 576 || out_row_stride % 8)
    return fail(SA_ERR_SHAPE, "out_row_stride %lld: at least %d elements and a multiple of 8",
                (long long)out_row_stride, num_kv_heads * 576);
  if (num_tokens == 0) return ok(SA_ENTRY_FP8_RECORDS_TO_BF16);
  if (!pool || !out) return fail(SA_ERR_NULL, "pool and out are required");
  if ((reinterpret_cast<uintptr_t>(pool) & 15u) || (reinterpret_cast<uintptr_t>(out) & 15u))
    return fail(SA_ERR_SHAPE, "pool and out must be 16-byte aligned");
  sa::Fp8RowsParams p{};
  p.pool = pool;
  p.pool_row_stride = pool_row_stride;
  p.mask = mask;
  p.out = static_cast<uint16_t*>(out);
  p.out_row_stride = out_row_stride;
  p.rows = (int64_t)num_tokens * num_kv_heads;
  p.num_kv_heads = num_kv_heads;
  const hipError_t e = sa::launch_fp8_records_to_bf16(p, stream);
  if (e != hipSuccess) return fail(SA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok(SA_ENTRY_FP8_RECORDS_TO_BF16);
}

sa_status page_mark(const int32_t* idx, int64_t num_idx, int32_t num_src_pages,
                    int32_t src_page_tokens, int8_t* mask, hipStream_t stream) {
  g_err[0] = 0;
  if (num_idx < 0 || num_src_pages < 0 || src_page_tokens <= 0)
    return fail(SA_ERR_SHAPE, "num_idx %lld, num_src_pages %d, src_page_tokens %d",
                (long long)num_idx, num_src_pages, src_page_tokens);
  if (num_src_pages == 0) return ok(SA_ENTRY_PAGE_MARK);
  if (!mask || (num_idx > 0 && !idx)) return fail(SA_ERR_NULL, "mask and idx are required");
  if (reinterpret_cast<uintptr_t>(idx) & 3) return fail(SA_ERR_SHAPE, "idx must be 4-byte aligned");
  if ((num_idx + 255) / 256 > INT32_MAX) return fail(SA_ERR_SHAPE, "too many indices");
  const hipError_t e = sa::launch_page_mark(idx, num_idx, num_src_pages, src_page_tokens, mask,
                                            stream);
  if (e != hipSuccess) return fail(SA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok(SA_ENTRY_PAGE_MARK);
}

sa_status page_split(const sa_page_desc* desc, const uint8_t* src, uint8_t* dst,
                     const int8_t* mask, int32_t num_src_pages, hipStream_t stream) {
  g_err[0] = 0;
  if (!desc) return fail(SA_ERR_NULL, "desc is NULL");
  if (desc->src_page_tokens <= 0 || desc->dst_page_tokens <= 0 ||
      desc->src_page_tokens % desc->dst_page_tokens || desc->row_bytes < 0 ||
      desc->scale_bytes < 0 || num_src_pages < 0)
    return fail(SA_ERR_SHAPE, "page geometry: src %d tokens must be a positive multiple of dst %d",
                desc->src_page_tokens, desc->dst_page_tokens);
  const int64_t src_bytes = (int64_t)desc->src_page_tokens * (desc->row_bytes + desc->scale_bytes);
  const int64_t dst_bytes = (int64_t)desc->dst_page_tokens * (desc->row_bytes + desc->scale_bytes);
  if (desc->src_page_stride < src_bytes || desc->dst_page_stride < dst_bytes)
    return fail(SA_ERR_SHAPE, "page strides %lld / %lld below page sizes %lld / %lld",
                (long long)desc->src_page_stride, (long long)desc->dst_page_stride,
                (long long)src_bytes, (long long)dst_bytes);
  const int64_t ratio = desc->src_page_tokens / desc->dst_page_tokens;
  if ((int64_t)num_src_pages * ratio > INT32_MAX) return fail(SA_ERR_SHAPE, "too many pages");
  if (num_src_pages == 0) return ok(SA_ENTRY_PAGE_SPLIT);
  if (!src || !dst) return fail(SA_ERR_NULL, "src and dst are required");
  sa::PageParams p{};
  p.src = src;
  p.dst = dst;
  p.mask = mask;
  p.src_page_stride = desc->src_page_stride;
  p.dst_page_stride = desc->dst_page_stride;
  p.num_src_pages = num_src_pages;
  p.src_page_tokens = desc->src_page_tokens;
  p.dst_page_tokens = desc->dst_page_tokens;
  p.row_bytes = desc->row_bytes;
  p.scale_bytes = desc->scale_bytes;
  const hipError_t e = sa::launch_page_split(p, stream);
  if (e != hipSuccess) return fail(SA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok(SA_ENTRY_PAGE_SPLIT);
}

sa_status sa_probe_gather(const void* k, const void* v, int32_t kv_len, const int32_t* idx,
                          int32_t num_rows, int32_t topk, int32_t eight_waves, uint32_t* out,
                          hipStream_t stream) {
  if (num_rows < 0 || topk <= 0 || kv_len < 0)
    return fail(SA_ERR_SHAPE, "num_rows %d, kv_len %d must be >= 0 and topk %d > 0", num_rows,
                kv_len, topk);
  if ((int64_t)kv_len * 512 > (1ll << 31))
    return fail(SA_ERR_SHAPE, "kv_len %d: the rows must lie within 2 GiB", kv_len);
  if (eight_waves != 0 && eight_waves != 1) return fail(SA_ERR_SHAPE, "eight_waves must be 0 or 1");
  if (num_rows == 0) return SA_OK;
  if (!k || !v || !idx || !out) return fail(SA_ERR_NULL, "k, v, idx and out are required");
  if (!aligned16(k) || !aligned16(v)) return fail(SA_ERR_SHAPE, "k and v must be 16-byte aligned");
  sa::GatherProbeParams p{};
  p.k = k;
  p.v = v;
  p.idx = idx;
  p.out = out;
  p.num_rows = num_rows;
  p.topk = topk;
  p.kv_len = kv_len;
  p.eight_waves = eight_waves;
  const hipError_t e = sa::launch_gather_probe(p, stream);
  if (e != hipSuccess) return fail(SA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return SA_OK;
}

}  // extern "C"
