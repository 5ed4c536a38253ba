/*
 * sparse_attn.h -- C ABI of the index-gathered sparse attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes, on the caller's HIP stream:
 *   - per-token sparse attention forward: every query row gathers its own
 *     top-k KV slots (int32 token indices, -1 = padding), scores them against
 *     the query heads of one GQA group (or MLA head set), and writes the
 *     softmax-weighted sum of the gathered V rows plus the log-sum-exp;
 *   - the same over ragged requests with cached prefixes (chunk prefill);
 *   - union mode: G adjacent rows share one sorted, deduplicated index set
 *     with per-row ownership bits that restore each row's own support;
 *   - the decode-pool page mark and (masked) page split;
 *   - sparse MLA decode over the split pool's FP8 records;
 *   - the indexer's top-k selection, from scores to index rows.
 *
 * Conventions for every entry point:
 *   - Device pointers are owned by the caller. The library allocates and
 *     frees nothing, keeps no state between calls except call counters, the
 *     last error message and the static decode scratch of
 *     sparse_attn_decode_paged_noalloc, and never reads device memory from
 *     the host.
 *   - Work is enqueued on `stream` and returns without synchronising; the
 *     grids depend on host scalars only, so every call can be captured in a
 *     HIP graph.
 *   - Argument errors are reported before anything is launched; a launch
 *     failure returns SA_ERR_HIP. sa_last_error() describes the last error
 *     of the calling thread.
 *   - bf16 tensors (q, k, v) need 16-byte aligned base pointers and row
 *     strides that are multiples of 8 elements; fp32 outputs need 16-byte
 *     aligned base pointers and row strides that are multiples of 4.
 *   - An index x of a row is valid iff 0 <= x < kv_len (kv_len of the row's
 *     request). Invalid slots are never dereferenced and contribute nothing.
 *     A row with no valid slot gets O = 0 and LSE = -inf.
 *   - Duplicated indices in one row count with multiplicity on the
 *     per-token paths (sglang PR 32779, "Accuracy Tests": a row selected
 *     twice counts twice there); union mode lists every row once.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SA_OK = 0,
  /* Union tile illegal for this head group (G * group > 32): the per-token
   * result was computed instead (sglang PR 32779, review item 1: an illegal
   * union tile falls back to the per-token path). */
  SA_OK_FALLBACK = 1,
  SA_ERR_NULL = -1,        /* a required pointer is NULL                    */
  SA_ERR_SHAPE = -2,       /* sizes, strides or alignment not acceptable    */
  SA_ERR_DTYPE = -3,       /* KV dtype not accepted: anything but bf16, or
                              FP8 records for the 576/512 MLA shape (PR
                              32779, "Robustness": a packed FP8 pool is
                              refused, not walked with a bf16 row pitch)   */
  SA_ERR_UNSUPPORTED = -4, /* valid but not built (head dims, group size)   */
  SA_ERR_WORKSPACE = -5,   /* workspace missing or too small                */
  SA_ERR_HIP = -6          /* the HIP runtime reported an error             */
} sa_status;

/* SA_DTYPE_FP8_E4M3: K rows are 656-byte FP8 MLA records (PR 32320: the
 * pool's 656-byte FP8 rows; PR 32779, "Accuracy Tests" (c): an FP8-native
 * kernel reads the pool with its scales), accepted for the (576, 512,
 * v_in_k) MLA shape only, with kv_row_stride in bytes (>= num_kv_heads *
 * 656, a multiple of 16). Record layout (the pages do not print it; this
 * is the reading that accounts for all 656 bytes of a 576-wide row):
 * bytes 0..511 latent values in OCP FP8 E4M3 (e4m3fn), bytes 512..527 four
 * little-endian fp32 scales (scale b multiplies latent values 128b ..
 * 128b+127), bytes 528..655 64 bf16 rope values. The kernel dequantises
 * each latent value as fp32(code) * scale rounded to bf16. */
typedef enum { SA_DTYPE_BF16 = 1, SA_DTYPE_FP8_E4M3 = 2 } sa_dtype;

/* Shape of one attention call.
 *
 * Layouts (elements, row-major):
 *   q   [rows][num_q_heads][head_dim_qk]      row stride q_row_stride
 *   k   [tokens][num_kv_heads][head_dim_qk]   row stride kv_row_stride
 *   v   [tokens][num_kv_heads][head_dim_v]    row stride v_row_stride
 *       (v_in_k = 1: V is the first head_dim_v columns of each K row, the
 *        MLA latent row of PR 32779 "Speed Tests": 576 wide, 512 used as V;
 *        the v pointer is then ignored)
 *   idx [rows][topk] int32                    row stride idx_row_stride
 *   out [rows][num_q_heads][head_dim_v] fp32  row stride out_row_stride
 *   lse [rows][num_q_heads] fp32, contiguous, natural log
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 * All strides are multiples of 8 elements (4 for out); kv_row_stride and
 * v_row_stride are below 2^31 elements (a K or V row fits 4 GiB).
 * Built shapes: (head_dim_qk, head_dim_v, v_in_k) = (256, 256, 0) with a
 * group of 1..32 query heads per KV head (PR 37275: group 6 and 12 at head
 * dim 256), and (576, 512, 1) with a group of 1..32 (PR 32779: 8 heads; more
 * than 16 heads only over one latent KV head). 32 is the pages' cap on query
 * heads per rank (PR 32779, "Robustness"); more is SA_ERR_UNSUPPORTED.
 */
typedef struct {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim_qk;
  int32_t head_dim_v;
  int32_t topk;
  int32_t v_in_k;
  int32_t kv_dtype;  /* sa_dtype: SA_DTYPE_BF16, or SA_DTYPE_FP8_E4M3 for the
                        (576, 512, v_in_k) shape (kv_row_stride in bytes) */
  float sm_scale;    /* multiplies q.k before the softmax */
  int64_t q_row_stride;
  int64_t kv_row_stride;
  int64_t v_row_stride;
  int64_t idx_row_stride;
  int64_t out_row_stride;
} sa_attn_desc;

/* Per-token sparse prefill over one request
 * (sglang PR 37275, "Motivation": each query row streams up to its top-k
 * selected slots; PR 32779, "Motivation": one program per query token with
 * the head group padded into a 16-row matrix tile, online softmax held in
 * registers, no split partials).
 *
 * q, k, v, idx, out, lse  device pointers, layouts in sa_attn_desc
 * topk_len  optional device int32 [num_rows]; slot j of row t is considered
 *           only if j < topk_len[t] (PR 32779, "Robustness": the per-token
 *           valid count); NULL = all topk slots
 * num_rows  query rows (0 is allowed and launches nothing)
 * kv_len    tokens in k/v; indices are valid in [0, kv_len)
 * out, lse  fully written for every row and head.
 */
sa_status sparse_attn_prefill(const sa_attn_desc* desc, const void* q, const void* k,
                              const void* v, const int32_t* idx, const int32_t* topk_len,
                              int32_t num_rows, int32_t kv_len, float* out, float* lse,
                              hipStream_t stream);

/* Ragged chunk prefill (sglang PR 37275, "Kernel measurements": the chunk
 * kernel runs when a prompt continues a cached prefix, i.e. for each chunk
 * past the first). Request r owns query rows [cu_seqlens_q[r], cu_seqlens_q[r+1]) and
 * KV tokens [cu_seqlens_kv[r], cu_seqlens_kv[r+1]) of the packed k/v; its
 * indices are local to that range.
 *
 * cu_seqlens_q   device int32 [num_reqs + 1], non-decreasing, [0] = 0,
 *                [num_reqs] = total_q
 * cu_seqlens_kv  device int64 [num_reqs + 1], non-decreasing, [0] = 0
 * total_q        host copy of cu_seqlens_q[num_reqs] (sizes the grid, so no
 *                device read is needed; PR 37275 "Not covered" notes the
 *                device read its wrapper still did)
 * The device arrays are trusted to be consistent with total_q.
 */
sa_status sparse_attn_chunk_prefill(const sa_attn_desc* desc, const void* q, const void* k,
                                    const void* v, const int32_t* idx,
                                    const int32_t* cu_seqlens_q, const int64_t* cu_seqlens_kv,
                                    int32_t num_reqs, int32_t total_q, float* out, float* lse,
                                    hipStream_t stream);

/* Bytes of device workspace sparse_attn_union_build and
 * sparse_attn_prefill_union need for these sizes (0 on invalid sizes). */
size_t sparse_attn_union_workspace_bytes(int32_t num_rows, int32_t topk, int32_t G);

/* Union-of-G index sets (sglang PR 32779, "Modifications",
 * --dsa-triton-union): rows g*G .. g*G+G-1 form group g (the last group may
 * be short). Each distinct valid index of a group is listed once, under
 * the lowest member row that selected it, and carries one ownership bit per
 * member that selected it (bit j = j-th row of the group). The page builds
 * the set by sorting each row and searching the other rows' sorted lists;
 * here that path serves G x kv_len > 2^19, and smaller groups are built from
 * one LDS bit plane per row over [0, kv_len) instead. Both give the same
 * output.
 *
 * idx         device int32 [num_rows][topk], row stride idx_row_stride
 * union_idx   device int32 [ceil(num_rows/G)][G*topk]: row 0's distinct
 *             valid indices ascending, then row 1's new ones ascending, ...;
 *             -1 after union_len[g]
 * union_bits  device uint8 [ceil(num_rows/G)][G*topk]; 0 after union_len[g]
 * union_len   device int32 [ceil(num_rows/G)]
 * ws          device workspace of sparse_attn_union_workspace_bytes bytes,
 *             used only during the call
 * G           1..8
 * topk        1..8192 (the sort path holds a row's padded keys in 32 KB of
 *             LDS); a larger topk returns SA_ERR_SHAPE
 * Output is bit-exact and deterministic.
 */
sa_status sparse_attn_union_build(const int32_t* idx, int64_t idx_row_stride, int32_t num_rows,
                                  int32_t topk, int32_t kv_len, int32_t G, int32_t* union_idx,
                                  uint8_t* union_bits, int32_t* union_len, void* ws,
                                  size_t ws_bytes, hipStream_t stream);

/* Union-mode sparse prefill (sglang PR 32779, "Modifications"): builds the
 * union sets into ws, then one program per group gathers each union row
 * once for all G * group query rows of the group; a row's scores are masked
 * to -inf where its ownership bit is clear, so every row's result is that of
 * the per-token path over its distinct valid indices.
 * Legal iff G * group <= 32; otherwise the per-token path runs instead and
 * SA_OK_FALLBACK is returned (PR 32779, review item 1). topk is at most 8192,
 * as for sparse_attn_union_build (SA_ERR_SHAPE above).
 * ws  device workspace of sparse_attn_union_workspace_bytes(num_rows, topk, G)
 */
sa_status sparse_attn_prefill_union(const sa_attn_desc* desc, const void* q, const void* k,
                                    const void* v, const int32_t* idx, int32_t num_rows,
                                    int32_t kv_len, int32_t G, void* ws, size_t ws_bytes,
                                    float* out, float* lse, hipStream_t stream);

/* Bytes of device workspace sparse_attn_chunk_prefill_union needs (0 on
 * invalid sizes). Layout, each part 256-byte aligned, with
 * groups = ceil(total_q / G) + num_reqs and stride = align16(G * topk):
 * int32 first group id per request [num_reqs + 1], then int32 union_idx
 * [groups][stride], uint8 union_bits [groups][stride], int32 union_len
 * [groups] (the union_build layout per group, request-local indices; groups
 * listed request by request; entries past union_len[g] are not written). */
size_t sparse_attn_chunk_union_workspace_bytes(int32_t total_q, int32_t num_reqs, int32_t topk,
                                               int32_t G);

/* Union-mode ragged chunk prefill: the union of sparse_attn_prefill_union
 * (sglang PR 32779, "Modifications") over the requests of
 * sparse_attn_chunk_prefill (PR 37275, "Kernel measurements": the chunk
 * kernel). Groups are G consecutive rows inside one request (the last group
 * of a request may be short) and never span requests; indices are local to
 * their request's KV range, as in sparse_attn_chunk_prefill. Every row's
 * result is the per-token result over its distinct valid indices.
 * Legal iff G * group <= 32; otherwise the per-token ragged path runs and
 * SA_OK_FALLBACK is returned.
 * cu_seqlens_q   device int32 [num_reqs + 1], non-decreasing, last = total_q
 * cu_seqlens_kv  device int64 [num_reqs + 1], KV rows below 2^31 in total
 * ws             device workspace of sparse_attn_chunk_union_workspace_bytes,
 *                256-byte aligned, used only during the call
 * Nothing is read back to the host; the grid depends on host scalars only.
 */
sa_status sparse_attn_chunk_prefill_union(const sa_attn_desc* desc, const void* q, const void* k,
                                          const void* v, const int32_t* idx,
                                          const int32_t* cu_seqlens_q,
                                          const int64_t* cu_seqlens_kv, int32_t num_reqs,
                                          int32_t total_q, int32_t G, void* ws, size_t ws_bytes,
                                          float* out, float* lse, hipStream_t stream);

/* Decode-pool page geometry (sglang PR 32320, "Modifications"). A source
 * page holds src_page_tokens rows of row_bytes followed by src_page_tokens
 * scales of scale_bytes; a destination page holds dst_page_tokens rows then
 * their scales. src_page_tokens must be a multiple of dst_page_tokens. */
typedef struct {
  int32_t src_page_tokens;  /* 256 */
  int32_t dst_page_tokens;  /* 64 */
  int32_t row_bytes;        /* 656: one FP8 token row */
  int32_t scale_bytes;      /* 4 */
  int64_t src_page_stride;  /* bytes between source pages */
  int64_t dst_page_stride;  /* bytes between destination pages */
} sa_page_desc;

/* Page mark (PR 32320, "_page_mark_kernel"): clears mask[0..num_src_pages)
 * with a fill kernel, then sets mask[t / src_page_tokens] = 1 for every
 * index t of idx[0..num_idx) with 0 <= t < num_src_pages * src_page_tokens.
 * Other values (-1 padding, out-of-pool ids) are skipped. Same-value
 * concurrent stores, no atomics; fixed grid, no host read.
 * idx   device int32 [num_idx]
 * mask  device int8 [num_src_pages], caller-owned and reusable
 */
sa_status page_mark(const int32_t* idx, int64_t num_idx, int32_t num_src_pages,
                    int32_t src_page_tokens, int8_t* mask, hipStream_t stream);

/* Page split (PR 32320, "_page_split_kernel" with HAS_MASK): destination
 * page p*ratio + s (ratio = src_page_tokens / dst_page_tokens) receives rows
 * [s*dst_page_tokens, (s+1)*dst_page_tokens) of source page p and their
 * scales. With a mask, source pages whose mask byte is 0 are skipped and
 * their destination pages keep their previous bytes; NULL mask splits every
 * page. Destination bytes past the scales of a page are never written.
 * src   device uint8, num_src_pages pages at src_page_stride
 * dst   device uint8, num_src_pages*ratio pages at dst_page_stride
 */
sa_status page_split(const sa_page_desc* desc, const uint8_t* src, uint8_t* dst,
                     const int8_t* mask, int32_t num_src_pages, hipStream_t stream);

/* Bytes of device workspace sparse_attn_decode_paged needs (0 on invalid
 * sizes, and for batch 0). */
size_t sparse_attn_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t topk);

/* Sparse MLA decode over the split pool (sglang PR 32320: the decode
 * attention that reads the 64-token pages page_split writes, listed after
 * the split in its "Accuracy Tests" profile). Request b has one query row,
 * q[b] (num_q_heads heads of 576 bf16), and top-k pool token ids idx[b]:
 * token t is the FP8 MLA record at row t % dst_page_tokens of destination
 * page t / dst_page_tokens (the ids page_mark takes; after the split, row s
 * of source page p is row s % dst_page_tokens of destination page
 * p * ratio + s / dst_page_tokens). The result is the per-token sparse
 * attention of sparse_attn_prefill over those records (dequantised as for
 * SA_DTYPE_FP8_E4M3), with t valid iff 0 <= t < num_dst_pages *
 * dst_page_tokens. The per-token words stored after a page's records are
 * not read: each record carries the scales of all its FP8 values.
 *
 * desc   head dims (576, 512), v_in_k = 1, num_kv_heads = 1, num_q_heads
 *        1..32, kv_dtype SA_DTYPE_FP8_E4M3, kv_row_stride = 656; topk,
 *        sm_scale and the q, idx, out row strides as for prefill
 * pages  dst_page_tokens (a power of two), row_bytes = 656, scale_bytes,
 *        dst_page_stride (>= dst_page_tokens * (row_bytes + scale_bytes), a
 *        multiple of 16, < 2^32); the source fields are not used
 * pool   device uint8, num_dst_pages pages at dst_page_stride, 16-byte
 *        aligned; num_dst_pages * dst_page_tokens < 2^31
 * topk_len  optional device int32 [batch], as for prefill
 * ws     device workspace of sparse_attn_decode_workspace_bytes(batch,
 *        num_q_heads, topk) bytes, 256-byte aligned, used only during the
 *        call: each request's 16-slot tiles are dealt round-robin to S
 *        ranges, one workgroup per (request, range) writes that range's
 *        normalised O and LSE there, and a second kernel merges them
 * out    [batch][num_q_heads][512] fp32, lse [batch][num_q_heads] fp32,
 *        fully written (a request with no valid slot gets O = 0, LSE = -inf)
 */
sa_status sparse_attn_decode_paged(const sa_attn_desc* desc, const sa_page_desc* pages,
                                   const void* q, const uint8_t* pool, int32_t num_dst_pages,
                                   const int32_t* idx, const int32_t* topk_len, int32_t batch,
                                   void* ws, size_t ws_bytes, float* out, float* lse,
                                   hipStream_t stream);

/* Bytes of the static device scratch behind sparse_attn_decode_paged_noalloc
 * (each GPU the library runs on holds its own copy until the process ends). */
#define SA_DECODE_SCRATCH_BYTES ((size_t)32 << 20)

/* sparse_attn_decode_paged without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation). Same arguments, results
 * and errors as sparse_attn_decode_paged, which it shares its kernels with;
 * the partial results live in a static device array of
 * SA_DECODE_SCRATCH_BYTES per GPU instead of `ws`.
 *
 * A call whose sparse_attn_decode_workspace_bytes(batch, num_q_heads, topk)
 * exceeds SA_DECODE_SCRATCH_BYTES returns SA_ERR_WORKSPACE before anything
 * is launched (at topk 2048 a request head takes 16 ranges of 2052 bytes,
 * so batch x num_q_heads up to 1022 fits). The first call on a device looks
 * up that device's scratch address (SA_ERR_HIP if the runtime refuses).
 * Calls on one GPU share its scratch, which keeps the last call's contents:
 * calls that overlap on one GPU (different streams, or different threads)
 * race and must be serialised by the caller. Nothing is allocated or freed;
 * no memset is enqueued.
 */
sa_status sparse_attn_decode_paged_noalloc(const sa_attn_desc* desc, const sa_page_desc* pages,
                                           const void* q, const uint8_t* pool,
                                           int32_t num_dst_pages, const int32_t* idx,
                                           const int32_t* topk_len, int32_t batch, float* out,
                                           float* lse, hipStream_t stream);

/* Indexer top-k selection (sglang PR 37275, "Motivation": each query row
 * gets a budget of 2051 token slots, its top-k plus the compression ratio
 * minus one, and fewer when it sees fewer tokens). Row t keeps the k
 * largest of its first n_t scores, n_t = row_len[t] clamped to [0, kv_len]
 * (kv_len when row_len is NULL); a larger score wins, equal scores go to the
 * lower position, and -0 ties with +0. The kept positions are written to
 * idx[t] in ascending order. A row with n_t <= k writes 0 .. n_t - 1, then
 * -1 up to k (the padding the attention entry points skip).
 *
 * scores  device fp32 [num_rows][score_row_stride], score_row_stride >=
 *         kv_len; no NaN (rows that start 16-byte aligned are read with
 *         16-byte loads, others one float at a time)
 * row_len optional device int32 [num_rows]
 * idx     device int32 [num_rows][idx_row_stride], idx_row_stride >= k;
 *         exactly k entries of every row are written
 * Deterministic; one workgroup per row, no workspace, no host read.
 */
sa_status indexer_topk(const float* scores, int64_t score_row_stride, const int32_t* row_len,
                       int32_t num_rows, int32_t kv_len, int32_t k, int32_t* idx,
                       int64_t idx_row_stride, hipStream_t stream);

/* FP8 MLA records to bf16 rows (PR 32779, "Accuracy Tests" (c): the kernel
 * measured there reads rows that were dequantised to bf16 before it ran).
 * For every token t < num_tokens with mask NULL or mask[t] != 0 and every KV
 * head h < num_kv_heads, writes the 576 bf16 values of record (t, h) to
 * out + t * out_row_stride + h * 576: latent value i as fp32(code_i) times
 * its block scale, rounded to nearest-even bf16 (the reading every FP8
 * attention path uses), then the 64 rope values unchanged. Other rows of
 * out are not written, so a bf16 attention call over out gives the same
 * result as the FP8 call over pool for index rows whose valid tokens are
 * all marked. page_mark with src_page_tokens = 1 marks the tokens a step's
 * index rows reference.
 * pool  device uint8 [num_tokens][pool_row_stride] records (record layout
 *       under SA_DTYPE_FP8_E4M3), pool_row_stride >= num_kv_heads * 656, a
 *       multiple of 16
 * mask  optional device int8 [num_tokens]
 * out   device bf16 [num_tokens][out_row_stride] (elements), out_row_stride
 *       >= num_kv_heads * 576, a multiple of 8; caller-owned
 * One wavefront per (token, head), no workspace, no host read.
 */
sa_status sparse_attn_fp8_records_to_bf16(const uint8_t* pool, int64_t pool_row_stride,
                                          int32_t num_tokens, int32_t num_kv_heads,
                                          const int8_t* mask, void* out, int64_t out_row_stride,
                                          hipStream_t stream);

/* Host-only check of an attention descriptor, as sparse_attn_prefill (G=1)
 * or sparse_attn_prefill_union (G>1) would do before launching. Touches no
 * device. Returns SA_OK, SA_OK_FALLBACK (union tile illegal) or an error. */
/* Measurement aid, not part of the attention path: the K/V row gathers that
 * the head-dim-256 per-token kernels issue, without their arithmetic, so a
 * benchmark can compare a kernel's gather rate with what the gather stream
 * alone sustains on the device. One wavefront per index row walks its slots
 * in tiles of 16 and reads 512 bytes of K and of V per valid slot in 16-byte
 * pieces through row buffer descriptors (the attention kernels' loads);
 * slots outside [0, kv_len) read zeros without touching memory. out[r][l]
 * is lane l's XOR of the 32-bit words it read for row r.
 * k, v  device bf16 [kv_len][256], 512-byte rows, kv_len * 512 <= 2^31
 * idx   device int32 [num_rows][topk], rows contiguous
 * out   device uint32 [num_rows][64]
 * eight_waves  1: 64 KB of LDS per four-wave workgroup, so at most eight
 *       waves per CU (the attention kernels' occupancy); 0: as many as the
 *       registers allow
 * Host checks only; no workspace, no host read. */
sa_status sa_probe_gather(const void* k, const void* v, int32_t kv_len, const int32_t* idx,
                          int32_t num_rows, int32_t topk, int32_t eight_waves, uint32_t* out,
                          hipStream_t stream);

int sa_validate_attn(const sa_attn_desc* desc, int32_t G);

/* Message for the calling thread's last error ("" if none). */
const char* sa_last_error(void);

/* Number of successful calls per entry point since load, to rule out silent
 * no-ops (PR 32779, "Speed Tests": invocations were counted). */
typedef enum {
  SA_ENTRY_PREFILL = 0,
  SA_ENTRY_CHUNK_PREFILL = 1,
  SA_ENTRY_UNION_BUILD = 2,
  SA_ENTRY_PREFILL_UNION = 3,
  SA_ENTRY_PAGE_MARK = 4,
  SA_ENTRY_PAGE_SPLIT = 5,
  SA_ENTRY_CHUNK_PREFILL_UNION = 6,
  SA_ENTRY_DECODE_PAGED = 7,
  SA_ENTRY_INDEXER_TOPK = 8,
  SA_ENTRY_DECODE_PAGED_NOALLOC = 9,
  SA_ENTRY_FP8_RECORDS_TO_BF16 = 10,
  SA_ENTRY_COUNT = 11
} sa_entry;
uint64_t sa_call_count(int32_t entry);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
