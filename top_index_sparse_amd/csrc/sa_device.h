// Device helpers shared by the gfx950 kernels: vector types, DPP wave
// scans, 16-byte loads, bf16 packing, MFMA wrappers, XCD-aware block
// remapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;

// Inclusive prefix sums within each row of 16 lanes (DPP row shifts; lanes
// shifted in from outside the row add 0).
__device__ __forceinline__ uint32_t row_scan16(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);   // row_shr:8
  return x;
}

// Inclusive prefix sums over the wave's 64 lanes: the rows' own scans, then
// row_bcast:15 adds row 0's total to row 1 and row 2's to row 3, and
// row_bcast:31 adds the total of rows 0-1 to rows 2 and 3 (the other rows
// are masked off and add 0).
__device__ __forceinline__ uint32_t wave_scan64(uint32_t x) {
  x = row_scan16(x);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);
  return x;
}


__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ void st16(void* p, f32x4_t v) {
  *reinterpret_cast<f32x4_t*>(p) = v;
}

// Row gathers through a structured buffer descriptor (MUBUF idxen + offen):
// 16 bytes at base + row * stride + off. Measured on gfx950: the byte offset
// row * stride + off is a 32-bit quantity (it wraps past 4 GiB), the stride
// field holds 14 bits, and a row >= num_records reads zeros without touching
// memory, which is how invalid slots are served. Windows are kept within
// 2 GiB of base, where no reading of the offset's top bit matters.
typedef __amdgpu_buffer_rsrc_t rows_rsrc_t;
__device__ u32x4_t sa_struct_buffer_load_v4(rows_rsrc_t r, int row, int off, int soff, int aux)
    __asm("llvm.amdgcn.struct.ptr.buffer.load.v4i32");

constexpr int kNoRow = 0x7fffffff;         // a row index every window treats as absent
constexpr uint32_t kMaxRowStride = 16383;  // bytes (14-bit field)

__device__ __forceinline__ rows_rsrc_t rows_rsrc(const void* base, uint32_t stride) {
  // num_records = kNoRow: rows are bounded by the kernel's own checks; 0x20000
  // is gfx9's untyped 32-bit data format word.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)stride, kNoRow,
                                           0x00020000);
}

__device__ u32x2_t sa_struct_buffer_load_v2(rows_rsrc_t r, int row, int off, int soff, int aux)
    __asm("llvm.amdgcn.struct.ptr.buffer.load.v2i32");
__device__ __forceinline__ u32x2_t ld_row8(rows_rsrc_t r, int row, int off) {
  return sa_struct_buffer_load_v2(r, row, off, 0, 0);
}

__device__ __forceinline__ u32x4_t ld_row16(rows_rsrc_t r, int row, int off) {
  return sa_struct_buffer_load_v4(r, row, off, 0, 0);
}

// x where bit `pos` of `bits` is set, else -inf: the sign-extended one-bit
// field selects between the two bit patterns (v_bfe_i32, v_bitop3_b32).
__device__ __forceinline__ float keep_if_bit(float x, int bits, int pos) {
  const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe(bits, pos, 1);
  return __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, x) & m) | (0xff800000u & ~m));
}

// Lane L's value of each row of 16 added to y in one DPP operation
// (row_newbcast:L on the add's first operand).
template <int L>
__device__ __forceinline__ int row_bcast_add(int v, int y) {
  return __builtin_amdgcn_update_dpp(0, v, 0x150 + L, 0xf, 0xf, true) + y;
}

// Two fp32 values to packed bf16 (round to nearest even), low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t h = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}

// bf16 element e (0..7) of a 16-byte chunk.
__device__ __forceinline__ uint32_t bf16_elem(u32x4_t v, int e) {
  const uint32_t w = v[e >> 1];
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// Pack element e of four chunks into the 4 x bf16 operand of a K=16 MFMA:
// one byte permute per output register (v_perm_b32 picks bytes 0-3 from its
// second source and 4-7 from its first).
__device__ __forceinline__ i16x4_t gather_col4(u32x4_t c0, u32x4_t c1, u32x4_t c2, u32x4_t c3,
                                               int e) {
  const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
  const uint32_t lo = __builtin_amdgcn_perm(c1[e >> 1], c0[e >> 1], sel);
  const uint32_t hi = __builtin_amdgcn_perm(c3[e >> 1], c2[e >> 1], sel);
  return __builtin_bit_cast(i16x4_t, (u32x2_t){lo, hi});
}

// Lane 4q+I's value in every lane of quad q (DPP quad_perm [I, I, I, I]);
// all lanes must be active.
template <int I>
__device__ __forceinline__ int quad_bcast(int v) {
  return __builtin_amdgcn_mov_dpp(v, I * 0x55, 0xf, 0xf, false);
}

// Max and sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one per row of
// 16), in every lane, with gfx950's row-swap permutes instead of an LDS
// round trip. Both halves of a swap pair combine the same two operands in
// the same order, so every lane gets the same bits.
__device__ __forceinline__ void swap_pair(const u32x2_t r, float& a, float& b) {
  const uint32_t x = r[0], y = r[1];   // (bit casts of vector elements read element 0)
  a = __builtin_bit_cast(float, x);
  b = __builtin_bit_cast(float, y);
}

// max(a, b) as one v_max_f32: fmaxf first quiets each operand that the
// compiler cannot prove canonical (a cross-lane result, a loop-carried
// value), one extra instruction per operand. Scores here are never NaN.
__device__ __forceinline__ float max2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ float max4(float a, float b, float c, float d) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return max2(r, d);
}

__device__ __forceinline__ float rows_max4(float v) {
  float a, b;
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  swap_pair(__builtin_bit_cast(u32x2_t, __builtin_amdgcn_permlane16_swap(u, u, false, false)), a, b);
  v = max2(a, b);
  const uint32_t w = __builtin_bit_cast(uint32_t, v);
  swap_pair(__builtin_bit_cast(u32x2_t, __builtin_amdgcn_permlane32_swap(w, w, false, false)), a, b);
  return max2(a, b);
}

__device__ __forceinline__ float rows_sum4(float v) {
  float a, b;
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  swap_pair(__builtin_bit_cast(u32x2_t, __builtin_amdgcn_permlane16_swap(u, u, false, false)), a, b);
  v = a + b;
  const uint32_t w = __builtin_bit_cast(uint32_t, v);
  swap_pair(__builtin_bit_cast(u32x2_t, __builtin_amdgcn_permlane32_swap(w, w, false, false)), a, b);
  return a + b;
}

// Lane L's value in every lane of its row of 16 (DPP row_newbcast:L).
template <int L>
__device__ __forceinline__ int row_bcast(int v) {
  return __builtin_amdgcn_mov_dpp(v, 0x150 + L, 0xf, 0xf, false);
}

// The values of lanes 0, 4, 8, 12 of each row of 16.
__device__ __forceinline__ void row_bcast4(int v, int out[4]) {
  out[0] = row_bcast<0>(v);
  out[1] = row_bcast<4>(v);
  out[2] = row_bcast<8>(v);
  out[3] = row_bcast<12>(v);
}

// 64-bit value from its two halves (a register pair, no arithmetic).
__device__ __forceinline__ uint64_t join64(int lo, int hi) {
  return __builtin_bit_cast(uint64_t, (u32x2_t){(uint32_t)lo, (uint32_t)hi});
}

__device__ __forceinline__ void quad_bcast4(int v, int out[4]) {
  out[0] = quad_bcast<0>(v);
  out[1] = quad_bcast<1>(v);
  out[2] = quad_bcast<2>(v);
  out[3] = quad_bcast<3>(v);
}

// D = A(16x32) * B(32x16) + C; lane l holds A row l%16, B column l%16, each
// with k = 8*(l/16) .. 8*(l/16)+7; C/D lane l holds column l%16, rows
// 4*(l/16) .. 4*(l/16)+3.
__device__ __forceinline__ f32x4_t mfma_16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// D = A(16x16) * B(16x16) + C with k = 4*(l/16) .. 4*(l/16)+3 per lane.
__device__ __forceinline__ f32x4_t mfma_16x16x16(i16x4_t a, i16x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Workgroups are dealt round-robin to the 8 XCDs (each with its own L2).
// Remap so that each XCD runs chunks of kXcdChunk consecutive logical blocks
// (neighbouring rows share most of their slots, so they should share an
// L2), with the chunks dealt round-robin to the XCDs so every XCD gets work
// from the whole range (rows with short visible prefixes carry less work).
// The last, partial round of chunks is split into contiguous bands.
constexpr int kXcdChunk = 32;   // of 16, 32, 64, 128, 256 measured, 32 fastest

__device__ __forceinline__ int xcd_remap(int b, int nblk) {
  constexpr int X = 8;
  const int xcd = b % X, local = b / X;
  const int rounds = nblk / (X * kXcdChunk);
  if (local < rounds * kXcdChunk)
    return (local / kXcdChunk) * (X * kXcdChunk) + xcd * kXcdChunk + local % kXcdChunk;
  const int tail = nblk - rounds * X * kXcdChunk;
  const int q = tail / X, r = tail % X;
  return rounds * X * kXcdChunk + xcd * q + (xcd < r ? xcd : r) + (local - rounds * kXcdChunk);
}

}  // namespace sa
