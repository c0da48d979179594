// Device-side helpers for gfx950 (CDNA4): vector types of the MFMA builtins,
// bf16 packing, raw loads and cross-lane reductions over a 64-wide wavefront.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lra {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;  // 16x16x32 operand
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;     // 16x16x16 operand
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// MFMA wrappers. Lane layout (gfx950, 64 lanes, l = lane):
//   A operand: row l%16, k-group l/16;  B operand: column l%16, k-group l/16;
//   accumulator: column l%16, rows 4*(l/16) + i for i = 0..3.
// The k slots inside a group are paired between A and B by position, so any
// fixed assignment of logical k to (group, slot) used for both is valid.
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(i16x4 a, i16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mfma32h(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ i16x4 as_i16x4(uint2 u) { return __builtin_bit_cast(i16x4, u); }
__device__ __forceinline__ bf16x8 cat8(uint2 lo, uint2 hi) {
  return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Round-to-nearest-even fp32 -> bf16, two at a time (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  return make_uint2(pack_bf16(a, b), pack_bf16(c, d));
}
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// Plain global loads of raw bits (vector loads; never the scalar data cache
// for writes anywhere in this library). The pointer is taken as a global
// (address space 1) pointer so no flat access is emitted.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld16(const void* p) {
  return __builtin_bit_cast(uint4, *(__attribute__((address_space(1))) const u32x4_t*)(p));
}
__device__ __forceinline__ uint2 ld8(const void* p) {
  return __builtin_bit_cast(uint2, *(__attribute__((address_space(1))) const u32x2_t*)(p));
}
__device__ __forceinline__ float4 ldf4(const float* p) {
  return __builtin_bit_cast(float4, *(__attribute__((address_space(1))) const f32x4*)(p));
}
__device__ __forceinline__ float2 ldf2(const float* p) {
  return __builtin_bit_cast(float2, *(__attribute__((address_space(1))) const f32x2_t*)(p));
}

// Buffer resources: a raw buffer load whose byte offset is at or past the
// resource's byte count returns zero without a memory access, so masked
// lanes take kOob instead of a branch.
constexpr int kOob = 0x7ffffff0;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bld16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
__device__ __forceinline__ uint2 bld8(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0));
}
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Byte offsets, within one cache block of an L_k pool, of the low-rank key
// row pieces a matrix operand takes. The pool keeps chunks of 8 ranks: rank j
// of token t at ((j/8)*16 + t)*8 + j%8, so the 16 tokens' rows of one chunk
// are one contiguous 256-byte run and a wave's load of 16-byte pieces reads
// whole runs (measured on MI355X: a quarter-wave reading 16 rows 128 bytes
// apart moves L2-resident data 2.6 times slower).
//   16-byte piece: ranks 32kc + 8g .. +7 of token t
__device__ __forceinline__ int lk_chunk_off32(int t, int g, int kc) { return ((4 * kc + g) * 16 + t) * 16; }
//   8-byte piece: ranks 4g .. 4g+3 of token t
__device__ __forceinline__ int lk_chunk_off16(int t, int g) { return (((g >> 1) * 16 + t) * 8 + 4 * (g & 1)) * 2; }

// Load of a value that is the same for the whole wave from memory the kernel
// never writes: read through the constant address space, so a wave-uniform
// address becomes a scalar load (counted apart from the vector loads in
// flight, so waiting for it never waits for them).
template <typename T>
__device__ __forceinline__ T sload(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

// Reductions over the 4 rows of 16 lanes (lanes l, l^16, l^32, l^48) that
// hold the same accumulator column, with the gfx950 row-swap moves (plain
// VALU data movement, no LDS round trip). Each step combines a lane's value
// with the partner row's, in an order that is the same for both partners.
__device__ __forceinline__ float wave_max_across_groups(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float wave_sum_across_groups(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Reductions over the 64 lanes of a wave without an LDS round trip: DPP moves
// within rows of 16 lanes (lanes 1 and 2 apart, then mirrored within 8 and
// within 16), then the gfx950 row swaps across rows; every lane gets the result.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kRowHalfMirror = 0x141, kRowMirror = 0x140;
__device__ __forceinline__ float wave_max64(float v) {
  v = fmaxf(v, dpp<kQuadXor1>(v));
  v = fmaxf(v, dpp<kQuadXor2>(v));
  v = fmaxf(v, dpp<kRowHalfMirror>(v));
  v = fmaxf(v, dpp<kRowMirror>(v));
  return wave_max_across_groups(v);
}
__device__ __forceinline__ float wave_sum64(float v) {
  v += dpp<kQuadXor1>(v);
  v += dpp<kQuadXor2>(v);
  v += dpp<kRowHalfMirror>(v);
  v += dpp<kRowMirror>(v);
  return wave_sum_across_groups(v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Rows of 16 tokens (a V^T dim row, an L_v rank row) read 16 bytes per lane:
// lane (c, g) of the wave holds tokens 8(g&1) .. +7 of row 16(2t + (g>>1)) + c
// for a pair of 16-row tiles t (a = its tokens +0..3, b = +4..7). Two row
// swaps of 16 lanes and two of 32 lanes turn that into the 16x16x16 operands
// of the two tiles (lane (c, g): tokens 4g .. 4g+3 of row c): a for tile 2t,
// b for tile 2t + 1. One 16-byte load moves twice the bytes of an 8-byte one
// at the same issue cost.
__device__ __forceinline__ void token_rows_to_operands(uint2& a, uint2& b) {
  const auto x = __builtin_amdgcn_permlane16_swap(a.x, b.x, false, false);
  const auto y = __builtin_amdgcn_permlane16_swap(a.y, b.y, false, false);
  const auto x2 = __builtin_amdgcn_permlane32_swap(x[0], x[1], false, false);
  const auto y2 = __builtin_amdgcn_permlane32_swap(y[0], y[1], false, false);
  a = make_uint2(x2[0], y2[0]);
  b = make_uint2(x2[1], y2[1]);
}
// Byte offset of lane (c, g)'s 16-byte piece of tile pair t, rows of 16 tokens.
__device__ __forceinline__ int token_rows_off(int t, int c, int g) {
  return ((16 * (2 * t + (g >> 1)) + c) * 16 + 8 * (g & 1)) * 2;
}

// Offset of element (row, col) of a bf16 matrix of `nrows` rows and W
// columns staged in LDS for MFMA operand reads, in which lane l reads row
// l % 16 (plus a multiple of 16) at column group l / 16. Rows are not padded;
// the pieces of a row are permuted by row bits so that one read instruction
// hits distinct banks of the 64 (measured on MI355X):
//   W = 16: 8-byte reads (4 columns per lane). A pass serves 32 lanes; rows 8
//           apart share banks, so the second 8 rows take the other half of
//           the row.
//   W = 32 or 64: 16-byte reads (8 columns per lane). A pass serves lanes 0-7
//           with 16-23 (and so on). The matrix is kept as W / 32 slabs of 32
//           columns (so the slab of a read is an immediate offset), and rows
//           4 apart, which share banks within a slab, take the other half of
//           the row.
template <int W>
__device__ __forceinline__ int tile_off(int row, int col, int nrows) {
  static_assert(W == 16 || W == 32 || W == 64, "tile width");
  if constexpr (W == 16) return row * 16 + 4 * ((col >> 2) ^ (((row >> 3) & 1) << 1)) + (col & 3);
  else return (col >> 5) * nrows * 32 + row * 32 + 8 * (((col >> 3) & 3) ^ (((row >> 2) & 1) << 1)) + (col & 7);
}

}  // namespace lra
