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

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace lra
