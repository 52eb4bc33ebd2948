// Device-side helpers shared by the gfx950 kernels: bf16 bit handling,
// MFMA operand types, wave-level exchanges and the workspace geometry
// that host and device agree on.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kve {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bits, round to nearest even (inputs are finite here).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 32x32x16 bf16 MFMA, fp32 accumulate.  Operand lane layout (wave64):
//   A: lane l holds A[m = l%32][k = 8*(l/32) .. +8]
//   B: lane l holds B[k = 8*(l/32) .. +8][n = l%32]
//   C: lane l, register r holds C[m = 8*(r/4) + 4*(l/32) + r%4][n = l%32]
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16 MFMA, fp32 accumulate.  Operand lane layout (wave64):
//   A: lane l holds A[m = l%16][k = 8*(l/16) .. +8]
//   B: lane l holds B[k = 8*(l/16) .. +8][n = l%16]
//   C: lane l, register r holds C[m = 4*(l/16) + r][n = l%16]
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Value held by lane (l ^ 32).
__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32, 64); }

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Order-preserving map of fp32 bits to uint32 (larger float -> larger key);
// -0 and +0 map to the same key; every NaN maps to 0, below -inf.
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Same for fp64 (callers never pass NaN).
__device__ __forceinline__ uint64_t f64_order_key(double f) {
  uint64_t u = static_cast<uint64_t>(__double_as_longlong(f));
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

}  // namespace kve
