// Shared device definitions for the gfx950 decode kernels: vector types,
// MFMA wrappers and small helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// 32x32 output, K = 16 per instruction. Lane l holds A[m = l%32][k = 8(l/32)+i]
// and B[k = 8(l/32)+i][n = l%32], i = 0..7; the accumulator register r of
// lane l is D[8(r/4) + 4(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16 output, K = 32 per instruction. Lane l holds A[m = l%16][k = 8(l/16)+i]
// and B[k = 8(l/16)+i][n = l%16]; accumulator register r of lane l is
// D[4(l/16) + r][l%16].
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}


__device__ __forceinline__ float wave_max32(float x) {
  // combine lane l with lane l ^ 32
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_sum32(float x) { return x + __shfl_xor(x, 32); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

}  // namespace mla
