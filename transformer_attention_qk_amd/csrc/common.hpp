// Shared device helpers for the gfx950 kernels of libattn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// bf16 <-> fp32. The narrowing conversion rounds to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }
__device__ __forceinline__ bf16 f2bf(float x) { return (bf16)x; }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 p;
  p[0] = (bf16)lo;
  p[1] = (bf16)hi;
  return __builtin_bit_cast(uint32_t, p);
}

// Widen the two bf16 halves of a 32-bit word (low half = lower address) to fp32 exactly.
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace attn
