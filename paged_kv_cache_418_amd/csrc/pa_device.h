// Device helpers for the gfx950 kernels: element conversions, wave shuffles and
// matrix-core operand types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN with its sign.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 -> packed bf16 pair (low half = a), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
// Two fp32 values rounded to fp16 (nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, f16x2_t));
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// fp32 -> OCP E4M3FN code: round to nearest even, |x| >= 464 (including inf)
// saturates to 448, NaN -> 0x7F with the sign kept.  Integer work on the fp32
// bit pattern: above 2^-6 keep 3 mantissa bits; below, count quanta of 2^-9.
__device__ __forceinline__ uint8_t f32_to_e4m3(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return (uint8_t)(sign | 0x7Fu);
  if (a >= 0x43E80000u) return (uint8_t)(sign | 0x7Eu);  // >= 464.0
  uint32_t exp = a >> 23;
  uint32_t code;
  if (exp >= 121u) {  // >= 2^-6: normal E4M3
    uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
    code = r - (120u << 3);
  } else if (exp == 0u) {  // fp32 subnormal: far below 2^-10
    code = 0u;
  } else {
    uint32_t m24 = (a & 0x7FFFFFu) | 0x800000u;  // value = m24 * 2^(exp-150)
    uint32_t shift = 141u - exp;                 // quanta of 2^-9: m24 * 2^(exp-141)
    if (shift > 25u) {
      code = 0u;
    } else {
      uint32_t q = m24 >> shift;
      uint32_t rem = m24 & ((1u << shift) - 1u);
      uint32_t half = 1u << (shift - 1u);
      if (rem > half || (rem == half && (q & 1u))) ++q;
      code = q;
    }
  }
  return (uint8_t)(sign | code);
}

// Four E4M3 codes (one dword) -> four bf16 values (exact: E4M3 values are a
// subset of bf16), two per gfx950 fp8 -> bf16 pair conversion at unit scale;
// code i of the dword lands in bf16 lane i (low half first).
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t w) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Calls f(integral_constant<int, i>) for i = I .. N-1 (unrolled at compile time).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}


}  // namespace pa
