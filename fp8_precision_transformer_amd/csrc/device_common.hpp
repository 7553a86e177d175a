// Device helpers for the gfx950 kernels: FP8/bf16 conversions, scale rule, reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace te {

constexpr float kE4M3Max = 448.0f;    // 1.75 * 2^8
constexpr float kE5M2Max = 57344.0f;  // 1.75 * 2^15
constexpr float kFltMax = 3.402823466e+38f;

template <bool E5M2>
struct Fp8Traits {
  static constexpr float max = E5M2 ? kE5M2Max : kE4M3Max;
  static constexpr int emax_elem = E5M2 ? 15 : 8;  // exponent of the largest power of two
};

// bf16 halves of a 32-bit word -> fp32 (exact widening)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Saturate to +-max; NaN passes through unchanged (the comparison is false for NaN),
// so the hardware convert sees only in-range values or NaN.
template <bool E5M2>
__device__ __forceinline__ float saturate(float v) {
  constexpr float M = Fp8Traits<E5M2>::max;
  return (__builtin_fabsf(v) > M) ? __builtin_copysignf(M, v) : v;
}

// Four in-range fp32 values -> four FP8 codes (byte 0 = a), round to nearest even
// via the gfx950 convert (OCP E4M3 / E5M2).
template <bool E5M2>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  int w;
  if constexpr (E5M2) {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  }
  return (uint32_t)w;
}

// Scaled saturating cast of four values.
template <bool E5M2>
__device__ __forceinline__ uint32_t quant4(float a, float b, float c, float d, float s) {
  return cvt4<E5M2>(saturate<E5M2>(__fmul_rn(a, s)), saturate<E5M2>(__fmul_rn(b, s)),
                    saturate<E5M2>(__fmul_rn(c, s)), saturate<E5M2>(__fmul_rn(d, s)));
}

// scale = fl32(fp8_max / amax) * 2^-margin; overflow -> FLT_MAX; a bad amax
// (0, negative, NaN or Inf) returns `fallback`.  Division is IEEE correctly
// rounded (built with -fhip-fp32-correctly-rounded-divide-sqrt).
__device__ __forceinline__ float scale_from_amax(float amax, float fp8_max, int margin,
                                                 float fallback) {
  if (!(amax > 0.0f) || !__builtin_isfinite(amax)) return fallback;
  float s = fp8_max / amax;
  if (!__builtin_isfinite(s)) s = kFltMax;
  return margin ? __builtin_ldexpf(s, -margin) : s;
}

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN with the sign kept.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace te
