// Device helpers shared by the fp8mi kernels (gfx950 / CDNA4, wave64).
//
// FP8 encoding follows "4.2 Hopper I — Transformer Engine·FP8" §4.2.4
// (round_to_fp8 of the scaled tensor; large values saturate) on the OCP
// formats the page names in §4.2.8.  The conversion itself is the gfx950
// V_CVT_PK_FP8_F32 / V_CVT_PK_BF8_F32 instruction (OCP E4M3 / E5M2).  Checked
// against the CPU oracle on every bf16 bit pattern (and on the same patterns
// scaled into the subnormal range), the instruction already rounds to
// nearest even with gradual underflow and keeps the sign of zero; it differs
// from the rule only on
//   * values beyond max and +-Inf (E4M3 gives a NaN code, E5M2 an Inf code):
//     the input is clamped to [-max, max] first (one V_MED3_F32), and
//   * NaN (it returns one fixed code): NaN inputs are rewritten to sign|0x7F
//     on a separate path that only runs when a NaN is present.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8mi {

enum : int { kE4M3 = 0, kE5M2 = 1 };
enum : int { kF32 = 0, kBF16 = 1 };

template <int FMT>
struct Fp8Traits;
template <>
struct Fp8Traits<kE4M3> {
  static constexpr uint32_t max_bits = 0x43E00000u;  // 448.0f
  static constexpr float max_value = 448.0f;
};
template <>
struct Fp8Traits<kE5M2> {
  static constexpr uint32_t max_bits = 0x47600000u;  // 57344.0f
  static constexpr float max_value = 57344.0f;
};

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }

// Clamp |p| to max keeping the sign; NaN passes through unchanged.
template <int FMT>
__device__ __forceinline__ float sat_clamp(float p) {
  const uint32_t u = f2u(p);
  uint32_t m = u & 0x7FFFFFFFu;
  m = (m > 0x7F800000u) ? m : (m < Fp8Traits<FMT>::max_bits ? m : Fp8Traits<FMT>::max_bits);
  return u2f(m | (u & 0x80000000u));
}

// 1 if |p| > max and p is not NaN (Inf counts): the saturation counter's rule.
template <int FMT>
__device__ __forceinline__ uint32_t is_saturated(float p) {
  const uint32_t m = f2u(p) & 0x7FFFFFFFu;
  return (m > Fp8Traits<FMT>::max_bits) & (m <= 0x7F800000u);
}

// Convert two fp32 values into the low (HI = false) or high (HI = true) 16 bits of `old`.
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t cvt_pk(float a, float b, uint32_t old) {
  if constexpr (FMT == kE4M3)
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
  else
    return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)old, HI);
}

template <int FMT>
__device__ __forceinline__ float clamp_to_max(float p) {
  return __builtin_amdgcn_fmed3f(p, -Fp8Traits<FMT>::max_value, Fp8Traits<FMT>::max_value);
}

// Encode four scaled fp32 values that are known not to be NaN: byte i = value i.
template <int FMT>
__device__ __forceinline__ uint32_t encode4_finite(float p0, float p1, float p2, float p3) {
  const uint32_t w = cvt_pk<FMT, false>(clamp_to_max<FMT>(p0), clamp_to_max<FMT>(p1), 0u);
  return cvt_pk<FMT, true>(clamp_to_max<FMT>(p2), clamp_to_max<FMT>(p3), w);
}

// Encode four scaled fp32 values of any kind (the full rule, NaN included).
template <int FMT>
__device__ __forceinline__ uint32_t encode4(float p0, float p1, float p2, float p3) {
  uint32_t w = cvt_pk<FMT, false>(sat_clamp<FMT>(p0), sat_clamp<FMT>(p1), 0u);
  w = cvt_pk<FMT, true>(sat_clamp<FMT>(p2), sat_clamp<FMT>(p3), w);
  const uint32_t u0 = f2u(p0), u1 = f2u(p1), u2 = f2u(p2), u3 = f2u(p3);
  const uint32_t sgn = ((u0 >> 24) & 0x80u) | ((u1 >> 16) & 0x8000u) | ((u2 >> 8) & 0x800000u) |
                       (u3 & 0x80000000u);
  const uint32_t nan = (((u0 & 0x7FFFFFFFu) > 0x7F800000u) ? 0x000000FFu : 0u) |
                       (((u1 & 0x7FFFFFFFu) > 0x7F800000u) ? 0x0000FF00u : 0u) |
                       (((u2 & 0x7FFFFFFFu) > 0x7F800000u) ? 0x00FF0000u : 0u) |
                       (((u3 & 0x7FFFFFFFu) > 0x7F800000u) ? 0xFF000000u : 0u);
  return (w & ~nan) | sgn | (nan & 0x7F7F7F7Fu);
}

// Single-value encoder for ragged tails.
template <int FMT>
__device__ __forceinline__ uint8_t encode1(float p) {
  return (uint8_t)(encode4<FMT>(p, 0.0f, 0.0f, 0.0f) & 0xFFu);
}

// Widen the i-th bf16 of a packed pair word (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return u2f(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return u2f(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += (uint32_t)__shfl_xor((int)v, off, 64);
  return v;
}

// Correctly rounded fp32 scale = MAX / m and its inverse, per the rule shared by
// the delayed and the per-block scaling: valid only when 0 < m < Inf and the
// quotient is finite.  HIP's fp32 division is IEEE correctly rounded here
// (the library is built without fast-math / approximate-division flags).
template <int FMT>
__device__ __forceinline__ bool scale_from_amax_bits(uint32_t m_bits, float* s, float* s_inv) {
  if (m_bits == 0u || m_bits >= 0x7F800000u) return false;
  const float q = Fp8Traits<FMT>::max_value / u2f(m_bits);
  if (!(f2u(q) < 0x7F800000u) || q == 0.0f) return false;
  *s = q;
  *s_inv = 1.0f / q;
  return true;
}

}  // namespace fp8mi
