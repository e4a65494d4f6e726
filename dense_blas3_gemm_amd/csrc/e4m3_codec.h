// OCP E4M3 ("E4M3FN": 1 sign, 4 exponent bits biased by 7, 3 mantissa bits; no
// infinities, S.1111.111 is NaN, largest finite 448, subnormals m * 2^-9) to and from
// fp32 on the device, exact integer arithmetic.  Used by the quantiser and by the
// epilogues that store C as E4M3.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dbgemm {

// E4M3 code of q rounded to the nearest E4M3 value, ties to the even code; magnitudes
// at or above 448 saturate to +-448 (the caller's scale keeps values in range; the
// fp8 paths of the fused protocol store already-scaled outputs); NaN stays NaN.
__device__ __forceinline__ uint32_t e4m3_from_f32(float q) {
  const uint32_t sign = (__builtin_bit_cast(uint32_t, q) >> 24) & 0x80u;
  const float a = __builtin_fabsf(q);
  if (!(a == a)) return sign | 0x7Fu;
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0x1p-6f) {  // subnormal range: multiples of 2^-9 (8 rounds up to 2^-6, code 8)
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  }
  int ex = (int)((__builtin_bit_cast(uint32_t, a) >> 23) & 0xFFu) - 127;  // -6 .. 8
  // mantissa on the 3-bit grid: m in [8, 16) before rounding (exact scaling by 2^(3-ex))
  uint32_t m = (uint32_t)__builtin_rintf(a * __builtin_bit_cast(float, (uint32_t)(127 + 3 - ex) << 23));
  if (m == 16u) {
    m = 8u;
    ++ex;
  }
  return sign | ((uint32_t)(ex + 7) << 3) | (m - 8u);
}

// fp32 value of E4M3 code c (low 8 bits).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v;
  if (e == 15u && m == 7u)
    v = __builtin_nanf("");
  else if (e == 0u)
    v = (float)m * 0x1p-9f;
  else
    v = __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20));  // (1 + m/8) * 2^(e-7)
  return (c & 0x80u) ? -v : v;
}

}  // namespace dbgemm

namespace dbgemm {

// Four values to four E4M3 codes (a in the low byte) with the gfx950 conversion
// instruction (round to nearest even) after saturating to +-448, so that the result is
// e4m3_from_f32 of each value; NaN stays NaN.  The epilogues use this short form.
__device__ __forceinline__ float e4m3_clamp(float x) {
  return x != x ? x : __builtin_fminf(__builtin_fmaxf(x, -448.0f), 448.0f);
}
__device__ __forceinline__ uint32_t e4m3x4_from_f32(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), w, true);
  return (uint32_t)w;
}

}  // namespace dbgemm
