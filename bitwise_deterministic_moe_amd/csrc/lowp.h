// Device helpers shared by the low-precision encoders (MXFP8, NVFP4).
#pragma once
#include "common.h"

namespace moedet {

// E4M3 code of y (|y| < 512 or saturated): nearest, ties to even,
// saturated at 448, sign kept; integer arithmetic on the float32 bits (v * 2^k
// scalings are exact, so the code is the exact nearest one).
DEV uint32_t e4m3_rne(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a >= 0x43e00000u) {                 // |y| >= 448
    code = 0x7e;
  } else if (a >= 0x3c800000u) {          // |y| >= 2^-6: normal E4M3
    const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;   // RNE to 3 mantissa bits
    code = r - (120u << 3);               // rebias the exponent: 127 -> 7
  } else {                                // subnormal E4M3: m * 2^-9, m in 0..8
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  }
  return sign | code;
}

// Four E4M3 codes (bytes 0..3 of the result) of a, b, c, d, each to nearest
// with ties to even and saturated at +-448, sign kept: the result of
// e4m3_rne on each, through gfx950's conversion instruction.  That
// instruction rounds to nearest even with E4M3 subnormals, but gives the
// NaN code past 464 instead of saturating, so the values are clamped to
// +-448 first (fmin / fmax keep the sign of zero).  A probe over every
// finite bf16 pattern, 8000 values around 448 and dense float32 steps around
// the powers of two 2^-40 .. 2^11 found it equal to e4m3_rne below 448.
DEV float clamp448(float y) { return fminf(fmaxf(y, -448.f), 448.f); }
DEV uint32_t e4m3x4(float a, float b, float c, float d) {
  typedef short s16x2_t __attribute__((ext_vector_type(2)));
  s16x2_t w = {0, 0};
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, clamp448(a), clamp448(b), 1.0f, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, clamp448(c), clamp448(d), 1.0f, true);
  return __builtin_bit_cast(uint32_t, w);
}

template <typename T>
DEV void load8(const T* p, float (&v)[8]);
template <>
DEV void load8(const uint16_t* p, float (&v)[8]) {
  const u32x4_t w = *(const u32x4_t*)p;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[2 * q] = bf16_to_f32(w[q] & 0xffffu);
    v[2 * q + 1] = bf16_to_f32(w[q] >> 16);
  }
}
template <>
DEV void load8(const float* p, float (&v)[8]) {
  const f32x4_t a = *(const f32x4_t*)p, b = *(const f32x4_t*)(p + 4);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[q] = a[q];
    v[4 + q] = b[q];
  }
}

}  // namespace moedet
