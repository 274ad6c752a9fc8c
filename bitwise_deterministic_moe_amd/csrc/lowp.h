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
