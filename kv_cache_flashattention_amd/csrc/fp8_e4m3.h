// OCP E4M3FN codec on the device: 1 sign bit, 4 exponent bits (bias 7),
// 3 mantissa bits, no infinities, 0x7F/0xFF are NaN, largest finite 448.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

namespace kvfa {

// Round to nearest, ties to even, saturating to +-448; the sign bit is kept
// (so -0 and negative values that round to zero give 0x80).  Works on the
// float32 bit pattern: the 23-bit mantissa is cut to 3 bits with the usual
// guard/sticky comparison, and a carry out of the mantissa simply increments
// the exponent field because codes of consecutive magnitudes are consecutive
// integers.  Below 2^-6 the format is subnormal with spacing 2^-9, handled by
// an exact scaling by 2^9 and a round-to-nearest-even to an integer.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;              // NaN stays NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;             // |x| >= 448: saturate
  if (a < 0x3C800000u) {                                 // |x| < 2^-6: subnormal band
    float n = __builtin_rintf(__uint_as_float(a) * 512.0f);
    return sign | (uint32_t)n;                           // 0..8 (8 is 2^-6 itself)
  }
  uint32_t e = (a >> 23) - 127u + 7u;                    // biased e4m3 exponent, 1..15
  uint32_t keep = (a >> 20) & 7u;
  uint32_t rest = a & 0xFFFFFu;
  uint32_t up = (rest > 0x80000u) || (rest == 0x80000u && (keep & 1u));
  uint32_t code = (e << 3) + keep + up;
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

// Exact value of a code (finite codes only; the encoder never makes NaN).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  uint32_t sign = (c & 0x80u) << 24;
  uint32_t e = (c >> 3) & 0xFu;
  uint32_t m = c & 7u;
  if (e == 0) return __uint_as_float(sign | __float_as_uint((float)m * 0x1p-9f));
  return __uint_as_float(sign | ((e + 120u) << 23) | (m << 20));
}

}  // namespace kvfa
