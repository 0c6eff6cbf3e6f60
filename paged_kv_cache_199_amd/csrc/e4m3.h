// The 8-bit E4M3 floating-point format of the open FP8 specification (bias 7, largest finite 448,
// NaN 0x7F / 0xFF, no infinities), as the KV pools store it: shared by the slot-mapped write and the
// decode pass that appends new tokens itself.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// The E4M3 code of x: the nearest code, ties to the even code, magnitudes from 448 up saturating to
// 448 (code 0x7E), NaN to the NaN code of its sign.  Below 2^-6 the codes are the multiples of 2^-9
// (code = multiple; 8 is the smallest normal, so the two ranges join); above, the code keeps the
// three leading fraction bits of x rounded half to even, with a carry into the exponent.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a != a) return sign | 0x7Fu;
  if (a >= 448.f) return sign | 0x7Eu;
  if (a < 0.015625f) return sign | (uint32_t)__builtin_rintf(a * 512.f);
  const uint32_t ab = __float_as_uint(a);
  int e = (int)(ab >> 23) - 127;                       // -6 .. 8
  uint32_t m = (ab >> 20) & 7u;
  const uint32_t rest = ab & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (m & 1u))) ++m;
  if (m == 8u) {
    m = 0u;
    ++e;
  }
  return sign | ((uint32_t)(e + 7) << 3) | m;
}

}  // namespace pkv
