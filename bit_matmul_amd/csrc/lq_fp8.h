// OCP FP8 E4M3 (bias 7, largest finite 448, no infinities) encode/decode with
// round-to-nearest-even, written out in integer/float arithmetic so that the
// rounding is exactly the one stated here. Used to cut an fp32 value into
// terms t_0 + t_1/16 + t_2/256 + ... of 4 significant bits each.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lq {

// |v| is clamped to 448; normal range uses the fp32 bit pattern rounded at
// mantissa bit 20, the subnormal range (|v| < 2^-6) multiples of 2^-9.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)__builtin_rintf(a * 512.0f);         // 0..8; 8 is the smallest normal
  } else {
    uint32_t u = __float_as_uint(a);
    u += 0x7FFFFu + ((u >> 20) & 1u);                      // round to 3 mantissa bits, ties even
    code = (((u >> 23) - 120u) << 3) | ((u >> 20) & 7u);
  }
  return sign | code;
}

__device__ __forceinline__ float e4m3_decode(uint32_t code) {
  const uint32_t e = (code >> 3) & 15u, m = code & 7u;
  const float a = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * (1.0f / 512.0f);
  return (code & 0x80u) ? -a : a;
}

// Term t of v: t_0 = fp8(v), t_i = fp8(16 * (r_{i-1} - t_{i-1})) with the
// residuals r exact in fp32, so v = t_0 + t_1/16 + t_2/256 + ... up to the
// rounding of the last term.
__device__ __forceinline__ uint32_t fp8_term(float v, int t) {
  uint32_t code = e4m3_encode(v);
  for (int i = 0; i < t; ++i) {
    v = (v - e4m3_decode(code)) * 16.0f;
    code = e4m3_encode(v);
  }
  return code;
}

}  // namespace lq
