// FP6 E2M3 (OCP microscaling element format: 1 sign, 2 exponent bits with
// bias 1, 3 mantissa bits; largest magnitude 7.5, no inf/nan) and its E8M0
// block scale, as used for the activation operand of the small-batch
// matrix-core product. Device-only helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lq {

constexpr float kE2M3Max = 7.5f;

// Round-to-nearest-even encoding of |v| <= 7.5 (larger magnitudes saturate).
__device__ __forceinline__ uint32_t e2m3_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 31) << 5;
  const float a = fabsf(v);
  uint32_t code;
  if (a < 1.0f) {
    code = (uint32_t)rintf(a * 8.0f);                 // subnormals m/8; 8 is 1.0 (e=1, m=0)
  } else {
    uint32_t u = __float_as_uint(a);
    u += 0x7FFFFu + ((u >> 20) & 1u);                 // round the fp32 mantissa to 3 bits
    code = ((((u >> 23) - 126u) << 3) | ((u >> 20) & 7u));
  }
  return sign | min(code, 31u);
}

__device__ __forceinline__ float e2m3_decode(uint32_t code) {
  const uint32_t c = code & 31u;
  const float a = c < 8u ? (float)c * 0.125f
                         : ldexpf(1.0f + (float)(c & 7u) * 0.125f, (int)(c >> 3) - 1);
  return (code & 32u) ? -a : a;
}

// Exponent e of the block scale 2^e for a block whose largest magnitude is
// amax: the largest e with amax * 2^-e <= 7.5 (so that the block's values fit
// E2M3 without saturation and its largest one lands in the top binade),
// clamped to the E8M0 range. amax == 0 gives 0.
__device__ __forceinline__ int e2m3_block_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  const int E = __builtin_amdgcn_frexp_expf(amax) - 1;  // 2^E <= amax < 2^(E+1)
  int e = (amax <= ldexpf(kE2M3Max, E - 2)) ? E - 2 : E - 1;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

}  // namespace lq
