// Matrix-core helpers of the small-batch sign product (FP4 signs x FP6
// activation terms), shared by the product kernel and the fused decode
// kernel. Device-only.
#pragma once

#include "lq_internal.h"

namespace lq {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;

template <int U>
__device__ __forceinline__ f32x4 mfma_fp4_fp6(uint32_t w, const i32x8& b, uint32_t scale, f32x4 c) {
  i32x8 a;
  a[0] = (int)(w & 0x11111111u);
  a[1] = (int)(w & 0x22222222u);
  a[2] = (int)(w & 0x44444444u);
  a[3] = (int)((w & 0x88888888u) | 0x22222222u);
  a[4] = a[5] = a[6] = a[7] = 0;   // unused by an FP4 operand
  // cbsz = 4: A is FP4 E2M1 (scale 2^0); blgp = 2: B is FP6 E2M3, its block
  // scale is byte U of `scale`.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 2, 0, 127, U, (int)scale);
}

__device__ __forceinline__ i32x8 lds_b_operand(const uint8_t* p) {
  const uint4 lo = *reinterpret_cast<const uint4*>(p);
  const uint4 hi = *reinterpret_cast<const uint4*>(p + 16);
  i32x8 b;
  b[0] = (int)lo.x; b[1] = (int)lo.y; b[2] = (int)lo.z; b[3] = (int)lo.w;
  b[4] = (int)hi.x; b[5] = (int)hi.y; b[6] = 0; b[7] = 0;
  return b;
}

}  // namespace lq
