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
  const uint2* q = reinterpret_cast<const uint2*>(p);
  const uint2 a = q[0], c = q[1], e = q[2];
  i32x8 b;
  b[0] = (int)a.x; b[1] = (int)a.y; b[2] = (int)c.x; b[3] = (int)c.y;
  b[4] = (int)e.x; b[5] = (int)e.y; b[6] = 0; b[7] = 0;
  return b;
}

// The lift as a small matrix product on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32): Z[b][e] = sum_i X[b][i] Mt[i][e] for the blocks
// b0 + 16 rt + [0, 16) of row tile rt (wavefront-strided), X[b][i] =
// xs[b d + i - xoff] (zero for i >= d or past K), Mt[i][e] = Ms[e DMr + i]
// (zero past d, D). Lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16]
// and receives D[4 (l / 16) + v][l % 16]; `emit(b, e, value)` stores one.
// fp32 products summed by the matrix core (not in the fmaf order of the
// two-launch path: the last bits may differ).
template <int DM, int DMr, typename Emit>
__device__ __forceinline__ void mfma_lift(const float* xs, int xoff, const float* Ms, int b0,
                                          int nb, int d, int D, int K, int wave, int nwaves,
                                          int lane, Emit emit) {
  constexpr int KS = (DM + 3) / 4;
  const int lr = lane & 15, lg = lane >> 4;
  float bm[2][KS];
#pragma unroll
  for (int cj = 0; cj < 2; ++cj)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int i = 4 * ks + lg, e = 16 * cj + lr;
      bm[cj][ks] = (i < d && e < D) ? Ms[e * DMr + i] : 0.0f;
    }
  const int ct = D > 16 ? 2 : 1;
  for (int rt = wave; rt * 16 < nb; rt += nwaves) {
    float av[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int bb = 16 * rt + lr, i = 4 * ks + lg;
      const int k = (b0 + bb) * d + i;
      av[ks] = (bb < nb && i < d && k < K) ? xs[k - xoff] : 0.0f;
    }
#pragma unroll
    for (int cj = 0; cj < 2; ++cj) {
      if (cj < ct) {
        f32x4 acc = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[ks], bm[cj][ks], acc, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int bb = 16 * rt + 4 * lg + v, e = 16 * cj + lr;
          if (bb < nb && e < D) emit(b0 + bb, e, acc[v]);
        }
      }
    }
  }
}

}  // namespace lq
