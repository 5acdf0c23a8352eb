// Device helpers of the activation preparation (whitening, lift and the
// FP6 operand), shared by the standalone preparation kernel and the fused
// decode kernel. Device-only.
#pragma once

#include "lq_fp6.h"
#include "lq_internal.h"

namespace lq {

// A tile's lifted columns come from at most 511/D + 2 d-blocks, i.e. at most
// 511 + 2D <= 639 original columns, which lie in at most 2 blocks of 1024,
// 3 of 512, 4 of 256, ...: never more than 2048 values.
constexpr int kSpanMax = 2048;

// The Hadamard blocks covering a tile's d-blocks: original columns
// [h_lo, h_lo + span).
struct TileSpan {
  int width;   // lifted columns of the tile
  int h_lo;    // first original column of the first covering Hadamard block
  int span;    // number of original columns loaded (a multiple of hb)
};
__device__ __forceinline__ TileSpan tile_span(int q, int K, int d, int D, int lhb, int L) {
  TileSpan t;
  const int c_lo = q * kTileCols;
  t.width = min(kTileCols, L - c_lo);
  const int j_lo = c_lo / D, j_hi = (c_lo + t.width - 1) / D + 1;
  const int k_lo = j_lo * d;
  const int k_hi = min(j_hi * d, K);
  t.h_lo = k_lo < K ? (k_lo >> lhb) << lhb : 0;
  t.span = k_lo < K ? (((k_hi - 1) >> lhb) + 1) * (1 << lhb) - t.h_lo : 0;
  return t;
}

// Value of lane ^ X (X a power of two up to 32), all on the vector ALU:
// DPP quad permutations for 1 and 2, a half-row mirror (lane ^ 7) then a
// quad reversal (lane ^ 3) for 4, a rotation of the 16-lane row by 8 for 8,
// and the gfx950 row-swap permutes for 16 and 32 (each returns the two
// halves of the exchange; a lane keeps the one that came from its partner).
template <int X>
__device__ __forceinline__ float lane_xor(float v) {
  const int i = __float_as_int(v);
  if constexpr (X == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, i, 0xB1, 0xF, 0xF, false));
  else if constexpr (X == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, i, 0x4E, 0xF, 0xF, false));
  else if constexpr (X == 4) {
    const int h = __builtin_amdgcn_update_dpp(0, i, 0x141, 0xF, 0xF, false);
    return __int_as_float(__builtin_amdgcn_update_dpp(0, h, 0x1B, 0xF, 0xF, false));
  } else if constexpr (X == 8) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, i, 0x128, 0xF, 0xF, false));
  } else if constexpr (X == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(i, i, false, false);
    return __int_as_float((threadIdx.x & 16) ? r[0] : r[1]);
  } else {
    static_assert(X == 32, "lane_xor: X is a power of two up to 32");
    const auto r = __builtin_amdgcn_permlane32_swap(i, i, false, false);
    return __int_as_float((threadIdx.x & 32) ? r[0] : r[1]);
  }
}

// One cross-lane butterfly stage over the 16 registers: all exchanges are
// issued before any is used.
template <int X>
__device__ __forceinline__ void lane_stage(float (&a)[16], int lane) {
  float p[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) p[k] = lane_xor<X>(a[k]);
  // a + p in the lower lane, p - a in the upper one, as one fma with a
  // multiplier of +-1 (exact, so the same single rounding as the add)
  const float sgn = (lane & X) != 0 ? -1.0f : 1.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) a[k] = fmaf(a[k], sgn, p[k]);
}

// In-place fast Walsh-Hadamard transform (unnormalised) of every 2^lhb-value
// block of the 1024 values xs[0..1023], by one wavefront. Index bit s of a
// value is butterflied in stage s (s < lhb). Lane l first holds xs[16l + k]
// (k = 0..15): bits 0..3 pair registers, bits 4 and 5 pair lanes l ^ 1 and
// l ^ 2 (DPP). For bits 6..9 the values go through LDS once so that lane l
// holds xs[l + 64k], where those bits pair registers again.
__device__ __forceinline__ void wave_fwht_1024(float* xs, int lhb, int lane) {
  float a[16];
  const float4* src = reinterpret_cast<const float4*>(xs + 16 * lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 v = src[i];
    a[4 * i] = v.x; a[4 * i + 1] = v.y; a[4 * i + 2] = v.z; a[4 * i + 3] = v.w;
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s < lhb) {
      const int h = 1 << s;
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if ((k & h) == 0) {
          const float x0 = a[k], x1 = a[k | h];
          a[k] = x0 + x1;
          a[k | h] = x0 - x1;
        }
    }
  }
  if (lhb > 4) lane_stage<1>(a, lane);
  if (lhb > 5) lane_stage<2>(a, lane);
  float4* dst = reinterpret_cast<float4*>(xs + 16 * lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = make_float4(a[4 * i], a[4 * i + 1], a[4 * i + 2], a[4 * i + 3]);
  if (lhb > 6) {
    // The wavefront's own LDS writes are seen by its later reads.
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int k = 0; k < 16; ++k) a[k] = xs[lane + 64 * k];
#pragma unroll
    for (int s = 6; s < 10; ++s) {
      if (s < lhb) {
        const int h = 1 << (s - 6);
#pragma unroll
        for (int k = 0; k < 16; ++k)
          if ((k & h) == 0) {
            const float x0 = a[k], x1 = a[k | h];
            a[k] = x0 + x1;
            a[k | h] = x0 - x1;
          }
      }
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) xs[lane + 64 * k] = a[k];
  }
}

// The same transform of 1024 values by 256 threads (four wavefronts; t =
// 0..255 within the group), every thread of the workgroup calling it (it
// holds workgroup barriers). Thread t brings v[j] = value (t % 64) + 64 j +
// 256 (t / 64): bits 0..5 of the index pair lanes t ^ 1 .. t ^ 32
// (vector-ALU exchanges), bits 6 and 7 pair registers. Through LDS, thread
// t then holds values (t % 64) + 64 (t / 64) + 256 j, where bits 8 and 9
// pair registers. Results land in xs[0..1023]. The stages run in the order
// of their bit and every butterfly is the same single add or subtract as in
// wave_fwht_1024, so both give identical results. A group past the values
// in use transforms whatever it holds (no branch, so the loads feeding v
// stay ahead of every wait).
template <int X>
__device__ __forceinline__ void lane_stage4(float (&v)[4], int t, int lhb, int bit) {
  if (bit < lhb) {
    float o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = lane_xor<X>(v[i]);
    const float sgn = (t & X) != 0 ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = fmaf(v[i], sgn, o[i]);
  }
}
__device__ __forceinline__ void reg_stages4(float (&v)[4], bool b0, bool b1) {
  if (b0) {
    float a = v[0], b = v[1]; v[0] = a + b; v[1] = a - b;
    a = v[2]; b = v[3]; v[2] = a + b; v[3] = a - b;
  }
  if (b1) {
    float a = v[0], b = v[2]; v[0] = a + b; v[2] = a - b;
    a = v[1]; b = v[3]; v[1] = a + b; v[3] = a - b;
  }
}
__device__ __forceinline__ void block_fwht_1024_regs(float* xs, float (&v)[4], int lhb, int t) {
  lane_stage4<1>(v, t, lhb, 0);
  lane_stage4<2>(v, t, lhb, 1);
  lane_stage4<4>(v, t, lhb, 2);
  lane_stage4<8>(v, t, lhb, 3);
  lane_stage4<16>(v, t, lhb, 4);
  lane_stage4<32>(v, t, lhb, 5);
  reg_stages4(v, lhb > 6, lhb > 7);
  const int lo = t & 63, hi = t >> 6;
#pragma unroll
  for (int j = 0; j < 4; ++j) xs[lo + 64 * j + 256 * hi] = v[j];
  __syncthreads();
  if (lhb > 8) {
    float w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = xs[lo + 64 * hi + 256 * j];
    reg_stages4(w, true, lhb > 9);
#pragma unroll
    for (int j = 0; j < 4; ++j) xs[lo + 64 * hi + 256 * j] = w[j];
    __syncthreads();
  }
}

// One lifted value z[col] = sum_{i < min(d, K - kb)} Ms[i * D + e] *
// xs[kb + i - h_lo] with col = blk * D + e and kb = blk * d (the lift of
// d-block blk; rows of the virtual zero pad are skipped). Products are added
// in order of i; the LDS reads of 16 terms are issued before they are used.
__device__ __forceinline__ float lift_column(const float* Ms, const float* xs, int col, int d,
                                             int D, int K, int h_lo) {
  const int blk = col / D;
  const int e = col - blk * D;
  const int kb = blk * d;
  const int nk = min(d, K - kb);
  float acc = 0.0f;
  for (int i0 = 0; i0 < nk; i0 += 16) {
    float mv[16], xv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = min(i0 + u, nk - 1);
      mv[u] = Ms[i * D + e];
      xv[u] = xs[kb + i - h_lo];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (i0 + u < nk) acc = fmaf(mv[u], xv[u], acc);
  }
  return acc;
}

// FP6 terms of one 32-value block held by ONE lane, on the gfx950 packed
// conversion instructions. The lane holds the value meeting reduction index
// 32g + n in va[n / 2] (n even) or vb[n / 2] (n odd): the conversion puts
// element i of its first source at code 2i and of its second at code 2i + 1,
// so code n lands at bit 6n of the six dwords, the matrix-core operand
// layout. Per term t: the block exponent e (the largest with
// max|v| * 2^-e <= 7.5), the codes round-to-nearest-even(v / 2^e), then
// v -= the decoded codes; va and vb end as the residual.
typedef float lq_v16f __attribute__((ext_vector_type(16)));
typedef float lq_v32f __attribute__((ext_vector_type(32)));
typedef int lq_v6i __attribute__((ext_vector_type(6)));
struct Fp6LaneTerms {
  uint32_t dw[4][6];
  int e[4];
};
__device__ __forceinline__ void fp6_lane_block_terms(lq_v16f& va, lq_v16f& vb, int nt,
                                                     Fp6LaneTerms& r) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (t < nt) {
      float m16[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) m16[i] = fmaxf(fabsf(va[i]), fabsf(vb[i]));
#pragma unroll
      for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w; ++i) m16[i] = fmaxf(m16[i], m16[i + w]);
      // (a normal scale: 2^-127 would be a subnormal fp32 operand)
      const int e = max(e2m3_block_exponent(m16[0]), -126);
      const float sc = ldexpf(1.0f, e);
      const lq_v6i codes = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(va, vb, sc);
      // The conversion must not write registers it still reads: keeping the
      // sources live past it stops the register allocator from giving the
      // destination any of their registers.
      asm volatile("" ::"v"(va), "v"(vb));
      const lq_v32f back = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(codes, sc);
      asm volatile("" ::"v"(codes));
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        va[i] -= back[2 * i];
        vb[i] -= back[2 * i + 1];
      }
#pragma unroll
      for (int k = 0; k < 6; ++k) r.dw[t][k] = (uint32_t)codes[k];
      r.e[t] = e;
    }
  }
}

// Where the lane-per-block conversion wants lifted column jj of a tile (its
// LDS slot) and the sign-plane factor the value is pre-multiplied by. Column
// offset r = jj % 32 of block (u, g) = jj / 32 meets plane j = r % 4 (factor
// -4, -2, -1, +1 for j = 0..3) at reduction index n = 8 j + r / 4; index n
// goes to va[n / 2] (n even, slot n / 2) or vb[n / 2] (n odd, slot
// 16 + n / 2) of the lane that converts the block.
__device__ __forceinline__ int fp6_slot(int jj, float& f) {
  const int r = jj & 31, j = r & 3, n = 8 * j + (r >> 2);
  f = j == 3 ? 1.0f : (j == 2 ? -1.0f : (j == 1 ? -2.0f : -4.0f));
  return (jj & ~31) + ((n & 1) ? 16 : 0) + (n >> 1);
}

// FP6 terms of one block held in va, vb (as fp6_lane_block_terms wants
// them, plane factors applied). Returns the sum over the block's plane 0..2
// values (n < 24) of what the terms represent, divided by the plane factor:
// the block's share of the plane-0..2 column sum the product adds back.
__device__ __forceinline__ float fp6_lane_block_regs(lq_v16f& va, lq_v16f& vb, int nt,
                                                     Fp6LaneTerms& r) {
  float oa[12], ob[12];
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    oa[i] = va[i];
    ob[i] = vb[i];
  }
  fp6_lane_block_terms(va, vb, nt, r);
  float tp = 0.0f;
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    const float inv = i < 4 ? -0.25f : (i < 8 ? -0.5f : -1.0f);    // 1 / factor of plane i / 4
    tp = fmaf(oa[i] - va[i], inv, tp);
    tp = fmaf(ob[i] - vb[i], inv, tp);
  }
  return tp;
}

// FP6 terms of block blk of a tile whose 512 values sit in LDS in the
// fp6_slot layout, by one lane.
__device__ __forceinline__ float fp6_lane_block(const float* zt, int blk, int nt, Fp6LaneTerms& r) {
  lq_v16f va, vb;
  const float4* p = reinterpret_cast<const float4*>(zt + 32 * blk);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 qa = p[i], qb = p[4 + i];
    va[4 * i] = qa.x; va[4 * i + 1] = qa.y; va[4 * i + 2] = qa.z; va[4 * i + 3] = qa.w;
    vb[4 * i] = qb.x; vb[4 * i + 1] = qb.y; vb[4 * i + 2] = qb.z; vb[4 * i + 3] = qb.w;
  }
  return fp6_lane_block_regs(va, vb, nt, r);
}

// The same from the block's 32 lifted values in column order (16-byte
// aligned, no factors applied): the fp6_slot placement and the plane factor
// (a power of two, so the product is exact) are applied in registers. Slot s
// of va holds column 8 (s % 4) + s / 4, of vb column 8 (s % 4) + 4 + s / 4,
// both with the factor of plane s / 4.
__device__ __forceinline__ float fp6_lane_block_cols(const float* z, int nt, Fp6LaneTerms& r) {
  float v[32];
  const float4* p = reinterpret_cast<const float4*>(z);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 q = p[i];
    v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
  }
  lq_v16f va, vb;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const float f = s < 4 ? -4.0f : (s < 8 ? -2.0f : (s < 12 ? -1.0f : 1.0f));
    va[s] = f * v[8 * (s % 4) + s / 4];
    vb[s] = f * v[8 * (s % 4) + 4 + s / 4];
  }
  return fp6_lane_block_regs(va, vb, nt, r);
}

}  // namespace lq
