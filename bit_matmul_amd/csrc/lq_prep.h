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

// Maximum over each 32-lane half of the wavefront: DPP within quads (lane
// xor 1, xor 2), half-row and row mirrors (8, 16 lanes), then a swizzle
// with lane xor 16.
__device__ __forceinline__ float half_wave_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F)));
  return v;
}

// Value of lane ^ X (X a power of two up to 32): DPP for 1 and 2, a
// swizzle for 4..16 (within 32 lanes), a permute for 32.
template <int X>
__device__ __forceinline__ float lane_xor(float v) {
  const int i = __float_as_int(v);
  if constexpr (X == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, i, 0xB1, 0xF, 0xF, false));
  else if constexpr (X == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, i, 0x4E, 0xF, 0xF, false));
  else if constexpr (X <= 16) return __int_as_float(__builtin_amdgcn_ds_swizzle(i, 0x1F | (X << 10)));
  else return __shfl_xor(v, X, 64);
}

// One cross-lane butterfly stage over the 16 registers: all exchanges are
// issued before any is used.
template <int X>
__device__ __forceinline__ void lane_stage(float (&a)[16], int lane) {
  float p[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) p[k] = lane_xor<X>(a[k]);
  const bool upper = (lane & X) != 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) a[k] = upper ? p[k] - a[k] : a[k] + p[k];
}

// In-place fast Walsh-Hadamard transform (unnormalised) of every 2^lhb-value
// block of the 1024 values xs[0..1023], by one wavefront: lane l holds
// xs[16l + k] (k = 0..15); stages with stride below 16 pair registers, the
// others pair lanes l and l ^ (stride / 16).
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
  if (lhb > 6) lane_stage<4>(a, lane);
  if (lhb > 7) lane_stage<8>(a, lane);
  if (lhb > 8) lane_stage<16>(a, lane);
  if (lhb > 9) lane_stage<32>(a, lane);
  float4* dst = reinterpret_cast<float4*>(xs + 16 * lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = make_float4(a[4 * i], a[4 * i + 1], a[4 * i + 2], a[4 * i + 3]);
}


// FP6 record of one 32-value block: lane m (0..31) of a half-wavefront holds
// value v (already multiplied by its plane factor); cuts it into nt terms
// and returns, per term t, the six code dwords in lanes 0..5 (dw[t]) and the
// E8M0 scale byte (e[t] + 127, the same in every lane). `orig - v` after the
// call is the value the terms represent.
struct Fp6Block {
  uint32_t dw[4];
  int e[4];
};
__device__ __forceinline__ Fp6Block fp6_block_terms(float& v, int nt, int m) {
  Fp6Block r;
  const int L6 = m < 6 ? m : 5;
  const int first = (32 * L6) / 6;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    r.dw[t] = 0u;
    r.e[t] = 0;
    if (t < nt) {
      const int e = e2m3_block_exponent(half_wave_max(fabsf(v)));
      const uint32_t code = e2m3_encode(ldexpf(v, -e));
      v -= ldexpf(e2m3_decode(code), e);
      // Lane L < 6 assembles dword L of the 192 code bits from the codes of
      // lanes first(L) .. first(L) + 5 (code n sits at bit 6n); all six
      // exchanges first, then the branch-free assembly.
      uint32_t cv[6];
#pragma unroll
      for (int s6 = 0; s6 < 6; ++s6) cv[s6] = __shfl(code & 63u, min(first + s6, 31), 32);
      uint32_t dw = 0u;
#pragma unroll
      for (int s6 = 0; s6 < 6; ++s6) {
        const int pos = 6 * (first + s6) - 32 * L6;
        const uint32_t lo = pos >= 0 ? (cv[s6] << (pos & 31)) : (cv[s6] >> ((-pos) & 31));
        dw |= (first + s6 <= 31 && pos < 32) ? lo : 0u;
      }
      r.dw[t] = dw;
      r.e[t] = e;
    }
  }
  return r;
}

}  // namespace lq
