// Small-batch sign product (B <= 16) on the gfx950 FP4 x FP8 matrix cores
// (v_mfma_scale_f32_16x16x128_f8f6f4, A = signs as FP4 E2M1, B = lifted
// activations as FP8 E4M3 terms, unit block scales, fp32 accumulation).
//
// Sign operand. A lane of a 16x16x128 MFMA supplies 32 reduction indices of
// one row: k = 32g + n for lane group g, in nibble n = 8*j + i of its 4-dword
// A operand. A packed word u of slot (g, r) holds row r's signs for tile
// columns 128u + 32g + b. One word becomes one whole A operand with four
// bit operations and no shifts, by splitting its bits into the four planes
// b = 4i + j (j = b mod 4):
//   dword 0 = w & 0x11111111   nibble 0x1 = 0.5 where the bit is set, else 0
//   dword 1 = w & 0x22222222   nibble 0x2 = 1.0
//   dword 2 = w & 0x44444444   nibble 0x4 = 2.0
//   dword 3 = (w & 0x88888888) | 0x22222222   nibble = +1.0 or -1.0 (0xA)
// so nibble 8j + i meets packed column 128u + 32g + 4i + j. With the sign
// s = 1 - 2*bit, sum_j s_j z_j = sum_{plane 3} s z + sum_{planes 0-2} z
// - 2 sum_{planes 0-2} bit z: the activation operand carries z on plane 3 and
// -4z, -2z, -z on planes 0, 1, 2 (pre-multiplied by the preparation kernel),
// and the plane-0..2 column sums of z are added once per batch row.
//
// Activation operand. Each lifted value is scaled per (tile, batch row) by a
// power of two and cut into NT fp8 terms (each 16x finer); the MFMA's 16
// columns hold (batch row, term) pairs, so for B <= 5 the three terms of
// every batch row ride along in one MFMA at no extra cost. The terms are
// combined (t0 + t1/16 + t2/256 ...) and unscaled in fp32.
//
// Work split, with no communication between workgroups: a workgroup owns
// PPW 16-row panels over the whole reduction length, which its W wavefronts
// split into contiguous slices of at most TPW tiles. A wavefront requests
// every packed slot of its slice at once (the HBM stream needs many bytes in
// flight), and the L2-resident activation operand one tile ahead of the
// MFMAs; lanes whose MFMA column is unused read the same operand address as
// column 0, so their loads merge.
// The wavefronts' accumulators are added in LDS in a fixed order, the terms
// combined, and y written: deterministic, no atomics, no partial buffers.
#include "lq_internal.h"

namespace lq {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;

__device__ __forceinline__ f32x4 mfma_fp4_fp8(uint32_t w, const uint4& blo, const uint4& bhi, f32x4 c) {
  i32x8 a;
  a[0] = (int)(w & 0x11111111u);
  a[1] = (int)(w & 0x22222222u);
  a[2] = (int)(w & 0x44444444u);
  a[3] = (int)((w & 0x88888888u) | 0x22222222u);
  a[4] = a[5] = a[6] = a[7] = 0;   // unused by an FP4 operand
  i32x8 b;
  b[0] = (int)blo.x; b[1] = (int)blo.y; b[2] = (int)blo.z; b[3] = (int)blo.w;
  b[4] = (int)bhi.x; b[5] = (int)bhi.y; b[6] = (int)bhi.z; b[7] = (int)bhi.w;
  // cbsz = 4: A is FP4 E2M1; blgp = 0: B is FP8 E4M3; scales 2^0 (E8M0 127).
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, 127, 0, 127);
}

// The activation-side registers of one tile.
template <int CS>
struct OpRegs {
  uint4 bop[4][CS][2];
  float inv[CS];
  float tp[CS];
};

template <int NT, int CS, int PPW, int W, int TPW>
__global__ __launch_bounds__(64 * W) void sign_fp4_kernel(
    const uint8_t* __restrict__ packed, int panels, int64_t panel_bytes, int full_tiles,
    int tail_bytes, int ext_tiles, const uint4* __restrict__ zop,
    const float* __restrict__ invscale, const float* __restrict__ tpart, int ncv, int B,
    const float* __restrict__ row_scale, void* __restrict__ y, int y_bf16, int N, int tpw) {
  constexpr int RP = 16 / NT;                         // batch rows per column set
  __shared__ f32x4 red[W][PPW][CS][64];
  __shared__ float tsw[W][CS][16];

  const int tid = threadIdx.x;
  const int wave = wave_id(), lane = tid & 63;
  const int g = lane >> 4, r = lane & 15;
  const int pbase = blockIdx.x * PPW;
  const int t0 = wave * tpw;
  const int nt_all = max(0, min(tpw, ext_tiles - t0));       // tiles of this slice

  int bclamp[CS], zcol[CS];
#pragma unroll
  for (int cs = 0; cs < CS; ++cs) {
    const int bcol = cs * RP + r / NT;
    const bool valid = (r < RP * NT) && (bcol < B) && (r < ncv);
    bclamp[cs] = valid ? bcol : 0;
    zcol[cs] = valid ? r : 0;
  }
  const uint8_t* prow[PPW];
#pragma unroll
  for (int i = 0; i < PPW; ++i) prow[i] = packed + (int64_t)min(pbase + i, panels - 1) * panel_bytes;

  f32x4 acc[PPW][CS];
  float tsum[CS];
#pragma unroll
  for (int cs = 0; cs < CS; ++cs) {
    tsum[cs] = 0.0f;
#pragma unroll
    for (int i = 0; i < PPW; ++i) acc[i][cs] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  }

  auto load_op = [&](int t, OpRegs<CS>& R) {
    t = min(t, ext_tiles - 1);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int cs = 0; cs < CS; ++cs)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          R.bop[u][cs][h] = zop[((((int64_t)t * 4 + u) * CS + cs) * 2 + h) * 4 * ncv + g * ncv + zcol[cs]];
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) {
      R.inv[cs] = invscale[(int64_t)t * B + bclamp[cs]];
      R.tp[cs] = tpart[(int64_t)t * B + bclamp[cs]];
    }
  };
  auto compute = [&](const uint4 (&sl)[PPW], const OpRegs<CS>& R) {
    f32x4 tacc[PPW][CS];
#pragma unroll
    for (int i = 0; i < PPW; ++i)
#pragma unroll
      for (int cs = 0; cs < CS; ++cs) tacc[i][cs] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < PPW; ++i) {
        const uint32_t w = (u == 0) ? sl[i].x : (u == 1) ? sl[i].y : (u == 2) ? sl[i].z : sl[i].w;
#pragma unroll
        for (int cs = 0; cs < CS; ++cs)
          tacc[i][cs] = mfma_fp4_fp8(w, R.bop[u][cs][0], R.bop[u][cs][1], tacc[i][cs]);
      }
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) {
      tsum[cs] += R.tp[cs];
#pragma unroll
      for (int i = 0; i < PPW; ++i) acc[i][cs] += tacc[i][cs] * R.inv[cs];
    }
  };

  // The slice is processed in chunks of TPW tiles.
  for (int c0 = 0; c0 < nt_all; c0 += TPW) {
    const int tc = t0 + c0;                          // first tile of the chunk
    const int nc = min(TPW, nt_all - c0);            // tiles in the chunk
    const int nf = max(0, min(nc, full_tiles - tc)); // of which full tiles

    // 1. Every packed slot of the chunk is requested at once (TPW * PPW
    // 128-bit loads per lane in flight), at clamped always-valid addresses;
    // then the tail tile's bytes, if the chunk ends with it.
    uint4 slot[PPW][TPW];
    if (full_tiles > 0) {
#pragma unroll
      for (int qq = 0; qq < TPW; ++qq) {
        const int t = min(tc + qq, full_tiles - 1);
#pragma unroll
        for (int i = 0; i < PPW; ++i) slot[i][qq] = load_full_slot(prow[i], t, g, r);
      }
    }
    uint4 tslot[PPW];
#pragma unroll
    for (int i = 0; i < PPW; ++i) tslot[i] = make_uint4(0u, 0u, 0u, 0u);
    if (nf < nc) {
#pragma unroll
      for (int i = 0; i < PPW; ++i) tslot[i] = load_tail_slot(prow[i], full_tiles, tail_bytes, g, r);
    }
    auto tile_slots = [&](int qq, uint4 (&sl)[PPW]) {
#pragma unroll
      for (int i = 0; i < PPW; ++i) sl[i] = qq < nf ? slot[i][qq] : tslot[i];
    };

    // 2. The activation operand (L2-resident) one tile ahead of the MFMAs.
    OpRegs<CS> oa, ob;
    load_op(tc, oa);
#pragma unroll
    for (int qq = 0; qq < TPW; qq += 2) {
      if (qq + 1 < nc) load_op(tc + qq + 1, ob);
      if (qq < nc) {
        uint4 sl[PPW];
        tile_slots(qq, sl);
        compute(sl, oa);
      }
      if (qq + 2 < nc) load_op(tc + qq + 2, oa);
      if (qq + 1 < nc) {
        uint4 sl[PPW];
        tile_slots(qq + 1, sl);
        compute(sl, ob);
      }
    }
  }

  // Add the wavefronts' accumulators in a fixed order.
#pragma unroll
  for (int i = 0; i < PPW; ++i)
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) red[wave][i][cs][lane] = acc[i][cs];
  if (g == 0) {
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) tsw[wave][cs][r] = tsum[cs];
  }
  __syncthreads();
  for (int item = tid; item < PPW * CS * 64; item += 64 * W) {
    const int i = item / (CS * 64), cs = (item / 64) % CS, l = item % 64;
    f32x4 s = red[0][i][cs][l];
#pragma unroll
    for (int w = 1; w < W; ++w) s += red[w][i][cs][l];
    red[0][i][cs][l] = s;
  }
  if (tid < CS * 16) {
    const int cs = tid / 16, rr = tid % 16;
    float s = tsw[0][cs][rr];
#pragma unroll
    for (int w = 1; w < W; ++w) s += tsw[w][cs][rr];
    tsw[0][cs][rr] = s;
  }
  __syncthreads();

  // Combine the terms of each batch row and write y: item = (panel, column
  // set, lane group, batch row of the set).
  for (int item = tid; item < PPW * CS * 4 * RP; item += 64 * W) {
    const int i = item / (CS * 4 * RP);
    const int cs = (item / (4 * RP)) % CS;
    const int gg = (item / RP) % 4;
    const int br = item % RP;
    const int b = cs * RP + br;
    const int p = pbase + i;
    if (b >= B || p >= panels) continue;
    const int rr = br * NT;                       // MFMA column of term 0
    f32x4 v = red[0][i][cs][16 * gg + rr];
    float f = 0.0625f;
#pragma unroll
    for (int t = 1; t < NT; ++t) {
      v += red[0][i][cs][16 * gg + rr + t] * f;
      f *= 0.0625f;
    }
    const float tp = tsw[0][cs][rr];
    const int n0 = p * kPanelRows + 4 * gg;
    const float4 rs = *reinterpret_cast<const float4*>(row_scale + n0);
    const float v0 = rs.x * (v[0] + tp), v1 = rs.y * (v[1] + tp);
    const float v2 = rs.z * (v[2] + tp), v3 = rs.w * (v[3] + tp);
    if (y_bf16) {
      const uint32_t lo = f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16);
      const uint32_t hi = f32_to_bf16_bits(v2) | (f32_to_bf16_bits(v3) << 16);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + (int64_t)b * N + n0) = make_uint2(lo, hi);
    } else {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + (int64_t)b * N + n0) = make_float4(v0, v1, v2, v3);
    }
  }
}

template <int NT, int CS, int PPW, int W>
hipError_t launch_fp4_t(const uint8_t* packed, const PackedGeom& g, const OperandPlan& op,
                        int64_t B, const float* row_scale, void* y, bool y_bf16,
                        const Fp4Plan& plan, hipStream_t stream) {
  const dim3 grid((unsigned)((g.panels + PPW - 1) / PPW));
  constexpr int TPW = CS == 1 ? 12 : 6;   // packed tiles in flight per chunk
  hipLaunchKernelGGL((sign_fp4_kernel<NT, CS, PPW, W, TPW>), grid, dim3(64 * W), 0, stream, packed,
                     (int)g.panels, g.panel_bytes, g.full_tiles, g.tail_bytes, g.ext_tiles, op.zop,
                     op.invscale, op.tpart, op.ncv, (int)B, row_scale, y, y_bf16 ? 1 : 0, (int)g.N,
                     plan.tpw);
  return hipGetLastError();
}

template <int NT, int CS, int PPW>
hipError_t launch_fp4_w(const uint8_t* packed, const PackedGeom& g, const OperandPlan& op,
                        int64_t B, const float* row_scale, void* y, bool y_bf16,
                        const Fp4Plan& plan, hipStream_t stream) {
  if constexpr (CS == 1) {
    if (plan.waves == 8)
      return launch_fp4_t<NT, CS, PPW, 8>(packed, g, op, B, row_scale, y, y_bf16, plan, stream);
  }
  return launch_fp4_t<NT, CS, PPW, 4>(packed, g, op, B, row_scale, y, y_bf16, plan, stream);
}

}  // namespace

Fp4Plan plan_fp4(int64_t B, const PackedGeom& g, const OperandShape& s) {
  (void)B;
  Fp4Plan p;
  // Two panels per workgroup when the operand is wide (reuses each operand
  // load for both). Wavefronts per workgroup: 4, or 8 when that keeps each
  // wavefront's slice within one chunk of 12 in-flight tiles (one column
  // set only; wider operands use 4 wavefronts and chunks of 6); longer
  // slices are streamed in several chunks.
  p.ppw = s.cs >= 2 ? 2 : 1;
  const int64_t groups = (g.panels + p.ppw - 1) / p.ppw;
  const int w_max = s.cs == 1 ? 8 : 4;
  int w = 4;
  auto chunk = [&](int ww) { (void)ww; return s.cs == 1 ? 12 : 6; };
  while (w < w_max && (g.ext_tiles + w - 1) / w > chunk(w)) w *= 2;
  p.waves = w;
  p.tpw = (g.ext_tiles + w - 1) / w;
  p.groups = (int)groups;
  return p;
}

hipError_t launch_sign_fp4(const uint8_t* packed, const PackedGeom& g, const OperandPlan& op,
                           int64_t B, const float* row_scale, void* y, bool y_bf16,
                           const Fp4Plan& plan, hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
#define LQ_FP4_CASE(NT_, CS_, PPW_)                                                          \
  if (op.nt == NT_ && op.cs == CS_ && plan.ppw == PPW_)                                      \
    return launch_fp4_w<NT_, CS_, PPW_>(packed, g, op, B, row_scale, y, y_bf16, plan, stream);
  LQ_FP4_CASE(3, 1, 1)
  LQ_FP4_CASE(3, 2, 2)
  LQ_FP4_CASE(2, 2, 2)
  LQ_FP4_CASE(4, 1, 1)
  LQ_FP4_CASE(4, 2, 2)
  LQ_FP4_CASE(4, 3, 2)
  LQ_FP4_CASE(4, 4, 2)
#undef LQ_FP4_CASE
  return hipErrorInvalidValue;
}

}  // namespace lq
