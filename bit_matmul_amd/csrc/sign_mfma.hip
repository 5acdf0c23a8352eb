// Large-batch sign product on the bf16 matrix cores (gfx950
// v_mfma_f32_16x16x32_bf16): a tiled GEMM y = diag(r) S z^T for B > 16.
//
// Operand construction. In a 16x16x32 MFMA, lane l = 16*g + r supplies row r
// of the A tile and column r of the B tile, each for the 8 reduction indices
// of lane group g. A packed slot gives lane (g, r) exactly row r's bits for
// 32 columns per word (word u of slot (g, r): tile columns 128u + 32g + b), so
// the sign operand is built in registers, with no data exchange: the bf16 pair
// of A-dword j in sub-step s takes bits p = 4s + j and p + 16 of the word,
//   ((w << (15 - p)) & 0x80008000) | 0x3F803F80     (+1 = 0x3F80, -1 = 0xBF80),
// so the B operand of lane (g, r) in sub-step s must hold, as bf16 pairs,
// (z[c + j], z[c + j + 16]) for j = 0..3, c = 128u + 32g + 4s. The pairing of
// reduction indices inside one MFMA is the same for A and B by construction.
//
// z is first rewritten into exactly that order ("zp", one pass: from z for
// lq_sign_gemm, or straight from the lift for lq_linear): for every 16 batch
// rows and every 128-column step, a 4 KB block of 16-byte units
// [s][g][r] = the B operand of lane (g, r) in sub-step s. One 1 KB DMA then
// fills 64 consecutive units of LDS, and every LDS read of the product is
// one conflict-free 1 KB wavefront read. fp32 z is carried as two bf16
// terms, hi = bf16(z) and lo = bf16(z - hi), in two zp planes; bf16 z as is.
// Accumulation is fp32.
#include "lq_internal.h"
#include "lq_prep.h"

namespace lq {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kZpBlock = 4096;   // bytes of one (16 rows x 128 columns) zp block

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// A operand (8 bf16 +-1) of sub-step s (0..3) from one packed word.
__device__ __forceinline__ u32x4 sign_operand(uint32_t w, int s) {
  u32x4 a;
  const int p0 = 4 * s;
  a.x = ((w << (15 - p0)) & 0x80008000u) | 0x3F803F80u;
  a.y = ((w << (14 - p0)) & 0x80008000u) | 0x3F803F80u;
  a.z = ((w << (13 - p0)) & 0x80008000u) | 0x3F803F80u;
  a.w = ((w << (12 - p0)) & 0x80008000u) | 0x3F803F80u;
  return a;
}

// ------------------------------------------------------------ zp
// Workgroup (step, jb): the 4 KB block of batch rows 16 jb .. 16 jb + 15 and
// columns 128 step .. 128 step + 127; thread t = unit (s, g, r) = t.
// kSrc 0: z fp32, 1: z bf16 (B x L, row-major), 2: lift from xt (B x K fp32)
// with M (the lq_linear path: z is never written in row-major form).
template <int kSrc, int NTERM>
__global__ __launch_bounds__(256) void zp_kernel(const void* __restrict__ src, int64_t B, int64_t L,
                                                 int64_t K, int d, int D,
                                                 const float* __restrict__ M, int64_t steps,
                                                 int64_t B16, int64_t jb_base, uint4* __restrict__ zp) {
  __shared__ float Ms[kSrc == 2 ? 64 * 64 : 1];
  __shared__ __align__(16) float xs[kSrc == 2 ? 16 * 256 : 1];
  const int64_t step = blockIdx.x, jb = jb_base + blockIdx.y;
  const int t = threadIdx.x;
  const int s = t >> 6, g = (t >> 4) & 3, r = t & 15;
  const int64_t b = 16 * jb + r;
  const int64_t c0 = 128 * step + 32 * g + 4 * s;
  float v[8];                                   // z[b][c0 + j] (j < 4), z[b][c0 + 12 + j] (j >= 4)
  if (kSrc == 2) {
    // The d-blocks of columns [128 step, 128 step + 128): original columns
    // [k_lo, k_lo + span), span <= (127 / D + 2) d <= 256.
    const int64_t col_lo = 128 * step;
    const int64_t blk_lo = col_lo / D;
    const int64_t blk_hi = (min(col_lo + 127, L - 1)) / D;
    const int64_t k_lo = blk_lo * d;
    const int64_t k_hi = min((blk_hi + 1) * d, K);
    const int span = col_lo < L ? (int)(k_hi - k_lo) : 0;
    for (int i = t; i < d * D; i += 256) Ms[i] = M[i];
    for (int i = t; i < 16 * 256; i += 256) {
      const int rr = i >> 8, k = i & 255;
      const int64_t bb = 16 * jb + rr;
      xs[i] = (bb < B && k < span) ? reinterpret_cast<const float*>(src)[bb * K + k_lo + k] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t c = c0 + (j < 4 ? j : 12 + j);
      v[j] = (b < B && c < L) ? lift_column(Ms, xs + 256 * r, (int)c, d, D, (int)K, (int)k_lo) : 0.0f;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t c = c0 + (j < 4 ? j : 12 + j);
      float x = 0.0f;
      if (b < B && c < L) {
        if (kSrc == 1) x = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(src)[b * L + c]);
        else x = reinterpret_cast<const float*>(src)[b * L + c];
      }
      v[j] = x;
    }
  }
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t h0 = f32_to_bf16_bits(v[j]), h1 = f32_to_bf16_bits(v[4 + j]);
    hi[j] = h0 | (h1 << 16);
    if (NTERM == 2) {
      const uint32_t l0 = f32_to_bf16_bits(v[j] - bf16_bits_to_f32(h0));
      const uint32_t l1 = f32_to_bf16_bits(v[4 + j] - bf16_bits_to_f32(h1));
      lo[j] = l0 | (l1 << 16);
    }
  }
  const int64_t unit = (jb * steps + step) * (kZpBlock / 16) + t;
  zp[unit] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  if (NTERM == 2) zp[B16 * steps * (kZpBlock / 16) + unit] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
}

// ------------------------------------------------------------ product
// Workgroup tile: 4 * PPW panels (64 PPW rows) x 16 JB batch rows. Waves
// 0..3 compute (wave w: panels w PPW .. w PPW + PPW - 1, all JB batch
// tiles); wave 4 only copies zp blocks into LDS, one 128-column step ahead,
// alternating between two stages. The packed slots go from memory straight
// into registers, one tile (4 steps) ahead. Per step t, two workgroup
// barriers: (A) every wave is done with step t - 1, whose stage the copy of
// step t + 1 overwrites; (B) the copy of step t has landed (the loader waits
// for its copies between A and B, then issues the next step's).
template <int NTERM, int PPW, int JB, bool kYBF16>
__global__ __launch_bounds__(320) void sign_mfma_large_kernel(
    const uint8_t* __restrict__ packed, int64_t panels, int64_t panel_bytes, int full_tiles,
    int tail_bytes, int ext_tiles, const uint4* __restrict__ zp, int64_t B16, int64_t B,
    const float* __restrict__ row_scale, void* __restrict__ y, int64_t N) {
  extern __shared__ uint4 lds[];              // [stage 2][term][jb][s][g][r]
  constexpr int kStageUnits = NTERM * JB * (kZpBlock / 16);
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int g = lane >> 4, r = lane & 15;
  const int64_t steps = 4 * (int64_t)ext_tiles;
  const int64_t jb0 = (int64_t)blockIdx.y * JB;

  if (wave == 4) {
    auto copy_step = [&](int64_t t, int st) {
#pragma unroll
      for (int term = 0; term < NTERM; ++term)
#pragma unroll
        for (int j = 0; j < JB; ++j) {
          const int64_t jb = min(jb0 + j, B16 - 1);
          const uint8_t* srcb = reinterpret_cast<const uint8_t*>(zp) +
                                ((term * B16 + jb) * steps + t) * kZpBlock;
          uint8_t* dstb = reinterpret_cast<uint8_t*>(lds + st * kStageUnits) + (term * JB + j) * kZpBlock;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(srcb + 1024 * i + 16 * lane),
                                             (__attribute__((address_space(3))) void*)(dstb + 1024 * i),
                                             16, 0, 0);
        }
    };
    copy_step(0, 0);
    for (int64_t t = 0; t < steps; t += 2) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {              // step t + k, stage k
        wg_barrier();                            // (A)
        __builtin_amdgcn_s_waitcnt(0);           // the copy of step t + k
        wg_barrier();                            // (B)
        if (t + k + 1 < steps) copy_step(t + k + 1, k ^ 1);
      }
    }
    return;
  }

  const int64_t pbase = (int64_t)blockIdx.x * 4 * PPW + wave * PPW;
  const uint8_t* prow[PPW];
#pragma unroll
  for (int i = 0; i < PPW; ++i) prow[i] = packed + min(pbase + i, panels - 1) * panel_bytes;

  f32x4 acc[PPW][JB];
#pragma unroll
  for (int i = 0; i < PPW; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j) acc[i][j] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

  uint4 wn[PPW];
#pragma unroll
  for (int i = 0; i < PPW; ++i) wn[i] = load_slot(prow[i], 0, full_tiles, tail_bytes, g, r);
  for (int q = 0; q < ext_tiles; ++q) {
    uint32_t w[PPW][4];
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      w[i][0] = wn[i].x; w[i][1] = wn[i].y; w[i][2] = wn[i].z; w[i][3] = wn[i].w;
    }
    const int qn = min(q + 1, ext_tiles - 1);
#pragma unroll
    for (int i = 0; i < PPW; ++i) wn[i] = load_slot(prow[i], qn, full_tiles, tail_bytes, g, r);
#pragma unroll
    for (int u = 0; u < 4; ++u) {                // step 4q + u, stage u & 1
      wg_barrier();                              // (A)
      wg_barrier();                              // (B)
      const uint4* st = lds + (u & 1) * kStageUnits;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 a[PPW];
#pragma unroll
        for (int i = 0; i < PPW; ++i) a[i] = sign_operand(w[i][u], s);
#pragma unroll
        for (int term = 0; term < NTERM; ++term)
#pragma unroll
          for (int j = 0; j < JB; ++j) {
            const uint4 bv = st[((term * JB + j) * 4 + s) * 64 + lane];
            const u32x4 bop = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
            for (int i = 0; i < PPW; ++i) acc[i][j] = mfma_bf16(a[i], bop, acc[i][j]);
          }
      }
    }
  }

  // Epilogue: lane (g, r) of tile (i, j) holds rows 4g..4g+3 of panel
  // pbase + i for batch row 16 (jb0 + j) + r.
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    const int64_t pnl = pbase + i;
    if (pnl >= panels) continue;
    const int64_t n0 = pnl * kPanelRows + 4 * g;
    const float4 rs = *reinterpret_cast<const float4*>(row_scale + n0);
#pragma unroll
    for (int j = 0; j < JB; ++j) {
      const int64_t b = 16 * (jb0 + j) + r;
      if (b >= B) continue;
      const float v0 = rs.x * acc[i][j][0], v1 = rs.y * acc[i][j][1];
      const float v2 = rs.z * acc[i][j][2], v3 = rs.w * acc[i][j][3];
      if (kYBF16) {
        uint16_t* yp = reinterpret_cast<uint16_t*>(y) + b * N + n0;
        const uint32_t lo = f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16);
        const uint32_t hi = f32_to_bf16_bits(v2) | (f32_to_bf16_bits(v3) << 16);
        *reinterpret_cast<uint2*>(yp) = make_uint2(lo, hi);
      } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + b * N + n0) = make_float4(v0, v1, v2, v3);
      }
    }
  }
}

template <int NTERM, int PPW, int JB, bool kYBF16>
hipError_t launch_large_t(const uint8_t* packed, const PackedGeom& g, const uint4* zp, int64_t B,
                          const float* row_scale, void* y, hipStream_t stream) {
  const size_t lds = (size_t)2 * NTERM * JB * kZpBlock;
  static size_t allowed = 0;
  if (lds > 64 * 1024 && lds > allowed) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&sign_mfma_large_kernel<NTERM, PPW, JB, kYBF16>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    allowed = lds;
  }
  const int64_t B16 = (B + 15) / 16;
  const dim3 grid((unsigned)((g.panels + 4 * PPW - 1) / (4 * PPW)), (unsigned)((B16 + JB - 1) / JB));
  return launch_timed(sign_mfma_large_kernel<NTERM, PPW, JB, kYBF16>, grid, dim3(320), lds, stream,
                      packed, g.panels, g.panel_bytes, g.full_tiles, g.tail_bytes, g.ext_tiles, zp,
                      B16, B, row_scale, y, g.N);
}

template <int NTERM, bool kYBF16>
hipError_t launch_large_y(const uint8_t* packed, const PackedGeom& g, const uint4* zp, int64_t B,
                          const float* row_scale, void* y, const LargePlan& p, hipStream_t stream) {
#define LQ_LARGE_CASE(PPW_, JB_)                                                                   \
  if (p.ppw == PPW_ && p.jb == JB_)                                                                \
    return launch_large_t<NTERM, PPW_, JB_, kYBF16>(packed, g, zp, B, row_scale, y, stream);
  LQ_LARGE_CASE(2, 8) LQ_LARGE_CASE(2, 4) LQ_LARGE_CASE(2, 2) LQ_LARGE_CASE(2, 1)
  LQ_LARGE_CASE(1, 8) LQ_LARGE_CASE(1, 4) LQ_LARGE_CASE(1, 2) LQ_LARGE_CASE(1, 1)
#undef LQ_LARGE_CASE
  return hipErrorInvalidValue;
}

}  // namespace

ZpGeom zp_geom(int64_t B, const PackedGeom& g, bool z_bf16) {
  ZpGeom z;
  z.B16 = (B + 15) / 16;
  z.steps = 4 * (int64_t)g.ext_tiles;
  z.nterm = z_bf16 ? 1 : 2;
  z.bytes = (size_t)z.nterm * z.B16 * z.steps * kZpBlock;
  return z;
}

LargePlan plan_large(int64_t B, const PackedGeom& g, bool z_bf16) {
  LargePlan p;
  const int64_t B16 = (B + 15) / 16;
  p.jb = B16 >= 8 ? 8 : (B16 >= 4 ? 4 : (B16 >= 2 ? 2 : 1));
  const int64_t bt = (B16 + p.jb - 1) / p.jb;
  // Two panels per wavefront when that still gives >= 512 workgroups (more
  // would not fit the registers of two wavefronts per SIMD).
  p.ppw = ((g.panels + 7) / 8) * bt >= 512 ? 2 : 1;
  return p;
}

hipError_t launch_zp(const void* src, int kind, int64_t B, int64_t L, int64_t K, int d, int D,
                     const float* M, const PackedGeom& g, void* zp, hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
  const ZpGeom z = zp_geom(B, g, kind == 1 || kind == 3);
  uint4* out = reinterpret_cast<uint4*>(zp);
  // Batch tiles map to grid.y, at most 65535 per launch.
  for (int64_t jb0 = 0; jb0 < z.B16; jb0 += 65535) {
    const dim3 grid((unsigned)z.steps, (unsigned)min(z.B16 - jb0, (int64_t)65535));
    switch (kind) {
      case 0: hipLaunchKernelGGL((zp_kernel<0, 2>), grid, dim3(256), 0, stream, src, B, L, K, d, D, M, z.steps, z.B16, jb0, out); break;
      case 1: hipLaunchKernelGGL((zp_kernel<1, 1>), grid, dim3(256), 0, stream, src, B, L, K, d, D, M, z.steps, z.B16, jb0, out); break;
      case 2: hipLaunchKernelGGL((zp_kernel<2, 2>), grid, dim3(256), 0, stream, src, B, L, K, d, D, M, z.steps, z.B16, jb0, out); break;
      case 3: hipLaunchKernelGGL((zp_kernel<2, 1>), grid, dim3(256), 0, stream, src, B, L, K, d, D, M, z.steps, z.B16, jb0, out); break;
      default: return hipErrorInvalidValue;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_sign_mfma_large(const uint8_t* packed, const PackedGeom& g, const void* zp,
                                  bool z_bf16, int64_t B, const float* row_scale, void* y,
                                  bool y_bf16, hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
  const LargePlan p = plan_large(B, g, z_bf16);
  const uint4* z = reinterpret_cast<const uint4*>(zp);
  if (z_bf16)
    return y_bf16 ? launch_large_y<1, true>(packed, g, z, B, row_scale, y, p, stream)
                  : launch_large_y<1, false>(packed, g, z, B, row_scale, y, p, stream);
  return y_bf16 ? launch_large_y<2, true>(packed, g, z, B, row_scale, y, p, stream)
                : launch_large_y<2, false>(packed, g, z, B, row_scale, y, p, stream);
}

}  // namespace lq
