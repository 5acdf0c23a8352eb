// Large-batch sign product on the bf16 matrix cores (gfx950
// v_mfma_f32_16x16x32_bf16): a tiled GEMM for B > 16.
//
// Operand construction. In a 16x16x32 MFMA, lane l = 16*g + r supplies row r
// of the A tile and column r of the B tile, each for the 8 reduction indices
// of lane group g. A packed slot gives lane (g, r) exactly row r's bits for
// 32 columns per word (word u of slot (g, r): tile columns 128u + 32g + b), so
// the sign operand is built in registers, with no data exchange: the bf16 pair
// of A-dword j in sub-step s takes bits p = 4s + j and p + 16 of the word,
//   ((w << (15 - p)) & 0x80008000) | 0x3F803F80     (+1 = 0x3F80, -1 = 0xBF80),
// and the B operand is read from LDS where z is stored in the matching order:
// dword p of a 32-column group holds (z[p], z[p + 16]) as a bf16 pair. The
// pairing of reduction indices inside one MFMA is therefore the same for A and
// B by construction.
//
// fp32 z is carried as two bf16 terms, hi = bf16(z) and lo = bf16(z - hi), and
// each tile is multiplied twice; bf16 z is used as is. Accumulation is fp32.
#include "lq_internal.h"

namespace lq {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

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

// z value (as float) of batch row b, column col; 0 outside [0,B) x [0,L).
template <bool kZBF16>
__device__ __forceinline__ float zval(const void* z, int64_t b, int64_t col, int64_t B, int64_t L) {
  if (b >= B || col >= L) return 0.0f;
  if (kZBF16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(z)[b * L + col]);
  return reinterpret_cast<const float*>(z)[b * L + col];
}

// bf16 pair (z[col], z[col + 16]) for term 0 (hi) or 1 (lo).
template <bool kZBF16>
__device__ __forceinline__ uint32_t zpair(const void* z, int64_t b, int64_t col, int64_t B,
                                          int64_t L, int term) {
  const float v0 = zval<kZBF16>(z, b, col, B, L);
  const float v1 = zval<kZBF16>(z, b, col + 16, B, L);
  uint32_t h0 = f32_to_bf16_bits(v0), h1 = f32_to_bf16_bits(v1);
  if (term) {
    h0 = f32_to_bf16_bits(v0 - bf16_bits_to_f32(h0));
    h1 = f32_to_bf16_bits(v1 - bf16_bits_to_f32(h1));
  }
  return h0 | (h1 << 16);
}

// ------------------------------------------------------------ large batch
// Workgroup tile: (4 * PPW) panels x 64 batch rows; wavefront w owns PPW
// panels and all 64 batch rows (4 MFMA column tiles). The packed slots go
// straight from HBM into registers; z is staged through LDS one 128-column
// word step at a time (64 batch rows x 4 groups x 16 dwords per term).
template <bool kZBF16, int NTERM, int PPW, bool kYBF16>
__global__ __launch_bounds__(256) void sign_mfma_large_kernel(
    const uint8_t* __restrict__ packed, int64_t panels, int64_t panel_bytes, int full_tiles,
    int tail_bytes, int ext_tiles, const void* __restrict__ z, int64_t B, int64_t L,
    const float* __restrict__ row_scale, void* __restrict__ y, int64_t N) {
  constexpr int kCS = 4 * 16 + 4;              // dwords per batch row (64 + pad)
  __shared__ uint32_t zl[NTERM * 64 * kCS];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, r = lane & 15;
  const int64_t pbase = (int64_t)blockIdx.x * 4 * PPW + wave * PPW;
  const int64_t b0 = (int64_t)blockIdx.y * 64;

  f32x4 acc[PPW][4];
#pragma unroll
  for (int i = 0; i < PPW; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

  // Staging assignment: thread t fills batch row t/4, group t%4 (16 dwords per term).
  const int sb = threadIdx.x >> 2, sg = threadIdx.x & 3;

  for (int q = 0; q < ext_tiles; ++q) {
    uint32_t w4[PPW][4];
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int64_t pnl = pbase + i;
      if (pnl < panels) {
        const uint4 sl = load_slot(packed + pnl * panel_bytes, q, full_tiles, tail_bytes, g, r);
        w4[i][0] = sl.x; w4[i][1] = sl.y; w4[i][2] = sl.z; w4[i][3] = sl.w;
      } else {
        w4[i][0] = w4[i][1] = w4[i][2] = w4[i][3] = 0u;
      }
    }
#pragma unroll 1
    for (int u = 0; u < 4; ++u) {
      __syncthreads();
      {
        const int64_t colg = (int64_t)q * kTileCols + 128 * u + 32 * sg;
#pragma unroll
        for (int term = 0; term < NTERM; ++term) {
          uint32_t* dst = zl + (term * 64 + sb) * kCS + sg * 16;
#pragma unroll
          for (int p = 0; p < 16; ++p) dst[p] = zpair<kZBF16>(z, b0 + sb, colg + p, B, L, term);
        }
      }
      __syncthreads();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 a[PPW];
#pragma unroll
        for (int i = 0; i < PPW; ++i) a[i] = sign_operand(w4[i][u], s);
#pragma unroll
        for (int term = 0; term < NTERM; ++term) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const u32x4 bop = *reinterpret_cast<const u32x4*>(zl + (term * 64 + 16 * j + r) * kCS + g * 16 + 4 * s);
#pragma unroll
            for (int i = 0; i < PPW; ++i) acc[i][j] = mfma_bf16(a[i], bop, acc[i][j]);
          }
        }
      }
    }
  }
  // Epilogue: lane (g, r) of tile (i, j) holds rows 4g..4g+3 of panel pbase+i
  // for batch row b0 + 16j + r.
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    const int64_t pnl = pbase + i;
    if (pnl >= panels) continue;
    const int64_t n0 = pnl * kPanelRows + 4 * g;
    const float4 rs = *reinterpret_cast<const float4*>(row_scale + n0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t b = b0 + 16 * j + r;
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

template <int PPW, bool kYBF16>
hipError_t launch_large_ppw(const uint8_t* packed, const PackedGeom& g, const void* z, bool z_bf16,
                            int64_t B, const float* row_scale, void* y, hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
  const dim3 grid((unsigned)((g.panels + 4 * PPW - 1) / (4 * PPW)), (unsigned)((B + 63) / 64));
  if (z_bf16)
    return launch_timed(sign_mfma_large_kernel<true, 1, PPW, kYBF16>, grid, dim3(256), 0, stream,
                        packed, g.panels, g.panel_bytes, g.full_tiles, g.tail_bytes, g.ext_tiles, z,
                        B, g.L, row_scale, y, g.N);
  return launch_timed(sign_mfma_large_kernel<false, 2, PPW, kYBF16>, grid, dim3(256), 0, stream,
                      packed, g.panels, g.panel_bytes, g.full_tiles, g.tail_bytes, g.ext_tiles, z,
                      B, g.L, row_scale, y, g.N);
}

}  // namespace

hipError_t launch_sign_mfma_large(const uint8_t* packed, const PackedGeom& g, const void* z,
                                  bool z_bf16, int64_t B, const float* row_scale, void* y,
                                  bool y_bf16, hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
  // Four panels per wavefront when that still gives >= 512 workgroups.
  const int64_t bch = (B + 63) / 64;
  const bool big = ((g.panels + 15) / 16) * bch >= 512;
  if (big)
    return y_bf16 ? launch_large_ppw<4, true>(packed, g, z, z_bf16, B, row_scale, y, stream)
                  : launch_large_ppw<4, false>(packed, g, z, z_bf16, B, row_scale, y, stream);
  return y_bf16 ? launch_large_ppw<1, true>(packed, g, z, z_bf16, B, row_scale, y, stream)
                : launch_large_ppw<1, false>(packed, g, z, z_bf16, B, row_scale, y, stream);
}

}  // namespace lq
