// Sign products on the bf16 matrix cores (gfx950 v_mfma_f32_16x16x32_bf16).
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

// ------------------------------------------------------------ small batch
// B <= 16. One wavefront per 16-row panel and column range; the 16 MFMA
// columns are the batch rows. LDS holds the range's z as bf16 pairs:
// zl[term][b][G*16 + p] (b < B) with a per-row stride of groups*16 + 4 dwords
// (padding that spreads the 16 batch rows over distinct LDS banks).
template <bool kZBF16, int NTERM>
__global__ __launch_bounds__(256) void sign_mfma_small_kernel(
    const uint8_t* __restrict__ packed, int64_t panels, int64_t panel_bytes, int full_tiles,
    int tail_bytes, int ext_tiles, const void* __restrict__ z, int64_t B, int64_t L, int tps,
    float* __restrict__ partial, int64_t N) {
  extern __shared__ uint32_t zl[];
  const int ks = blockIdx.y;
  const int q0 = ks * tps;
  const int q1 = min(q0 + tps, ext_tiles);
  const int groups = (q1 - q0) * (kTileCols / 32);
  const int cs = groups * 16 + 4;
  const int bn = (int)B;                       // <= 16
  const int64_t c0 = (int64_t)q0 * kTileCols;

  const int per_term = bn * groups * 16;
  for (int idx = threadIdx.x; idx < NTERM * per_term; idx += blockDim.x) {
    const int term = idx / per_term;
    const int rem = idx - term * per_term;
    const int b = rem / (groups * 16);
    const int gp = rem - b * (groups * 16);
    const int G = gp >> 4, p = gp & 15;
    zl[(term * bn + b) * cs + gp] = zpair<kZBF16>(z, b, c0 + 32 * G + p, B, L, term);
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, r = lane & 15;
  const int64_t pnl = (int64_t)blockIdx.x * 4 + wave;
  if (pnl >= panels) return;
  const uint8_t* panel = packed + pnl * panel_bytes;
  const bool has_col = r < bn;

  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int q = q0; q < q1; ++q) {
    const uint4 sl = load_slot(panel, q, full_tiles, tail_bytes, g, r);
    const uint32_t w4[4] = {sl.x, sl.y, sl.z, sl.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int G = (q - q0) * 16 + 4 * u + g;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 a = sign_operand(w4[u], s);
#pragma unroll
        for (int term = 0; term < NTERM; ++term) {
          u32x4 bop = {0u, 0u, 0u, 0u};
          if (has_col) bop = *reinterpret_cast<const u32x4*>(zl + (term * bn + r) * cs + G * 16 + 4 * s);
          acc = mfma_bf16(a, bop, acc);
        }
      }
    }
  }
  // Lane (g, r) holds rows 4g..4g+3 of the panel for batch row r.
  if (has_col) {
    float* dst = partial + ((int64_t)ks * B + r) * N + pnl * kPanelRows + 4 * g;
    *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  }
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

constexpr int kSmallLdsDwords = 16384;   // 64 KiB

template <int PPW, bool kYBF16>
hipError_t launch_large_ppw(const uint8_t* packed, const PackedGeom& g, const void* z, bool z_bf16,
                            int64_t B, const float* row_scale, void* y, hipStream_t stream) {
  const dim3 grid((unsigned)((g.panels + 4 * PPW - 1) / (4 * PPW)), (unsigned)((B + 63) / 64));
  if (z_bf16)
    hipLaunchKernelGGL((sign_mfma_large_kernel<true, 1, PPW, kYBF16>), grid, dim3(256), 0, stream,
                       packed, g.panels, g.panel_bytes, g.full_tiles, g.tail_bytes, g.ext_tiles, z,
                       B, g.L, row_scale, y, g.N);
  else
    hipLaunchKernelGGL((sign_mfma_large_kernel<false, 2, PPW, kYBF16>), grid, dim3(256), 0, stream,
                       packed, g.panels, g.panel_bytes, g.full_tiles, g.tail_bytes, g.ext_tiles, z,
                       B, g.L, row_scale, y, g.N);
  return hipGetLastError();
}

}  // namespace

SplitPlan plan_mfma_small(int64_t B, const PackedGeom& g, bool z_bf16) {
  SplitPlan p;
  p.batch_tile = 16;
  const int64_t wgx = (g.panels + 3) / 4;
  int64_t ks = (1024 + wgx - 1) / wgx;
  // LDS: nterm x B rows x (tps * 256 + 4) dwords <= 16384.
  const int bn = (int)(B < 1 ? 1 : B);
  const int nterm = z_bf16 ? 1 : 2;
  int max_tps = (kSmallLdsDwords / (nterm * bn) - 4) / 256;
  if (max_tps < 1) max_tps = 1;
  const int64_t ks_lds = (g.ext_tiles + max_tps - 1) / max_tps;
  if (ks < ks_lds) ks = ks_lds;
  if (ks > g.ext_tiles) ks = g.ext_tiles;
  if (ks < 1) ks = 1;
  int tps = (int)((g.ext_tiles + ks - 1) / ks);
  if (tps > max_tps) tps = max_tps;
  p.tiles_per_split = tps;
  p.ksplit = (g.ext_tiles + tps - 1) / tps;
  p.ws_bytes = (size_t)p.ksplit * B * g.N * sizeof(float);
  return p;
}

hipError_t launch_sign_mfma_small(const uint8_t* packed, const PackedGeom& g, const void* z,
                                  bool z_bf16, int64_t B, const SplitPlan& plan, float* partial,
                                  hipStream_t stream) {
  const dim3 grid((unsigned)((g.panels + 3) / 4), (unsigned)plan.ksplit);
  const int nterm = z_bf16 ? 1 : 2;
  const size_t lds = (size_t)nterm * B * (plan.tiles_per_split * 256 + 4) * sizeof(uint32_t);
  if (z_bf16)
    hipLaunchKernelGGL((sign_mfma_small_kernel<true, 1>), grid, dim3(256), lds, stream, packed,
                       g.panels, g.panel_bytes, g.full_tiles, g.tail_bytes, g.ext_tiles, z, B, g.L,
                       plan.tiles_per_split, partial, g.N);
  else
    hipLaunchKernelGGL((sign_mfma_small_kernel<false, 2>), grid, dim3(256), lds, stream, packed,
                       g.panels, g.panel_bytes, g.full_tiles, g.tail_bytes, g.ext_tiles, z, B, g.L,
                       plan.tiles_per_split, partial, g.N);
  return hipGetLastError();
}

hipError_t launch_sign_mfma_large(const uint8_t* packed, const PackedGeom& g, const void* z,
                                  bool z_bf16, int64_t B, const float* row_scale, void* y,
                                  bool y_bf16, hipStream_t stream) {
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
