// Internal declarations of liblq: device helpers shared by the kernels and the
// launchers that the C ABI (api.cpp) calls. Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lq {

constexpr int kPanelRows = 16;     // rows per packed panel
constexpr int kTileCols = 512;     // lifted columns per full packed tile
constexpr int kTileBytes = 1024;   // 16 rows x 512 bits

// Geometry of a packed N x L sign matrix (see include/lq.h for the layout).
struct PackedGeom {
  int64_t N, L;
  int64_t panels;       // N / 16
  int64_t panel_bytes;  // 2 L
  int full_tiles;       // L / 512
  int tail_bytes;       // (L % 512) / 8 bytes per row in the tail
  int ext_tiles;        // full tiles plus one for a non-empty tail
};

inline PackedGeom make_geom(int64_t N, int64_t L) {
  PackedGeom g;
  g.N = N;
  g.L = L;
  g.panels = N / kPanelRows;
  g.panel_bytes = 2 * L;
  g.full_tiles = (int)(L / kTileCols);
  g.tail_bytes = (int)((L % kTileCols) / 8);
  g.ext_tiles = g.full_tiles + (g.tail_bytes ? 1 : 0);
  return g;
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u)               // inf / nan: keep, quiet nans
    return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
  u += 0x7fffu + ((u >> 16) & 1u);                     // round to nearest, ties to even
  return u >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// The 16-byte slot (g, r) of tile q of one panel, as four 32-bit words:
// word u, bit b = sign bit of row r at tile column 128u + 32g + b.
// For the tail tile (q == full_tiles) the words are assembled from the
// row-major tail bytes; columns beyond L read as 0 (sign +1).
__device__ __forceinline__ uint4 load_slot(const uint8_t* __restrict__ panel, int q,
                                           int full_tiles, int tail_bytes, int g, int r) {
  if (q < full_tiles) {
    return *reinterpret_cast<const uint4*>(panel + (int64_t)q * kTileBytes + 16 * (16 * g + r));
  }
  const uint8_t* row = panel + (int64_t)full_tiles * kTileBytes + r * tail_bytes;
  uint32_t w[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    uint32_t v = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      int t = 16 * u + 4 * g + k;
      if (t < tail_bytes) v |= (uint32_t)row[t] << (8 * k);
    }
    w[u] = v;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// ---------------------------------------------------------------- launchers
// Every launcher enqueues on `stream` and returns hipGetLastError().

hipError_t launch_pack(const int8_t* signs, int64_t N, int64_t L, uint8_t* packed,
                       hipStream_t stream);
hipError_t launch_unpack(const uint8_t* packed, int64_t N, int64_t L, int8_t* signs,
                         hipStream_t stream);
hipError_t launch_hadamard_scale(const void* x, bool x_bf16, int64_t B, int64_t K, int hb,
                                 const float* c, float* xt, hipStream_t stream);
hipError_t launch_lift(const float* xt, int64_t B, int64_t K, int d, int D, const float* M,
                       void* z, bool z_bf16, hipStream_t stream);

// Split-K plan shared by the panel-parallel sign products (VALU and small
// MFMA). Workspace: partial[ksplit][B][N] and colsum[ksplit][B] floats.
struct SplitPlan {
  int ksplit;           // number of column ranges
  int tiles_per_split;  // packed tiles per range
  int batch_tile;       // batch columns per workgroup (VALU) or 16 (MFMA)
  size_t ws_bytes;
};
SplitPlan plan_valu(int64_t B, const PackedGeom& g);
SplitPlan plan_mfma_small(int64_t B, const PackedGeom& g, bool z_bf16);

hipError_t launch_sign_valu(const uint8_t* packed, const PackedGeom& g, const void* z,
                            bool z_bf16, int64_t B, const SplitPlan& plan, float* partial,
                            float* colsum, hipStream_t stream);
hipError_t launch_sign_mfma_small(const uint8_t* packed, const PackedGeom& g, const void* z,
                                  bool z_bf16, int64_t B, const SplitPlan& plan, float* partial,
                                  hipStream_t stream);
// y[b][n] = row_scale[n] * (sum_k colsum[k][b] (if colsum) + sum_k partial[k][b][n])
hipError_t launch_split_epilogue(const float* partial, const float* colsum, int ksplit,
                                 int64_t B, int64_t N, const float* row_scale, void* y,
                                 bool y_bf16, hipStream_t stream);
hipError_t launch_sign_mfma_large(const uint8_t* packed, const PackedGeom& g, const void* z,
                                  bool z_bf16, int64_t B, const float* row_scale, void* y,
                                  bool y_bf16, hipStream_t stream);

}  // namespace lq
