// Sign packing into the panel/tile layout of include/lq.h, and its inverse.
// One thread per packed byte: the byte's 8 signs are 8 consecutive int8
// values of one row, read with a single 64-bit load.
#include "lq_internal.h"

namespace lq {
namespace {

// Row and first lifted column of packed byte `o` (the layout's inverse map).
__device__ __forceinline__ void byte_origin(int64_t o, int64_t L, int full_tiles, int tail_bytes,
                                            int64_t* row, int64_t* col0) {
  const int64_t panel_bytes = 2 * L;
  const int64_t p = o / panel_bytes;
  const int64_t rem = o - p * panel_bytes;
  const int64_t full = (int64_t)full_tiles * kTileBytes;
  if (rem < full) {
    const int64_t q = rem / kTileBytes;
    const int w = (int)(rem - q * kTileBytes);
    const int slot = w >> 4, u = (w >> 2) & 3, bb = w & 3;
    const int r = slot & 15, g = slot >> 4;
    *row = p * kPanelRows + r;
    *col0 = q * kTileCols + 128 * u + 32 * g + 8 * bb;
  } else {
    const int64_t t_all = rem - full;
    const int r = (int)(t_all / tail_bytes), t = (int)(t_all - (int64_t)r * tail_bytes);
    *row = p * kPanelRows + r;
    *col0 = (int64_t)full_tiles * kTileCols + 8 * t;
  }
}

__global__ __launch_bounds__(256) void pack_kernel(const int8_t* __restrict__ signs, int64_t L,
                                                   int full_tiles, int tail_bytes,
                                                   uint8_t* __restrict__ packed, int64_t total) {
  for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < total;
       o += (int64_t)gridDim.x * blockDim.x) {
    int64_t row, col0;
    byte_origin(o, L, full_tiles, tail_bytes, &row, &col0);
    const uint64_t v = *reinterpret_cast<const uint64_t*>(signs + row * L + col0);
    // Gather the sign bit (bit 7) of each of the 8 bytes into one byte:
    // multiplying by sum_j 2^(7j) moves bit 8i+7 to bit 56+i without carries.
    packed[o] = (uint8_t)(((v & 0x8080808080808080ull) * 0x0002040810204081ull) >> 56);
  }
}

__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t* __restrict__ packed, int64_t L,
                                                     int full_tiles, int tail_bytes,
                                                     int8_t* __restrict__ signs, int64_t total) {
  for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < total;
       o += (int64_t)gridDim.x * blockDim.x) {
    int64_t row, col0;
    byte_origin(o, L, full_tiles, tail_bytes, &row, &col0);
    const uint32_t byte = packed[o];
    uint64_t v = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) v |= (uint64_t)(((byte >> e) & 1u) ? 0xffu : 0x01u) << (8 * e);
    *reinterpret_cast<uint64_t*>(signs + row * L + col0) = v;
  }
}

int grid_for(int64_t total) {
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  return (int)(blocks > 0 ? blocks : 1);
}

}  // namespace

hipError_t launch_pack(const int8_t* signs, int64_t N, int64_t L, uint8_t* packed,
                       hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
  const PackedGeom g = make_geom(N, L);
  const int64_t total = N * L / 8;
  hipLaunchKernelGGL(pack_kernel, dim3(grid_for(total)), dim3(256), 0, stream, signs, L,
                     g.full_tiles, g.tail_bytes, packed, total);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* packed, int64_t N, int64_t L, int8_t* signs,
                         hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
  const PackedGeom g = make_geom(N, L);
  const int64_t total = N * L / 8;
  hipLaunchKernelGGL(unpack_kernel, dim3(grid_for(total)), dim3(256), 0, stream, packed, L,
                     g.full_tiles, g.tail_bytes, signs, total);
  return hipGetLastError();
}

}  // namespace lq
