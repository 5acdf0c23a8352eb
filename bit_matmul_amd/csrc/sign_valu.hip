// Sign product on the vector ALUs, fp32 throughout (the exact path):
//   y[b][n] = row_scale[n] * sum_j S[n][j] z[b][j]
// computed as  sum_j z[b][j]  -  2 * sum_{j : S[n][j] = -1} z[b][j],
// so each sign costs one bit-field extract (shared by the batch columns) plus
// a masked add per batch column: acc += z & (bit ? ~0 : 0).
//
// Work split: one wavefront per 16-row panel and column range (split-K);
// the 4 wavefronts of a workgroup take 4 consecutive panels of the same range
// and share the range's z values, staged in LDS with 4 floats of padding after
// every 32 so that the 4 lane groups (g = 0..3) hit different banks. Lane
// (g, r) streams its 16-byte slot of every tile with one 128-bit load; the
// four lane groups are summed with cross-lane shuffles at the end. Per range
// the workgroups of panel block 0 also write the column sums of z. A separate
// epilogue adds the ranges in a fixed order: no atomics, deterministic.
#include "lq_internal.h"

namespace lq {
namespace {

constexpr int kLdsFloats = 16384;   // 64 KiB of staged z per workgroup

template <int BT, bool kZBF16>
__global__ __launch_bounds__(256) void sign_valu_kernel(
    const uint8_t* __restrict__ packed, int64_t panels, int64_t panel_bytes, int full_tiles,
    int tail_bytes, int ext_tiles, const void* __restrict__ z, int64_t B, int64_t L, int tps,
    float* __restrict__ partial, float* __restrict__ colsum, int64_t N) {
  extern __shared__ float zs[];
  const int ks = blockIdx.y;
  const int64_t b0 = (int64_t)blockIdx.z * BT;
  const int q0 = ks * tps;
  const int q1 = min(q0 + tps, ext_tiles);
  const int width = (q1 - q0) * kTileCols;
  const int stride = width + width / 8;      // 4 pad floats per 32 columns
  const int64_t c0 = (int64_t)q0 * kTileCols;

  for (int idx = threadIdx.x; idx < BT * width; idx += blockDim.x) {
    const int bt = idx / width, col = idx - bt * width;
    const int64_t gb = b0 + bt, gc = c0 + col;
    float v = 0.0f;
    if (gb < B && gc < L) {
      if (kZBF16) v = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(z)[gb * L + gc]);
      else v = reinterpret_cast<const float*>(z)[gb * L + gc];
    }
    zs[bt * stride + col + 4 * (col >> 5)] = v;
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, r = lane & 15;

  if (blockIdx.x == 0 && wave == 0) {       // column sums of this range
    for (int bt = 0; bt < BT; ++bt) {
      float s = 0.0f;
      for (int col = lane; col < width; col += 64) s += zs[bt * stride + col + 4 * (col >> 5)];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
      if (lane == 0 && b0 + bt < B) colsum[(int64_t)ks * B + b0 + bt] = s;
    }
  }

  const int64_t p = (int64_t)blockIdx.x * 4 + wave;
  if (p >= panels) return;
  const uint8_t* panel = packed + p * panel_bytes;

  float acc[BT];
#pragma unroll
  for (int bt = 0; bt < BT; ++bt) acc[bt] = 0.0f;

  for (int q = q0; q < q1; ++q) {
    const uint4 s = load_slot(panel, q, full_tiles, tail_bytes, g, r);
    const uint32_t w4[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t w = w4[u];
      const int cb = (q - q0) * kTileCols + 128 * u + 32 * g;   // multiple of 32
      const float* zp = zs + cb + 4 * (cb >> 5);
#pragma unroll
      for (int b4 = 0; b4 < 8; ++b4) {
        float4 zv[BT];
#pragma unroll
        for (int bt = 0; bt < BT; ++bt)
          zv[bt] = *reinterpret_cast<const float4*>(zp + bt * stride + 4 * b4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int bit = 4 * b4 + k;
          const uint32_t m = (uint32_t)((int32_t)(w << (31 - bit)) >> 31);
#pragma unroll
          for (int bt = 0; bt < BT; ++bt) {
            const float zk = (k == 0) ? zv[bt].x : (k == 1) ? zv[bt].y : (k == 2) ? zv[bt].z : zv[bt].w;
            acc[bt] += __uint_as_float(__float_as_uint(zk) & m);
          }
        }
      }
    }
  }
#pragma unroll
  for (int bt = 0; bt < BT; ++bt) {
    acc[bt] += __shfl_xor(acc[bt], 16, 64);
    acc[bt] += __shfl_xor(acc[bt], 32, 64);
  }
  if (g == 0) {
#pragma unroll
    for (int bt = 0; bt < BT; ++bt)
      if (b0 + bt < B) partial[((int64_t)ks * B + b0 + bt) * N + p * kPanelRows + r] = -2.0f * acc[bt];
  }
}

template <bool kYBF16>
__global__ __launch_bounds__(256) void split_epilogue_kernel(const float* __restrict__ partial,
                                                             const float* __restrict__ colsum,
                                                             int ksplit, int64_t B, int64_t N,
                                                             const float* __restrict__ row_scale,
                                                             void* __restrict__ y) {
  const int64_t total = B * N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = i / N, n = i - b * N;
    float s = 0.0f;
    if (colsum)
      for (int k = 0; k < ksplit; ++k) s += colsum[(int64_t)k * B + b];
    for (int k = 0; k < ksplit; ++k) s += partial[((int64_t)k * B + b) * N + n];
    const float v = row_scale[n] * s;
    if (kYBF16) reinterpret_cast<uint16_t*>(y)[i] = (uint16_t)f32_to_bf16_bits(v);
    else reinterpret_cast<float*>(y)[i] = v;
  }
}

int max_tps_valu(int bt) { return (kLdsFloats / (bt * 576)) > 0 ? kLdsFloats / (bt * 576) : 1; }

template <int BT>
hipError_t launch_valu_bt(const uint8_t* packed, const PackedGeom& g, const void* z, bool z_bf16,
                          int64_t B, const SplitPlan& plan, float* partial, float* colsum,
                          hipStream_t stream) {
  const dim3 grid((unsigned)((g.panels + 3) / 4), (unsigned)plan.ksplit,
                  (unsigned)((B + BT - 1) / BT));
  const size_t lds = (size_t)BT * plan.tiles_per_split * 576 * sizeof(float);
  if (z_bf16)
    hipLaunchKernelGGL((sign_valu_kernel<BT, true>), grid, dim3(256), lds, stream, packed,
                       g.panels, g.panel_bytes, g.full_tiles, g.tail_bytes, g.ext_tiles, z, B, g.L,
                       plan.tiles_per_split, partial, colsum, g.N);
  else
    hipLaunchKernelGGL((sign_valu_kernel<BT, false>), grid, dim3(256), lds, stream, packed,
                       g.panels, g.panel_bytes, g.full_tiles, g.tail_bytes, g.ext_tiles, z, B, g.L,
                       plan.tiles_per_split, partial, colsum, g.N);
  return hipGetLastError();
}

}  // namespace

SplitPlan plan_valu(int64_t B, const PackedGeom& g) {
  SplitPlan p;
  int bt = 16;
  if (B <= 1) bt = 1;
  else if (B <= 2) bt = 2;
  else if (B <= 4) bt = 4;
  else if (B <= 8) bt = 8;
  p.batch_tile = bt;
  const int64_t wgx = (g.panels + 3) / 4;
  const int64_t bchunks = (B + bt - 1) / bt;
  int64_t ks = (1024 + wgx * bchunks - 1) / (wgx * bchunks);   // aim for >= 1024 workgroups
  const int max_tps = max_tps_valu(bt);
  const int64_t ks_lds = (g.ext_tiles + max_tps - 1) / max_tps;
  if (ks < ks_lds) ks = ks_lds;
  if (ks > g.ext_tiles) ks = g.ext_tiles;
  if (ks < 1) ks = 1;
  int tps = (int)((g.ext_tiles + ks - 1) / ks);
  if (tps > max_tps) tps = max_tps;
  if (tps < 1) tps = 1;
  p.tiles_per_split = tps;
  p.ksplit = (g.ext_tiles + tps - 1) / tps;
  p.ws_bytes = ((size_t)p.ksplit * B * g.N + (size_t)p.ksplit * B) * sizeof(float);
  return p;
}

hipError_t launch_sign_valu(const uint8_t* packed, const PackedGeom& g, const void* z, bool z_bf16,
                            int64_t B, const SplitPlan& plan, float* partial, float* colsum,
                            hipStream_t stream) {
  switch (plan.batch_tile) {
    case 1: return launch_valu_bt<1>(packed, g, z, z_bf16, B, plan, partial, colsum, stream);
    case 2: return launch_valu_bt<2>(packed, g, z, z_bf16, B, plan, partial, colsum, stream);
    case 4: return launch_valu_bt<4>(packed, g, z, z_bf16, B, plan, partial, colsum, stream);
    case 8: return launch_valu_bt<8>(packed, g, z, z_bf16, B, plan, partial, colsum, stream);
    default: return launch_valu_bt<16>(packed, g, z, z_bf16, B, plan, partial, colsum, stream);
  }
}

hipError_t launch_split_epilogue(const float* partial, const float* colsum, int ksplit, int64_t B,
                                 int64_t N, const float* row_scale, void* y, bool y_bf16,
                                 hipStream_t stream) {
  int64_t blocks = (B * N + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (y_bf16)
    hipLaunchKernelGGL(split_epilogue_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       partial, colsum, ksplit, B, N, row_scale, y);
  else
    hipLaunchKernelGGL(split_epilogue_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       partial, colsum, ksplit, B, N, row_scale, y);
  return hipGetLastError();
}

}  // namespace lq
