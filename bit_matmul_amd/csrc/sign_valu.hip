// Sign product on the vector ALUs, fp32 throughout (the exact path):
//   y[b][n] = row_scale[n] * sum_j S[n][j] z[b][j]
// computed as  sum_j z[b][j]  -  2 * sum_{j : S[n][j] = -1} z[b][j],
// so each sign costs one bit-field extract (shared by the batch rows) plus a
// masked add per batch row: acc += z & (bit ? ~0 : 0).
//
// Work split: one wavefront per 16-row panel and column range of TPS tiles
// (split-K); the 4 wavefronts of a workgroup take 4 consecutive panels of the
// same range and share the range's z values, staged in LDS with 4 floats of
// padding after every 32 so that the 4 lane groups (g = 0..3) hit different
// banks. Lane (g, r) loads its 16-byte slot of every tile of the range up
// front; the four lane groups are summed with cross-lane shuffles at the
// end. Each workgroup adds the column sum of its range to its partial, takes
// a ticket, and the last workgroup of a panel group adds the partials in
// range order: no floating-point atomics, deterministic.
#include "lq_internal.h"

namespace lq {
namespace {

template <int BT, int TPS, bool kZBF16>
__global__ __launch_bounds__(256) void sign_valu_kernel(
    const uint8_t* __restrict__ packed, int64_t panels, int64_t panel_bytes, int full_tiles,
    int tail_bytes, int ext_tiles, const void* __restrict__ z, int64_t B, int64_t L,
    const float* __restrict__ row_scale, void* __restrict__ y, int y_bf16, int64_t N,
    float* __restrict__ partial, unsigned* __restrict__ tickets, int ksplit) {
  extern __shared__ float zs[];
  __shared__ float csum[BT];
  __shared__ int last_flag;
  const int tid = threadIdx.x;
  const int ks = blockIdx.y;
  const int64_t b0 = (int64_t)blockIdx.z * BT;
  const int q0 = ks * TPS;
  const int nq = min(TPS, ext_tiles - q0);
  const int width = nq * kTileCols;
  const int stride = width + width / 8;      // 4 pad floats per 32 columns
  const int64_t c0 = (int64_t)q0 * kTileCols;
  const int wave = wave_id(), lane = tid & 63;
  const int g = lane >> 4, r = lane & 15;
  const int64_t p = (int64_t)blockIdx.x * 4 + wave;

  // Full-tile slots first, at clamped always-valid addresses (no load in a
  // branch); the tail tile's bytes are assembled after z is staged.
  const int n_full = max(0, min(nq, full_tiles - q0));
  const bool has_tail = q0 + nq > full_tiles;
  const int64_t pc = min(p, panels - 1);
  uint4 slot[TPS];
  if (full_tiles > 0) {
#pragma unroll
    for (int qq = 0; qq < TPS; ++qq)
      slot[qq] = load_full_slot(packed + pc * panel_bytes, min(q0 + qq, full_tiles - 1), g, r);
  }

  // Stage z of the range: each thread issues 8 loads before its LDS stores.
  for (int base = 0; base < BT * width; base += 8 * 256) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int idx = base + j * 256 + tid;
      const int bt = idx / width, col = idx - bt * width;
      const int64_t gb = b0 + bt, gc = c0 + col;
      const bool in = idx < BT * width && gb < B && gc < L;
      const int64_t off = in ? gb * L + gc : 0;
      float t;
      if (kZBF16) t = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(z)[off]);
      else t = reinterpret_cast<const float*>(z)[off];
      v[j] = in ? t : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int idx = base + j * 256 + tid;
      const int bt = idx / width, col = idx - bt * width;
      // out-of-range stores go to the spare float after the staged ranges
      zs[idx < BT * width ? bt * stride + col + 4 * (col >> 5) : BT * TPS * 576] = v[j];
    }
  }
  uint4 tslot = make_uint4(0u, 0u, 0u, 0u);
  if (has_tail) tslot = load_tail_slot(packed + pc * panel_bytes, full_tiles, tail_bytes, g, r);
  __syncthreads();
  for (int bt = wave; bt < BT; bt += 4) {   // column sums of the range, one wave per batch row
    float s = 0.0f;
    for (int col = lane; col < width; col += 64) s += zs[bt * stride + col + 4 * (col >> 5)];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
    if (lane == 0) csum[bt] = s;
  }
  __syncthreads();

  float acc[BT];
#pragma unroll
  for (int bt = 0; bt < BT; ++bt) acc[bt] = 0.0f;
#pragma unroll
  for (int qq = 0; qq < TPS; ++qq) {
    if (qq < nq) {
      const uint4 sl = qq < n_full ? slot[qq] : tslot;
      const uint32_t w4[4] = {sl.x, sl.y, sl.z, sl.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t w = w4[u];
        const int cb = qq * kTileCols + 128 * u + 32 * g;   // multiple of 32
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
  }
#pragma unroll
  for (int bt = 0; bt < BT; ++bt) {
    acc[bt] += __shfl_xor(acc[bt], 16, 64);
    acc[bt] += __shfl_xor(acc[bt], 32, 64);
  }

  if (ksplit == 1) {
    if (g == 0 && p < panels) {
      const int64_t n = p * kPanelRows + r;
#pragma unroll
      for (int bt = 0; bt < BT; ++bt) {
        if (b0 + bt >= B) continue;
        const float v = row_scale[n] * (csum[bt] - 2.0f * acc[bt]);
        if (y_bf16) reinterpret_cast<uint16_t*>(y)[(b0 + bt) * N + n] = (uint16_t)f32_to_bf16_bits(v);
        else reinterpret_cast<float*>(y)[(b0 + bt) * N + n] = v;
      }
    }
    return;
  }
  if (g == 0 && p < panels) {
#pragma unroll
    for (int bt = 0; bt < BT; ++bt)
      if (b0 + bt < B)
        store_coherent(partial + ((int64_t)ks * B + b0 + bt) * N + p * kPanelRows + r,
                       csum[bt] - 2.0f * acc[bt]);
  }
  const int64_t group = (int64_t)blockIdx.z * gridDim.x + blockIdx.x;
  if (!last_ticket(&tickets[group], ksplit, &last_flag)) return;
  const int64_t row0 = (int64_t)blockIdx.x * 4 * kPanelRows;
  constexpr int rows = 4 * kPanelRows;
  for (int idx = tid; idx < rows * BT; idx += blockDim.x) {
    const int bt = idx / rows;
    const int64_t n = row0 + (idx - bt * rows), b = b0 + bt;
    if (n >= N || b >= B) continue;
    float s = 0.0f;
    for (int k = 0; k < ksplit; ++k) s += load_coherent(partial + ((int64_t)k * B + b) * N + n);
    const float v = row_scale[n] * s;
    if (y_bf16) reinterpret_cast<uint16_t*>(y)[b * N + n] = (uint16_t)f32_to_bf16_bits(v);
    else reinterpret_cast<float*>(y)[b * N + n] = v;
  }
}

__global__ void zero_u32_kernel(unsigned* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

template <int BT, int TPS>
hipError_t launch_valu_bt(const uint8_t* packed, const PackedGeom& g, const void* z, bool z_bf16,
                          int64_t B, const float* row_scale, void* y, bool y_bf16,
                          const ValuPlan& plan, float* partial, unsigned* tickets,
                          hipStream_t stream) {
  const dim3 grid((unsigned)((g.panels + 3) / 4), (unsigned)plan.ksplit, (unsigned)((B + BT - 1) / BT));
  const size_t lds = ((size_t)BT * TPS * 576 + 1) * sizeof(float);
  if (z_bf16)
    return launch_timed(sign_valu_kernel<BT, TPS, true>, grid, dim3(256), lds, stream, packed,
                        g.panels, g.panel_bytes, g.full_tiles, g.tail_bytes, g.ext_tiles, z, B, g.L,
                        row_scale, y, y_bf16 ? 1 : 0, g.N, partial, tickets, plan.ksplit);
  return launch_timed(sign_valu_kernel<BT, TPS, false>, grid, dim3(256), lds, stream, packed,
                      g.panels, g.panel_bytes, g.full_tiles, g.tail_bytes, g.ext_tiles, z, B, g.L,
                      row_scale, y, y_bf16 ? 1 : 0, g.N, partial, tickets, plan.ksplit);
}

}  // namespace

// Batch tile and tiles per range: LDS holds BT * TPS * 576 floats (<= 36 KiB).
ValuPlan plan_valu(int64_t B, const PackedGeom& g) {
  ValuPlan p;
  if (B <= 1) { p.bt = 1; p.tps = 4; }
  else if (B <= 2) { p.bt = 2; p.tps = 4; }
  else if (B <= 4) { p.bt = 4; p.tps = 4; }
  else if (B <= 8) { p.bt = 8; p.tps = 2; }
  else { p.bt = 16; p.tps = 1; }
  p.ksplit = (g.ext_tiles + p.tps - 1) / p.tps;
  p.groups = (int)(((g.panels + 3) / 4) * ((B + p.bt - 1) / p.bt));
  p.partial_bytes = p.ksplit > 1 ? (size_t)p.ksplit * B * g.N * sizeof(float) : 0;
  return p;
}

hipError_t launch_sign_valu(const uint8_t* packed, const PackedGeom& g, const void* z, bool z_bf16,
                            int64_t B, const float* row_scale, void* y, bool y_bf16,
                            const ValuPlan& plan, float* partial, unsigned* tickets,
                            hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
  switch (plan.bt) {
    case 1: return launch_valu_bt<1, 4>(packed, g, z, z_bf16, B, row_scale, y, y_bf16, plan, partial, tickets, stream);
    case 2: return launch_valu_bt<2, 4>(packed, g, z, z_bf16, B, row_scale, y, y_bf16, plan, partial, tickets, stream);
    case 4: return launch_valu_bt<4, 4>(packed, g, z, z_bf16, B, row_scale, y, y_bf16, plan, partial, tickets, stream);
    case 8: return launch_valu_bt<8, 2>(packed, g, z, z_bf16, B, row_scale, y, y_bf16, plan, partial, tickets, stream);
    default: return launch_valu_bt<16, 1>(packed, g, z, z_bf16, B, row_scale, y, y_bf16, plan, partial, tickets, stream);
  }
}

hipError_t launch_zero_u32(unsigned* p, int n, hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
  if (n <= 0) return hipSuccess;
  const int blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  hipLaunchKernelGGL(zero_u32_kernel, dim3(blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace lq
