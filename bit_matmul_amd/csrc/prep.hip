// Activation preparation for the small-batch sign products (B <= 16), fused
// into one launch per call: whitening xt = H_hb (c .* x), the lift
// z[j*D + e] = sum_i M[i][e] xt[j*d + i], and the operand format the sign
// product reads.
//
// One 512-thread workgroup per (512-column lifted tile q, batch row b). The tile's
// lifted columns need the original columns [k_lo, k_hi) of its d-blocks;
// the workgroup loads the whole Hadamard blocks covering them into LDS,
// transforms them in place (at most 2048 values: a tile spans at most 640
// original columns), lifts, and writes either
//   - fp32 z (the VALU product's input), or
//   - the FP6 operand of the FP4 x FP6 matrix-core product (record layout in
//     lq_internal.h): each 32-value block of the operand (the values one
//     MFMA lane supplies: MFMA u, lane group g) is pre-multiplied by the
//     factor of the sign-bit plane it meets (-4, -2, -1 or +1), then cut into
//     nt terms; term t is the E2M3 rounding of the residual left by terms
//     < t under its own power-of-two block scale (the largest that keeps the
//     block's residual within E2M3's range). One lane converts one block
//     with the packed conversion instructions. The record also gets the sum
//     over the tile's plane-0..2 columns of the values the terms represent.
// Workgroup (0, 0) also clears the split-K tickets of the VALU product that
// follows on the same stream. One launch can prepare several layers that read
// the same x (their tiles one after another along the grid's x dimension).
#include "lq_prep.h"

namespace lq {
namespace {

constexpr int kThreads = 512;

// kMode 0: write fp32 z. kMode 1: write the FP6 operand.
// kXKind 0: x fp32, 1: x bf16, 2: input is already-lifted z in fp32,
// 3: already-lifted z in bf16 (whitening and lift skipped).
// Index arithmetic is 32-bit (K, L < 2^31 is checked on the host).
template <int kMode, int kXKind>
__global__ __launch_bounds__(kThreads) void prep_kernel(
    const void* __restrict__ x, int B, int K, PrepTable tab,
    float* __restrict__ zf32,                      // kMode 0: B x L
    int nt, int ncv, int rec, unsigned* __restrict__ tickets, int n_tickets) {
  __shared__ __align__(16) float xs[kSpanMax];
  __shared__ __align__(16) float zt[kTileCols];   // kMode 1: fp6_slot layout, plane factors applied
  __shared__ float Ms[64 * 64];
  // this workgroup's layer (a wave-uniform choice among at most kMultiMax)
  int li = 0;
#pragma unroll
  for (int i = 1; i < kMultiMax; ++i)
    if (i < tab.n && (int)blockIdx.x >= tab.l[i].tile_begin) li = i;
  const PrepLayer& ly = tab.l[li];
  const int d = ly.d, D = ly.D, lhb = ly.lhb, L = ly.L;
  const float norm = ly.norm;
  const float* __restrict__ c = ly.c;
  const float* __restrict__ M = ly.M;
  uint8_t* __restrict__ aop = ly.aop;
  const int q = (int)blockIdx.x - ly.tile_begin;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;

  if (blockIdx.x == 0 && b == 0)
    for (int i = tid; i < n_tickets; i += blockDim.x) tickets[i] = 0u;

  const int c_lo = q * kTileCols;
  const int width = min(kTileCols, L - c_lo);

  if (kXKind <= 1) {
    // Original columns [k_lo, k_hi) feed this tile's d-blocks; load the
    // whole Hadamard blocks that cover them.
    const int hb = 1 << lhb;
    const int j_lo = c_lo / D, j_hi = (c_lo + width - 1) / D + 1;
    const int k_lo = j_lo * d;
    const int k_hi = min(j_hi * d, K);
    const int h_lo = k_lo < K ? (k_lo >> lhb) << lhb : 0;
    const int span = k_lo < K ? (((k_hi - 1) >> lhb) + 1) * hb - h_lo : 0;
    const int64_t xrow = (int64_t)b * K;
    // Every global load of the thread first (x, c and M), then the LDS stores.
    float xv[kSpanMax / kThreads], cv[kSpanMax / kThreads], mv[4096 / kThreads];
#pragma unroll
    for (int j = 0; j < kSpanMax / kThreads; ++j) {
      const int i = tid + kThreads * j;
      const int k = h_lo + (i < span ? i : 0);
      if (kXKind == 1) xv[j] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(x)[xrow + k]);
      else xv[j] = reinterpret_cast<const float*>(x)[xrow + k];
      cv[j] = c[k];
    }
#pragma unroll
    for (int j = 0; j < 4096 / kThreads; ++j) {
      const int i = tid + kThreads * j;
      mv[j] = M[i < d * D ? i : 0];
    }
    // Unconditional stores (entries past span and d*D are never read).
#pragma unroll
    for (int j = 0; j < kSpanMax / kThreads; ++j) xs[tid + kThreads * j] = xv[j] * cv[j];
#pragma unroll
    for (int j = 0; j < 4096 / kThreads; ++j) Ms[tid + kThreads * j] = mv[j] * norm;   // fold 1/sqrt(hb) into M
    __syncthreads();
    // Fast Walsh-Hadamard transform of each hb-block of the span, 1024
    // values per 256 threads (hb divides 1024; values past the span are
    // transformed too and never read). Ends with a workgroup barrier.
    block_fwht_1024(xs + 1024 * (tid >> 8), lhb, tid & 255, 1024 * (tid >> 8) < span);
    // Lift the tile: one column per thread, d multiply-adds.
#pragma unroll
    for (int jr = 0; jr < kTileCols / kThreads; ++jr) {
      const int jj = tid + kThreads * jr;
      const float z = jj < width ? lift_column(Ms, xs, c_lo + jj, d, D, K, h_lo) : 0.0f;
      if (kMode == 1) {
        float f;
        const int slot = fp6_slot(jj, f);
        zt[slot] = f * z;
      } else {
        zt[jj] = z;
      }
    }
  } else {
    const int64_t zrow = (int64_t)b * L + c_lo;
    float v[kTileCols / kThreads];
#pragma unroll
    for (int jr = 0; jr < kTileCols / kThreads; ++jr) {
      const int jj = tid + kThreads * jr;
      const int jc = jj < width ? jj : 0;
      float t;
      if (kXKind == 3) t = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(x)[zrow + jc]);
      else t = reinterpret_cast<const float*>(x)[zrow + jc];
      v[jr] = jj < width ? t : 0.0f;
    }
#pragma unroll
    for (int jr = 0; jr < kTileCols / kThreads; ++jr) {
      const int jj = tid + kThreads * jr;
      if (kMode == 1) {
        float f;
        const int slot = fp6_slot(jj, f);
        zt[slot] = f * v[jr];
      } else {
        zt[jj] = v[jr];
      }
    }
  }
  __syncthreads();

  if (kMode == 0) {
    const int64_t zrow = (int64_t)b * L + c_lo;
#pragma unroll
    for (int jr = 0; jr < kTileCols / kThreads; ++jr) {
      const int jj = tid + kThreads * jr;
      if (jj < width) zf32[zrow + jj] = zt[jj];
    }
    return;
  }

  // ---- FP6 operand (kMode 1): lane h < 16 of the first wavefront converts
  // block h = (u, g) = (h / 4, h % 4) of the tile.
  if (tid >= 16) return;
  uint8_t* recp = aop + (int64_t)q * rec;
  const int u = tid >> 2, g = tid & 3;
  Fp6LaneTerms r;
  float tp = fp6_lane_block(zt, tid, nt, r);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (t < nt) {
      const int cc = b * nt + t, cs = cc >> 4, cl = cc & 15;
      const int ncs = min(16, ncv - 16 * cs);
      aop_store_block(recp + aop_data_offset(cs, u, g, cl, ncs), r.dw[t]);
      recp[aop_scale_offset(ncv, cs, g, cl, ncs) + u] = (uint8_t)(127 + r.e[t]);
    }
  }
  // Plane-0..2 sum over the tile's 16 blocks (fixed-order butterfly).
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) tp += __shfl_xor(tp, o, 16);
  if (tid == 0) *reinterpret_cast<float*>(recp + aop_tpart_offset(ncv) + 4 * b) = tp;
}

template <int kMode, int kXKind>
hipError_t launch_prep_t(const void* x, int64_t B, int64_t K, const PrepTable& tab, int tiles,
                         float* zf32, const OperandShape* s, unsigned* tickets, int n_tickets,
                         hipStream_t stream) {
  const int nt = s ? s->nt : 0, ncv = s ? s->ncv : 0, rec = s ? s->rec : 0;
  hipLaunchKernelGGL((prep_kernel<kMode, kXKind>), dim3((unsigned)tiles, (unsigned)B), dim3(kThreads),
                     0, stream, x, (int)B, (int)K, tab, zf32, nt, ncv, rec, tickets, n_tickets);
  return hipGetLastError();
}

PrepLayer prep_layer(int d, int D, int hb, const float* c, const float* M, int64_t L, uint8_t* aop,
                     int tile_begin) {
  PrepLayer l;
  int k = 0;
  while ((1 << k) < hb) ++k;
  l.norm = (k % 2 == 0) ? ldexpf(1.0f, -k / 2) : (float)(1.0 / sqrt((double)hb));
  l.d = d;
  l.D = D;
  l.lhb = k;
  l.L = (int)L;
  l.c = c;
  l.M = M;
  l.aop = aop;
  l.tile_begin = tile_begin;
  return l;
}

hipError_t launch_prep_table(const void* x, int xkind, int64_t B, int64_t K, const PrepTable& tab,
                             int tiles, float* zf32, const OperandShape* s, unsigned* tickets,
                             int n_tickets, hipStream_t stream) {
  if (s == nullptr) {
    switch (xkind) {
      case 0: return launch_prep_t<0, 0>(x, B, K, tab, tiles, zf32, s, tickets, n_tickets, stream);
      case 1: return launch_prep_t<0, 1>(x, B, K, tab, tiles, zf32, s, tickets, n_tickets, stream);
      case 2: return launch_prep_t<0, 2>(x, B, K, tab, tiles, zf32, s, tickets, n_tickets, stream);
      default: return launch_prep_t<0, 3>(x, B, K, tab, tiles, zf32, s, tickets, n_tickets, stream);
    }
  }
  switch (xkind) {
    case 0: return launch_prep_t<1, 0>(x, B, K, tab, tiles, zf32, s, tickets, n_tickets, stream);
    case 1: return launch_prep_t<1, 1>(x, B, K, tab, tiles, zf32, s, tickets, n_tickets, stream);
    case 2: return launch_prep_t<1, 2>(x, B, K, tab, tiles, zf32, s, tickets, n_tickets, stream);
    default: return launch_prep_t<1, 3>(x, B, K, tab, tiles, zf32, s, tickets, n_tickets, stream);
  }
}

}  // namespace

OperandShape operand_shape(int64_t B, bool z_bf16) {
  OperandShape s;
  // 4 terms for fp32 z (3 beyond B = 12, where 4 would need a fourth
  // 16-column set: about 2^-20 / 2^-15 of each 32-value block's largest
  // magnitude); 2 for bf16 z (about 2^-10: finer than a bf16 rounding of z,
  // which the large-batch path makes); at most 48 columns.
  s.nt = z_bf16 ? 2 : (4 * B > 48 ? 3 : 4);
  s.ncv = (int)B * s.nt;
  s.cs = (s.ncv + 15) / 16;
  // Records are 128-byte aligned: a cache line never holds parts of two.
  s.rec = ((400 * s.ncv + 4 * (int)B) + 127) / 128 * 128;
  return s;
}

size_t operand_bytes(int64_t L, const OperandShape& s) {
  const int64_t ext = (L + kTileCols - 1) / kTileCols;
  return (size_t)ext * s.rec + 1024;
}

hipError_t launch_prep(const void* x, int xkind, int64_t B, int64_t K, int d, int D, int hb,
                       const float* c, const float* M, int64_t L, float* zf32,
                       const OperandPlan* op, unsigned* tickets, int n_tickets,
                       hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
  PrepTable tab;
  tab.n = 1;
  tab.l[0] = prep_layer(d, D, hb, c, M, L, op ? op->aop : nullptr, 0);
  for (int i = 1; i < kMultiMax; ++i) tab.l[i] = tab.l[0];
  const int ext = (int)((L + kTileCols - 1) / kTileCols);
  return launch_prep_table(x, xkind, B, K, tab, ext, zf32, op ? &op->s : nullptr, tickets,
                           n_tickets, stream);
}

hipError_t launch_prep_multi(const void* x, bool x_bf16, int64_t B, int64_t K, int n,
                             const PrepLayerDesc* layers, const OperandShape& s,
                             hipStream_t stream) {
  (void)hipGetLastError();
  if (n < 1 || n > kMultiMax) return hipErrorInvalidValue;
  PrepTable tab;
  tab.n = n;
  int tiles = 0;
  for (int i = 0; i < n; ++i) {
    const PrepLayerDesc& l = layers[i];
    tab.l[i] = prep_layer(l.d, l.D, l.hb, l.c, l.M, l.L, l.aop, tiles);
    tiles += (int)((l.L + kTileCols - 1) / kTileCols);
  }
  for (int i = n; i < kMultiMax; ++i) tab.l[i] = tab.l[n - 1];
  return launch_prep_table(x, x_bf16 ? 1 : 0, B, K, tab, tiles, nullptr, &s, nullptr, 0, stream);
}

}  // namespace lq
