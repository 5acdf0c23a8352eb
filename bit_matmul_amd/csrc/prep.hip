// Activation preparation for the small-batch sign products (B <= 16), fused
// into one launch per call: whitening xt = H_hb (c .* x), the lift
// z[j*D + e] = sum_i M[i][e] xt[j*d + i], and the operand format the sign
// product reads.
//
// One 512-thread workgroup per (512-column lifted tile q, batch row b);
// thread jj owns lifted column jj of the tile. The tile's lifted columns
// need the original columns [k_lo, k_hi) of its d-blocks; the workgroup
// brings the whole Hadamard blocks covering them (at most 2048 values: a
// tile spans at most 640 original columns) and M into registers with every
// global load issued before any is used, transforms the blocks (lanes
// exchange values on the vector ALU; one pass through LDS), lifts, and
// writes either
//   - fp32 z (the VALU product's input), or
//   - the FP6 operand of the FP4 x FP6 matrix-core product (record layout in
//     lq_internal.h): each 32-value block of the operand (the values one
//     MFMA lane supplies: MFMA u, lane group g; 32 consecutive columns of
//     the tile, so 32 consecutive threads) is pre-multiplied by the factor
//     of the sign-bit plane it meets (-4, -2, -1 or +1), then cut into nt
//     terms; term t is the E2M3 rounding (to nearest, ties to even) of the
//     residual left by terms < t under its own power-of-two block scale (the
//     largest that keeps the block's residual within E2M3's range). Every
//     thread rounds its own value; the block's largest magnitude comes from
//     a 32-lane exchange. The 6-bit codes go through LDS once to be packed
//     into the MFMA operand's dwords (code m of a block at bit 6m), 16 codes
//     (three dwords) per thread. The record also gets the sum over the
//     tile's plane-0..2 columns of the values the terms represent.
// Workgroup (0, 0) also clears the split-K tickets of the VALU product that
// follows on the same stream. One launch can prepare several layers that read
// the same x (their tiles one after another along the grid's x dimension).
#include <algorithm>

#include "lq_prep.h"

namespace lq {
namespace {

constexpr int kThreads = 512;
static_assert(kThreads == kTileCols, "one thread per lifted column of a tile");

// Largest magnitude over the 32 lanes of this lane's half-wavefront.
__device__ __forceinline__ float half_wave_absmax(float v) {
  float m = fabsf(v);
  m = fmaxf(m, lane_xor<1>(m));
  m = fmaxf(m, lane_xor<2>(m));
  m = fmaxf(m, lane_xor<4>(m));
  m = fmaxf(m, lane_xor<8>(m));
  m = fmaxf(m, lane_xor<16>(m));
  return m;
}

// Block exponent of the FP6 terms: the largest e with amax * 2^-e <= 7.5
// (0 for an all-zero block), kept at or above -126 so that the scale 2^e
// stays a normal fp32 number. Branch-free.
__device__ __forceinline__ int fp6_block_exponent(float amax) {
  const int E = __builtin_amdgcn_frexp_expf(amax) - 1;   // 2^E <= amax < 2^(E+1)
  const int e = amax <= ldexpf(kE2M3Max, E - 2) ? E - 2 : E - 1;
  return amax > 0.0f ? min(max(e, -126), 127) : 0;
}

// E2M3 code of a (|a| <= 7.5), rounded to nearest with ties to even, and
// the value it stands for. The grid step is 1/8 below 2, 1/4 in [2, 4) and
// 1/2 from 4: n = rint(|a| / step) is the code's magnitude less 0, 8 or 16
// (so n's parity is the mantissa's, and a tie goes to the even code).
__device__ __forceinline__ uint32_t e2m3_round(float a, float& rep) {
  const float aa = fabsf(a);
  const bool lo = aa < 2.0f, mid = aa < 4.0f;
  const float s = lo ? 8.0f : (mid ? 4.0f : 2.0f);
  const float n = fminf(rintf(aa * s), lo ? 16.0f : (mid ? 16.0f : 15.0f));
  const float q = n * (lo ? 0.125f : (mid ? 0.25f : 0.5f));
  rep = a < 0.0f ? -q : q;
  const uint32_t mag = (uint32_t)n + (lo ? 0u : (mid ? 8u : 16u));
  return (a < 0.0f ? 32u : 0u) | mag;
}

// The lift of one column from M's entries in registers: z = sum over
// i < min(d, K - kb) of (M[i][e] / sqrt(hb)) * xs[kb + i - h_lo], kb = blk d,
// added in order of i (mr[i] holds M[i][e] / sqrt(hb), d <= 16); the LDS
// reads are issued before any is used.
__device__ __forceinline__ float lift_regs(const float (&mr)[16], const float* xs, int blk, int d,
                                           int K, int h_lo) {
  const int kb = blk * d;
  const int nk = min(d, K - kb);
  float xv[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) xv[u] = u < nk ? xs[kb + u - h_lo] : 0.0f;
  float acc = 0.0f;
#pragma unroll
  for (int u = 0; u < 16; ++u)
    if (u < nk) acc = fmaf(mr[u], xv[u], acc);
  return acc;
}

// kMode 0: write fp32 z. kMode 1: write the FP6 operand.
// kXKind 0: x fp32, 1: x bf16, 2: input is already-lifted z in fp32,
// 3: already-lifted z in bf16 (whitening and lift skipped).
// kFast (every layer with hb = 1024 and d <= 16, the LLM rates): the
// transform's size is fixed at compile time, and each thread loads the d
// entries of M its column needs into registers with the other loads, so the
// lift reads only the transformed values from LDS; otherwise M is staged in
// LDS for any d <= 64.
// Index arithmetic is 32-bit (K, L < 2^31 is checked on the host).
template <int kMode, int kXKind, bool kFast>
__global__ __launch_bounds__(kThreads) void prep_kernel(
    const void* __restrict__ x, int B, int K, PrepTable tab,
    float* __restrict__ zf32,                      // kMode 0: B x L
    int nt, int ncv, int rec, unsigned* __restrict__ tickets, int n_tickets) {
  __shared__ __align__(16) float xs[kSpanMax];
  __shared__ float Ms[kFast ? 1 : 64 * 64];
  __shared__ __align__(16) uint8_t codes[4][kTileCols];   // [term][block * 32 + code index]
  __shared__ float tp_wave[kThreads / 64];
  // grid: (tile q, layer, batch row b); layers with fewer tiles than the
  // grid's x dimension leave the rest idle
  const PrepLayer& ly = tab.l[blockIdx.y];
  const int d = ly.d, D = ly.D, lhb = kFast ? 10 : ly.lhb, L = ly.L, tiles = ly.tiles;
  const float norm = ly.norm;
  const float* __restrict__ cvec = ly.c;
  const float* __restrict__ M = ly.M;
  uint8_t* __restrict__ aop = ly.aop;
  const int q = (int)blockIdx.x;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;

  if (q == 0 && blockIdx.y == 0 && b == 0)
    for (int i = tid; i < n_tickets; i += blockDim.x) tickets[i] = 0u;
  if (q >= tiles) return;

  const int c_lo = q * kTileCols;
  const int width = min(kTileCols, L - c_lo);
  const int jj = tid;                              // this thread's lifted column
  float z = 0.0f;

  if (kXKind <= 1) {
    const TileSpan ts = tile_span(q, K, d, D, lhb, L);
    const int64_t xrow = (int64_t)b * K;
    // Thread t of Hadamard group gi = tid / 256 brings values (t % 64) +
    // 64 j + 256 (t / 64) of the group's 1024 (clamped into the span; values
    // past it are never read), and entries tid + 512 j of M: every global
    // load is issued before any result is used.
    const int gi = tid >> 8, t = tid & 255;
    // (raw bits first: a conversion placed among the loads would wait for them)
    uint32_t xb[4];
    float cv[4], mv[4096 / kThreads];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 1024 * gi + (t & 63) + 64 * j + 256 * (t >> 6);
      const int k = ts.h_lo + (i < ts.span ? i : 0);
      if (kXKind == 1) xb[j] = reinterpret_cast<const uint16_t*>(x)[xrow + k];
      else xb[j] = reinterpret_cast<const uint32_t*>(x)[xrow + k];
      cv[j] = cvec[k];
    }
    // kFast: this thread's column c_lo + jj is element e of d-block blk
    // (c_lo / D once, then a quotient below 576 in fp32, corrected to exact)
    float mr[16];
    int blk = 0;
    if constexpr (kFast) {
      const int cq = c_lo / D, r0 = c_lo - cq * D;
      const int tt = r0 + jj;
      int bq = (int)((float)tt * (1.0f / (float)D));
      bq += (bq + 1) * D <= tt ? 1 : 0;
      bq -= bq * D > tt ? 1 : 0;
      blk = cq + bq;
      const int e = tt - bq * D;
      // (column e's address once, then a uniform row offset per entry)
      const float* __restrict__ Me = M + e;
#pragma unroll
      for (int i = 0; i < 16; ++i) mr[i] = Me[min(i, d - 1) * D];   // rows past d: never used
    } else {
      const int dD = d * D;
#pragma unroll
      for (int j = 0; j < 4096 / kThreads; ++j) {
        const int i = tid + kThreads * j;
        mv[j] = M[i < dD ? i : 0];                 // entries past d*D: stored, never read
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kFast) {
#pragma unroll
      for (int i = 0; i < 16; ++i) mr[i] *= norm;   // 1/sqrt(hb) folded in
    } else {
#pragma unroll
      for (int j = 0; j < 4096 / kThreads; ++j) Ms[tid + kThreads * j] = mv[j] * norm;
    }
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = (kXKind == 1 ? bf16_bits_to_f32(xb[j]) : __uint_as_float(xb[j])) * cv[j];
    // Hadamard transform of each hb-block (in groups of 1024; ends with a
    // workgroup barrier, so Ms is complete too)
    block_fwht_1024_regs(xs + 1024 * gi, v, lhb, t);
    if (jj < width) {
      if constexpr (kFast) z = lift_regs(mr, xs, blk, d, K, ts.h_lo);
      else z = lift_column(Ms, xs, c_lo + jj, d, D, K, ts.h_lo);
    }
  } else {
    const int64_t zi = (int64_t)b * L + c_lo + (jj < width ? jj : 0);
    float tz;
    if (kXKind == 3) tz = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(x)[zi]);
    else tz = reinterpret_cast<const float*>(x)[zi];
    z = jj < width ? tz : 0.0f;
  }

  if (kMode == 0) {
    if (jj < width) zf32[(int64_t)b * L + c_lo + jj] = z;
    return;
  }

  // ---- FP6 operand (kMode 1). Column jj: block blk = jj / 32 (MFMA u =
  // blk / 4, lane group g = blk % 4), offset r = jj % 32, sign plane
  // pl = r % 4 (factor -4, -2, -1, +1), code index m = 8 pl + r / 4.
  uint8_t* recp = aop + (int64_t)q * rec;
  const int r = jj & 31, pl = r & 3, m = 8 * pl + (r >> 2), blk = jj >> 5;
  const float f = pl == 3 ? 1.0f : (pl == 2 ? -1.0f : (pl == 1 ? -2.0f : -4.0f));
  const float v0 = f * z;                          // exact: a power of two
  float res = v0;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (t < nt) {
      const int e = fp6_block_exponent(half_wave_absmax(res));
      float rep;
      const uint32_t code = e2m3_round(ldexpf(res, -e), rep);
      res -= ldexpf(rep, e);                       // exact: the value minus its rounding
      codes[t][(jj & ~31) | m] = (uint8_t)code;
      if (r == 0) {
        const int cc = b * nt + t, cs = cc >> 4, cl = cc & 15;
        const int ncs = min(16, ncv - 16 * cs);
        recp[aop_scale_offset(ncv, cs, blk & 3, cl, ncs) + (blk >> 2)] = (uint8_t)(127 + e);
      }
    }
  }
  // Plane-0..2 sum of the represented values, divided by the plane factor
  // (fixed order: lanes by butterfly, then wavefronts in order).
  float tp = pl < 3 ? (v0 - res) * (pl == 0 ? -0.25f : (pl == 1 ? -0.5f : -1.0f)) : 0.0f;
  tp += lane_xor<1>(tp);
  tp += lane_xor<2>(tp);
  tp += lane_xor<4>(tp);
  tp += lane_xor<8>(tp);
  tp += lane_xor<16>(tp);
  tp += lane_xor<32>(tp);
  if ((tid & 63) == 0) tp_wave[tid >> 6] = tp;
  __syncthreads();

  // Codes 16 h .. 16 h + 15 of block bk, term t: three dwords of the
  // block's six (16 codes of 6 bits are 96 bits).
  if (tid < 32 * nt) {
    const int t = tid >> 5, bk = (tid >> 1) & 15, h = tid & 1;
    const uint4 w = *reinterpret_cast<const uint4*>(&codes[t][32 * bk + 16 * h]);
    uint32_t c[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x4 = i == 0 ? w.x : (i == 1 ? w.y : (i == 2 ? w.z : w.w));
#pragma unroll
      for (int k = 0; k < 4; ++k) c[4 * i + k] = (x4 >> (8 * k)) & 63u;
    }
    const uint32_t d0 = c[0] | c[1] << 6 | c[2] << 12 | c[3] << 18 | c[4] << 24 | c[5] << 30;
    const uint32_t d1 = c[5] >> 2 | c[6] << 4 | c[7] << 10 | c[8] << 16 | c[9] << 22 | c[10] << 28;
    const uint32_t d2 = c[10] >> 4 | c[11] << 2 | c[12] << 8 | c[13] << 14 | c[14] << 20 | c[15] << 26;
    const int cc = b * nt + t, cs = cc >> 4, cl = cc & 15;
    const int ncs = min(16, ncv - 16 * cs);
    uint32_t* dst = reinterpret_cast<uint32_t*>(recp + aop_data_offset(cs, bk >> 2, bk & 3, cl, ncs) + 12 * h);
    dst[0] = d0;
    dst[1] = d1;
    dst[2] = d2;
  }
  if (tid == 0) {
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) s += tp_wave[w];
    *reinterpret_cast<float*>(recp + aop_tpart_offset(ncv) + 4 * b) = s;
  }
}

template <int kMode, int kXKind>
hipError_t launch_prep_t(const void* x, int64_t B, int64_t K, const PrepTable& tab, int tiles,
                         float* zf32, const OperandShape* s, unsigned* tickets, int n_tickets,
                         hipStream_t stream) {
  const int nt = s ? s->nt : 0, ncv = s ? s->ncv : 0, rec = s ? s->rec : 0;
  bool fast = kXKind <= 1;
  for (int i = 0; i < tab.n; ++i) fast = fast && tab.l[i].lhb == 10 && tab.l[i].d <= 16;
  const dim3 grid((unsigned)tiles, (unsigned)tab.n, (unsigned)B);
  if (fast)
    hipLaunchKernelGGL((prep_kernel<kMode, kXKind, true>), grid, dim3(kThreads), 0, stream, x,
                       (int)B, (int)K, tab, zf32, nt, ncv, rec, tickets, n_tickets);
  else
    hipLaunchKernelGGL((prep_kernel<kMode, kXKind, false>), grid, dim3(kThreads), 0, stream, x,
                       (int)B, (int)K, tab, zf32, nt, ncv, rec, tickets, n_tickets);
  return hipGetLastError();
}

PrepLayer prep_layer(int d, int D, int hb, const float* c, const float* M, int64_t L, uint8_t* aop) {
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
  l.tiles = (int)((L + kTileCols - 1) / kTileCols);
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
  tab.l[0] = prep_layer(d, D, hb, c, M, L, op ? op->aop : nullptr);
  for (int i = 1; i < kMultiMax; ++i) tab.l[i] = tab.l[0];
  return launch_prep_table(x, xkind, B, K, tab, tab.l[0].tiles, zf32, op ? &op->s : nullptr,
                           tickets, n_tickets, stream);
}

hipError_t launch_prep_multi(const void* x, bool x_bf16, int64_t B, int64_t K, int n,
                             const PrepLayerDesc* layers, const OperandShape& s,
                             hipStream_t stream) {
  (void)hipGetLastError();
  if (n < 1 || n > kMultiMax) return hipErrorInvalidValue;
  PrepTable tab;
  tab.n = n;
  int tiles = 0;                                   // the grid's x dimension: the most of any layer
  for (int i = 0; i < n; ++i) {
    const PrepLayerDesc& l = layers[i];
    tab.l[i] = prep_layer(l.d, l.D, l.hb, l.c, l.M, l.L, l.aop);
    tiles = std::max(tiles, tab.l[i].tiles);
  }
  for (int i = n; i < kMultiMax; ++i) tab.l[i] = tab.l[n - 1];
  return launch_prep_table(x, x_bf16 ? 1 : 0, B, K, tab, tiles, nullptr, &s, nullptr, 0, stream);
}

}  // namespace lq
