// One-launch decode for batch 1 split over the reduction: workgroup (kg, pg)
// takes the tiles of tile group kg (at most 6 consecutive 512-column tiles,
// the last group with the partial tail) for the 16 panels of panel group pg.
// It whitens only the Hadamard blocks its columns draw on, lifts only its
// columns, converts only its tiles to FP6 terms (all in LDS), multiplies its
// panels' slots on the FP4 x FP6 matrix cores, and hands its 256 partial row
// sums to the tile groups' last workgroup through the workspace: coherent
// stores, a per-panel-group ticket, the last one adds the partials in tile
// group order, scales the rows and writes y, and resets the ticket for the
// next launch ([paper] §3 introduction: T, the lift and the sign product
// fold into one operator; here into one launch).
//
// Against the self-sufficient one-launch decode, each workgroup prepares
// 1 / KG of the operand instead of all of it; against two launches, the
// operand never goes to memory and the weight stream starts at entry.
// Arithmetic per tile is that of the two-launch path (same transform, lift
// order, FP6 terms, MFMAs); the tile products of a row are summed per tile
// group first, then over the groups in order (deterministic).
#include <algorithm>

#include "lq_fp6_mma.h"
#include "lq_prep.h"

namespace lq {
namespace {

constexpr int kSpWaves = kOneLaunchWaves;
constexpr int kSpThreads = 64 * kSpWaves;
constexpr int kSpPanels = kSplitPanels;     // panels per workgroup (two per wavefront)
static_assert(kSpPanels == 2 * kSpWaves, "two panels per wavefront");
constexpr int kSpMaxXLoads = 10;            // x values per thread (whitened span <= 5120)
constexpr int kSpMaxTiles = 6;              // tiles per group (slots held in registers)

// XL: x values per thread (2 per 1024-input chunk of the widest span).
template <int kXKind, int DM, int XL>
__global__ __launch_bounds__(kSpThreads) void decode_split_kernel(
    const uint8_t* __restrict__ packed, int panels, int64_t panel_bytes, int full_tiles,
    int tail_bytes, int ext, int tpg, const void* __restrict__ x, int K, int d, int D, int lhb,
    float norm, const float* __restrict__ c, const float* __restrict__ M, int L, int nt, int rec,
    const float* __restrict__ row_scale, void* __restrict__ y, int y_bf16, int N,
    float* __restrict__ partial, unsigned* __restrict__ tickets, int kgroups) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int DMr = (DM + 3) & ~3;
  const int tid = threadIdx.x;
  const int wave = wave_id(), lane = tid & 63;
  const int g = lane >> 4, r = lane & 15;
  const int kg = blockIdx.x, pg = blockIdx.y;

  // ---- this workgroup's columns, blocks and inputs
  const int t0 = kg * tpg, t1 = min(t0 + tpg, ext), ntl = t1 - t0;
  const int c_lo = t0 * kTileCols, c_hi = min(t1 * kTileCols, L);
  const int b0 = c_lo / D, b1 = (c_hi - 1) / D;
  const int k_hi = min((b1 + 1) * d, K);
  // whitened span: the whole 1024-input chunks (hb divides 1024) that hold
  // inputs of the group; all of their inputs are loaded (the transform mixes
  // each hb block), zero past K
  const int kx0 = (b0 * d) & ~1023;
  const int nchunk = (k_hi - kx0 + 1023) >> 10;
  const int nx = nchunk << 10;
  const int kend = min(kx0 + nx, K);

  // LDS: records [ntl][rec] | xs [nx] | M transposed [D][DMr] | z [ntl][512]
  uint8_t* recs = smem;
  float* xs = reinterpret_cast<float*>(smem + (size_t)tpg * rec);
  float* Ms = xs + XL * kSpThreads;
  float* zt = Ms + 32 * DMr;
  __shared__ int s_last;

  // ---- inputs (unconditional: every loaded value is used, so that no
  // loaded register is waited for behind the weight loads), then the slots
  float xv[XL], cv[XL];
  const int kalt = kx0 + tid % (kend - kx0);
#pragma unroll
  for (int j = 0; j < XL; ++j) {
    const int k = kx0 + j * kSpThreads + tid;
    const int kk = k < kend ? k : kalt;
    if (kXKind == 1) xv[j] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(x)[kk]);
    else xv[j] = reinterpret_cast<const float*>(x)[kk];
    cv[j] = c[kk];
  }
  const int dD = d * D;
  const float mv = M[tid < dD ? tid : tid % dD];
  __builtin_amdgcn_s_barrier();              // every input request ahead of the weights

  // two panels per wavefront: pnl0 = 2 wave, pnl0 + 1; the tiles of the group
  const int pbase = pg * kSpPanels + 2 * wave;
  const uint8_t* prow0 = packed + (int64_t)min(pbase, panels - 1) * panel_bytes;
  const uint8_t* prow1 = packed + (int64_t)min(pbase + 1, panels - 1) * panel_bytes;
  const bool has_tail = tail_bytes > 0 && t1 == ext;         // this group holds the tail
  const int nfull = has_tail ? ntl - 1 : ntl;
  uint4 A0[kSpMaxTiles], A1[kSpMaxTiles];
#pragma unroll
  for (int q = 0; q < kSpMaxTiles; ++q) {
    const int t = min(t0 + min(q, max(nfull - 1, 0)), full_tiles - 1);
    A0[q] = load_full_slot(prow0, t, g, r);
    A1[q] = load_full_slot(prow1, t, g, r);
  }
  const uint4 T0 = load_tail_slot(prow0, has_tail ? full_tiles : 0, max(tail_bytes, 1), g, r);
  const uint4 T1 = load_tail_slot(prow1, has_tail ? full_tiles : 0, max(tail_bytes, 1), g, r);

#pragma unroll
  for (int j = 0; j < XL; ++j) {
    const int k = kx0 + j * kSpThreads + tid;
    if (j * kSpThreads + tid < nx) xs[j * kSpThreads + tid] = k < kend ? xv[j] * cv[j] : 0.0f;
  }
  if (tid < dD) {
    const int i = tid / D;
    Ms[(tid - i * D) * DMr + i] = mv * norm;
  }
  for (int jj = c_hi - c_lo + tid; jj < ntl * kTileCols; jj += kSpThreads) zt[jj] = 0.0f;
  __syncthreads();

  // ---- whitening of the span: one wavefront per 1024 values
  for (int ch = wave; ch < nchunk; ch += kSpWaves) wave_fwht_1024(xs + 1024 * ch, lhb, lane);
  __syncthreads();

  // ---- lift on the fp32 matrix cores (row tiles of 16 blocks over the
  // wavefronts); only the group's columns are stored
  mfma_lift<DM, DMr>(xs, kx0, Ms, b0, b1 - b0 + 1, d, D, K, wave, kSpWaves, lane,
                     [&](int b, int e, float v) {
                       const int col = b * D + e;
                       if (col >= c_lo && col < c_hi) zt[col - c_lo] = v;
                     });
  __syncthreads();

  // ---- FP6 terms of the group's tiles: one 32-value block per thread
  const int ncs = nt;                             // one batch row: nt columns
  for (int h = tid; h < ntl * 16; h += kSpThreads) {
    const int q = h >> 4, blk = h & 15;
    const int u = blk >> 2, gg = blk & 3;
    uint8_t* recp = recs + (size_t)q * rec;
    Fp6LaneTerms rt;
    float tp = fp6_lane_block_cols(zt + 32 * h, nt, rt);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < nt) {
        aop_store_block(recp + aop_data_offset(0, u, gg, t, ncs), rt.dw[t]);
        recp[aop_scale_offset(nt, 0, gg, t, ncs) + u] = (uint8_t)(127 + rt.e[t]);
      }
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) tp += __shfl_xor(tp, o, 16);
    if (blk == 0) *reinterpret_cast<float*>(recp + aop_tpart_offset(nt)) = tp;
  }
  __syncthreads();

  // ---- products of the wavefront's two panels with the group's tiles
  const int col = min(r, ncs - 1);
  const int boff = aop_data_offset(0, 0, g, col, ncs);
  const int soff = aop_scale_offset(nt, 0, g, col, ncs);
  const int u_str = aop_u_stride(ncs);
  const int tpoff = aop_tpart_offset(nt);
  f32x4 acc0 = (f32x4){0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
  float tacc = 0.0f;
  auto tile_mfma = [&](const uint8_t* recp, const uint4& S0, const uint4& S1) {
    i32x8 bop[4];
    const uint32_t sc = *reinterpret_cast<const uint32_t*>(recp + soff);
#pragma unroll
    for (int u = 0; u < 4; ++u) bop[u] = lds_b_operand(recp + boff + u * u_str);
    tacc += *reinterpret_cast<const float*>(recp + tpoff);
    acc0 = mfma_fp4_fp6<0>(S0.x, bop[0], sc, acc0);
    acc1 = mfma_fp4_fp6<0>(S1.x, bop[0], sc, acc1);
    acc0 = mfma_fp4_fp6<1>(S0.y, bop[1], sc, acc0);
    acc1 = mfma_fp4_fp6<1>(S1.y, bop[1], sc, acc1);
    acc0 = mfma_fp4_fp6<2>(S0.z, bop[2], sc, acc0);
    acc1 = mfma_fp4_fp6<2>(S1.z, bop[2], sc, acc1);
    acc0 = mfma_fp4_fp6<3>(S0.w, bop[3], sc, acc0);
    acc1 = mfma_fp4_fp6<3>(S1.w, bop[3], sc, acc1);
  };
#pragma unroll
  for (int q = 0; q < kSpMaxTiles; ++q)
    if (q < nfull) tile_mfma(recs + (size_t)q * rec, A0[q], A1[q]);
  if (has_tail) tile_mfma(recs + (size_t)nfull * rec, T0, T1);

  // ---- partial row sums of the group: lane (g, r = 0) of panel p holds
  // rows 4g .. 4g + 3 (the sum of the nt term columns, plus the plane sum)
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const f32x4 acc = half ? acc1 : acc0;
    const int pnl = pbase + half;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float s = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (t < nt) s += __shfl(acc[k], 16 * g + t, 64);
      if (r == 0 && pnl < panels)
        store_coherent(partial + (int64_t)kg * N + pnl * kPanelRows + 4 * g + k, s + tacc);
    }
  }

  // ---- the last of the tile groups adds the partials in group order
  if (!last_ticket(tickets + pg, kgroups, &s_last)) return;
  if (tid < kSpPanels * kPanelRows) {
    const int n = pg * kSpPanels * kPanelRows + tid;
    if (n < N) {
      float s = 0.0f;
      for (int q = 0; q < kgroups; ++q) s += load_coherent(partial + (int64_t)q * N + n);
      const float out = row_scale[n] * s;
      if (y_bf16) reinterpret_cast<uint16_t*>(y)[n] = (uint16_t)f32_to_bf16_bits(out);
      else reinterpret_cast<float*>(y)[n] = out;
    }
  }
  if (tid == 0) __hip_atomic_store(tickets + pg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int kXKind, int DM, int XL>
hipError_t launch_split_t(const uint8_t* packed, const PackedGeom& g, const void* x, int64_t K,
                          int d, int D, int hb, const float* c, const float* M, int nt, int rec,
                          const float* row_scale, void* y, bool y_bf16, const SplitPlan& plan,
                          float* partial, unsigned* tickets, hipStream_t stream) {
  int lhb = 0;
  while ((1 << lhb) < hb) ++lhb;
  const float norm = (lhb % 2 == 0) ? ldexpf(1.0f, -lhb / 2) : (float)(1.0 / sqrt((double)hb));
  static size_t allowed = 0;
  if (plan.lds_bytes > allowed) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&decode_split_kernel<kXKind, DM, XL>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)plan.lds_bytes);
    if (e != hipSuccess) return e;
    allowed = plan.lds_bytes;
  }
  return launch_timed(decode_split_kernel<kXKind, DM, XL>,
                      dim3((unsigned)plan.kgroups, (unsigned)plan.pgroups), dim3(kSpThreads),
                      plan.lds_bytes, stream, packed, (int)g.panels, g.panel_bytes, g.full_tiles,
                      g.tail_bytes, g.ext_tiles, plan.tpg, x, (int)K, d, D, lhb, norm, c, M,
                      (int)g.L, nt, rec, row_scale, y, y_bf16 ? 1 : 0, (int)g.N, partial, tickets,
                      plan.kgroups);
}

template <int kXKind, int XL>
hipError_t launch_split_d(const uint8_t* packed, const PackedGeom& g, const void* x, int64_t K,
                          int d, int D, int hb, const float* c, const float* M, int nt, int rec,
                          const float* row_scale, void* y, bool y_bf16, const SplitPlan& plan,
                          float* partial, unsigned* tickets, hipStream_t stream) {
  if (d <= 4)
    return launch_split_t<kXKind, 4, XL>(packed, g, x, K, d, D, hb, c, M, nt, rec, row_scale, y,
                                         y_bf16, plan, partial, tickets, stream);
  if (d <= 10)
    return launch_split_t<kXKind, 10, XL>(packed, g, x, K, d, D, hb, c, M, nt, rec, row_scale, y,
                                          y_bf16, plan, partial, tickets, stream);
  return launch_split_t<kXKind, 16, XL>(packed, g, x, K, d, D, hb, c, M, nt, rec, row_scale, y,
                                        y_bf16, plan, partial, tickets, stream);
}

template <int kXKind>
hipError_t launch_split_x(const uint8_t* packed, const PackedGeom& g, const void* x, int64_t K,
                          int d, int D, int hb, const float* c, const float* M, int nt, int rec,
                          const float* row_scale, void* y, bool y_bf16, const SplitPlan& plan,
                          float* partial, unsigned* tickets, hipStream_t stream) {
  switch (plan.xl) {
    case 2: return launch_split_d<kXKind, 2>(packed, g, x, K, d, D, hb, c, M, nt, rec, row_scale,
                                             y, y_bf16, plan, partial, tickets, stream);
    case 4: return launch_split_d<kXKind, 4>(packed, g, x, K, d, D, hb, c, M, nt, rec, row_scale,
                                             y, y_bf16, plan, partial, tickets, stream);
    case 6: return launch_split_d<kXKind, 6>(packed, g, x, K, d, D, hb, c, M, nt, rec, row_scale,
                                             y, y_bf16, plan, partial, tickets, stream);
    case 10: return launch_split_d<kXKind, 10>(packed, g, x, K, d, D, hb, c, M, nt, rec, row_scale,
                                               y, y_bf16, plan, partial, tickets, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

SplitPlan plan_split(int64_t B, int64_t K, int d, int D, const PackedGeom& g,
                     const OperandShape& s, int cus) {
  SplitPlan p{};
  p.ok = false;
  // (at least one full tile: the slot loads of a tail-only group read one)
  if (B != 1 || s.cs != 1 || d > 16 || D > 32 || d * D > kSpThreads || g.full_tiles < 1)
    return p;
  p.pgroups = (int)((g.panels + kSpPanels - 1) / kSpPanels);
  if (p.pgroups > kSplitTickets) return p;
  // tile groups: about one workgroup per compute unit, at most kSpMaxTiles
  // tiles each
  const int ext = g.ext_tiles;
  int kgw = std::max(1, cus / p.pgroups);
  kgw = std::max(kgw, (ext + kSpMaxTiles - 1) / kSpMaxTiles);
  kgw = std::min(kgw, ext);
  p.tpg = (ext + kgw - 1) / kgw;
  p.kgroups = (ext + p.tpg - 1) / p.tpg;
  // the whitened span of every group fits the x registers (5120 values)
  size_t xs_max = 0;
  for (int kg = 0; kg < p.kgroups; ++kg) {
    const int64_t t0 = (int64_t)kg * p.tpg, t1 = std::min<int64_t>(t0 + p.tpg, ext);
    const int64_t c_lo = t0 * kTileCols, c_hi = std::min<int64_t>(t1 * kTileCols, g.L);
    const int64_t b0 = c_lo / D, b1 = (c_hi - 1) / D;
    const int64_t k_hi = std::min<int64_t>((b1 + 1) * d, K);
    const int64_t kx0 = (b0 * d) & ~(int64_t)1023;
    xs_max = std::max<size_t>(xs_max, (size_t)((k_hi - kx0 + 1023) / 1024) * 1024);
  }
  if (xs_max > (size_t)kSpMaxXLoads * kSpThreads) return p;
  const int need = (int)(xs_max / kSpThreads);              // 2 per 1024-input chunk
  p.xl = need <= 2 ? 2 : (need <= 4 ? 4 : (need <= 6 ? 6 : 10));
  const int dmr = d <= 4 ? 4 : (d <= 10 ? 12 : 16);
  p.lds_bytes = (size_t)p.tpg * s.rec + (size_t)p.xl * kSpThreads * 4 + (size_t)32 * dmr * 4 +
                (size_t)p.tpg * kTileCols * 4;
  if (p.lds_bytes > 160 * 1024 - 256) return p;
  p.partial_bytes = (size_t)p.kgroups * g.N * sizeof(float);
  p.ok = true;
  return p;
}

hipError_t launch_decode_split(const uint8_t* packed, const PackedGeom& g, const void* x,
                               bool x_bf16, int64_t K, int d, int D, int hb, const float* c,
                               const float* M, const OperandShape& s, const float* row_scale,
                               void* y, bool y_bf16, const SplitPlan& plan, float* partial,
                               unsigned* tickets, hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
  if (!plan.ok || d > 16) return hipErrorInvalidValue;
  return x_bf16 ? launch_split_x<1>(packed, g, x, K, d, D, hb, c, M, s.nt, s.rec, row_scale, y,
                                    y_bf16, plan, partial, tickets, stream)
                : launch_split_x<0>(packed, g, x, K, d, D, hb, c, M, s.nt, s.rec, row_scale, y,
                                    y_bf16, plan, partial, tickets, stream);
}

}  // namespace lq
