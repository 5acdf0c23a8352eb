// One-launch decode for batch 1 with no communication between workgroups:
// every workgroup prepares the whole activation operand of the layer itself
// (whitening, lift and FP6 terms, all in LDS), then multiplies its own 4 or 8
// panels by it on the FP4 x FP6 matrix cores ([paper] §3 introduction: T and
// the lift fold into the operator that multiplies the packed signs).
//
// Worth it where the preparation is small next to what it saves (a launch
// and its gap, the operand's trip through memory, the product's own wait for
// its first operand): layers with short rows, whose operand fits LDS next to
// the transformed input. The weight stream overlaps the preparation: every
// wavefront requests all its slots right after the input loads (a barrier
// between the two keeps the inputs ahead of the weights in the unit's queue).
//
// Four panels per workgroup, two wavefronts per panel: wavefront w works on
// panel w % 4 and on the tiles t with t % 2 == w / 4 of it (so twice as many
// compute units share the matrix work as with one wavefront per panel, and
// each holds half a panel's slots in registers); the two partial sums of a
// panel meet in LDS. Arithmetic is that of the two-launch path: the same transform,
// lift order and FP6 terms, and the same MFMA per tile; only the order in
// which tile products are summed differs.
#include <algorithm>

#include "lq_fp6_mma.h"
#include "lq_prep.h"

namespace lq {
namespace {

constexpr int kSelfWaves = kOneLaunchWaves;
constexpr int kSelfThreads = 64 * kSelfWaves;
constexpr int kSelfMaxTiles = 20;        // full tiles of a panel (registers of its 2 wavefronts)

// DM: an upper bound of d (the lift keeps a block's inputs in registers).
// XL: x values per thread (K <= 512 XL).
template <int kXKind, int DM, int XL>
__global__ __launch_bounds__(kSelfThreads) void decode_self_kernel(
    const uint8_t* __restrict__ packed, int panels, int64_t panel_bytes, int full_tiles,
    int tail_bytes, const void* __restrict__ x, int K, int Kx, int d, int D, int lhb, float norm,
    const float* __restrict__ c, const float* __restrict__ M, int L, int nt, int rec,
    const float* __restrict__ row_scale, void* __restrict__ y, int y_bf16) {
  constexpr int NH = 2;                                  // wavefronts per panel
  constexpr int kPw = kSelfWaves / NH;                   // panels per workgroup
  constexpr int kSlots = (kSelfMaxTiles + NH - 1) / NH;  // full-tile slots per wavefront
  constexpr int DMr = (DM + 3) & ~3;
  extern __shared__ __align__(16) uint8_t smem[];
  const bool has_tail = tail_bytes > 0;
  const int ext = full_tiles + (has_tail ? 1 : 0);
  const int tid = threadIdx.x;
  const int wave = wave_id(), lane = tid & 63;
  const int g = lane >> 4, r = lane & 15;
  const int pw_idx = wave % kPw, half = wave / kPw;
  // LDS: records [ext][rec], then xs [Kx] (x * c, transformed; Kx = K rounded
  // up to 1024, zero past K), M transposed [D][DMr] (column e's d entries
  // contiguous), z [ext][512] (lifted values in column order, zero past L),
  // the partial sums [kPw][64][5].
  uint8_t* recs = smem;
  float* xs = reinterpret_cast<float*>(smem + (size_t)ext * rec);
  float* Ms = xs + Kx;
  float* zt = Ms + D * DMr;
  float* part = zt + ext * kTileCols;

  // ---- input loads, all unconditional (a load under a branch is waited for
  // at the branch's end); an index past the end reads an element the
  // thread's first load covers (spread over the array: every workgroup reads
  // these, and one hot line would queue them).
  float xv[XL], cv[XL];
  const int kalt = tid % K;
  auto load_x = [&](int j) {
    const int k = j * kSelfThreads + tid < K ? j * kSelfThreads + tid : kalt;
    if (kXKind == 1) xv[j] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(x)[k]);
    else xv[j] = reinterpret_cast<const float*>(x)[k];
    cv[j] = c[k];
  };
#pragma unroll
  for (int j = 0; j < XL; ++j) load_x(j);
  constexpr int kMPer = 8;                   // M values per thread (d * D <= 4096)
  float mv[kMPer];
  const int malt = tid % (d * D);
#pragma unroll
  for (int j = 0; j < kMPer; ++j)
    mv[j] = M[j * kSelfThreads + tid < d * D ? j * kSelfThreads + tid : malt];
  // every wavefront's input requests go out before any weight request
  __builtin_amdgcn_s_barrier();

  // ---- weight slots: the tail's bytes first (they are assembled at once),
  // then the full tiles of this wavefront's share. Every wavefront makes the
  // same number of loads, so all run one instruction stream whose waits
  // count the same loads; loads past the share repeat its last tile.
  const int pnl = min((int)blockIdx.x * kPw + pw_idx, panels - 1);
  const uint8_t* prow = packed + (int64_t)pnl * panel_bytes;
  const bool owns_tail = has_tail && full_tiles % NH == half;
  // (without the tail, a harmless in-bounds read of the first tile instead)
  const uint4 At = load_tail_slot(prow, owns_tail ? full_tiles : 0, max(tail_bytes, 1), g, r);
  uint4 A[kSlots];
#pragma unroll
  for (int j = 0; j < kSlots; ++j)
    A[j] = load_full_slot(prow, min(half + NH * j, full_tiles - 1), g, r);
  // the loaded inputs are all used here (a loaded register left unused would
  // be reused later, and waited for there, behind every weight load)
#pragma unroll
  for (int j = 0; j < XL; ++j) asm volatile("" ::"v"(xv[j]), "v"(cv[j]));
#pragma unroll
  for (int j = 0; j < kMPer; ++j) asm volatile("" ::"v"(mv[j]));

#pragma unroll
  for (int j = 0; j < XL; ++j) {
    const int k = j * kSelfThreads + tid;
    if (k < Kx) xs[k] = k < K ? xv[j] * cv[j] : 0.0f;
  }
#pragma unroll
  for (int j = 0; j < kMPer; ++j) {
    const int idx = j * kSelfThreads + tid, i = idx / D;
    if (idx < d * D) Ms[(idx - i * D) * DMr + i] = mv[j] * norm;
  }
  // zero the lifted tail of the last tile (columns >= L)
  for (int jj = L + tid; jj < ext * kTileCols; jj += kSelfThreads) zt[jj] = 0.0f;
  __syncthreads();

  // ---- whitening: one wavefront per 1024 values
  for (int ch = wave; ch * 1024 < Kx; ch += kSelfWaves) wave_fwht_1024(xs + 1024 * ch, lhb, lane);
  __syncthreads();

  // ---- lift on the fp32 matrix cores, row tiles of 16 blocks over the
  // wavefronts
  mfma_lift<DM, DMr>(xs, 0, Ms, 0, (K + d - 1) / d, d, D, K, wave, kSelfWaves, lane,
                     [&](int b, int e, float v) { zt[b * D + e] = v; });
  __syncthreads();

  // ---- FP6 terms: one 32-value block per thread (16 per tile)
  const int ncs = nt;                            // one batch row: nt columns
  for (int h = tid; h < ext * 16; h += kSelfThreads) {
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
    // the tile's 16 blocks are 16 consecutive lanes
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) tp += __shfl_xor(tp, o, 16);
    if (blk == 0) *reinterpret_cast<float*>(recp + aop_tpart_offset(nt)) = tp;
  }
  __syncthreads();

  // ---- product of this wavefront's share of its panel with the records
  const int col = min(r, ncs - 1);
  const int boff = aop_data_offset(0, 0, g, col, ncs);
  const int soff = aop_scale_offset(nt, 0, g, col, ncs);
  const int u_str = aop_u_stride(ncs);
  const int tpoff = aop_tpart_offset(nt);
  f32x4 acc = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  float tacc = 0.0f;
  auto tile_mfma = [&](const uint8_t* recp, const uint4& S) {
    i32x8 bop[4];
    const uint32_t sc = *reinterpret_cast<const uint32_t*>(recp + soff);
#pragma unroll
    for (int u = 0; u < 4; ++u) bop[u] = lds_b_operand(recp + boff + u * u_str);
    tacc += *reinterpret_cast<const float*>(recp + tpoff);
    acc = mfma_fp4_fp6<0>(S.x, bop[0], sc, acc);
    acc = mfma_fp4_fp6<1>(S.y, bop[1], sc, acc);
    acc = mfma_fp4_fp6<2>(S.z, bop[2], sc, acc);
    acc = mfma_fp4_fp6<3>(S.w, bop[3], sc, acc);
  };
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const int t = half + NH * j;
    if (t < full_tiles) tile_mfma(recs + (size_t)t * rec, A[j]);
  }
  if (owns_tail) tile_mfma(recs + (size_t)full_tiles * rec, At);
  {
    float* pp = part + (pw_idx * 64 + lane) * 5;
    if (half == 1) {
      pp[0] = acc[0]; pp[1] = acc[1]; pp[2] = acc[2]; pp[3] = acc[3]; pp[4] = tacc;
    }
    __syncthreads();
    if (half == 1) return;
    acc[0] += pp[0]; acc[1] += pp[1]; acc[2] += pp[2]; acc[3] += pp[3];
    tacc += pp[4];
  }

  // ---- epilogue: lane (g, r) holds rows 4g..4g+3 of the panel for record
  // column r; the row's value is the sum of its nt term columns plus the
  // plane-0..2 sum, times the row scale.
  const bool live = (int)blockIdx.x * kPw + pw_idx < panels;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float s = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (t < nt) s += __shfl(acc[k], 16 * g + t, 64);
    const int n = pnl * kPanelRows + 4 * g + k;
    if (live && r == 0) {
      const float out = row_scale[n] * (s + tacc);
      if (y_bf16) reinterpret_cast<uint16_t*>(y)[n] = (uint16_t)f32_to_bf16_bits(out);
      else reinterpret_cast<float*>(y)[n] = out;
    }
  }
}

template <int kXKind, int DM, int XL>
hipError_t launch_self_t(const uint8_t* packed, const PackedGeom& g, const void* x, int64_t K,
                         int d, int D, int hb, const float* c, const float* M, int nt, int rec,
                         const float* row_scale, void* y, bool y_bf16, const SelfPlan& plan,
                         hipStream_t stream) {
  int lhb = 0;
  while ((1 << lhb) < hb) ++lhb;
  const float norm = (lhb % 2 == 0) ? ldexpf(1.0f, -lhb / 2) : (float)(1.0 / sqrt((double)hb));
  static size_t allowed = 0;
  if (plan.lds_bytes > allowed) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&decode_self_kernel<kXKind, DM, XL>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)plan.lds_bytes);
    if (e != hipSuccess) return e;
    allowed = plan.lds_bytes;
  }
  return launch_timed(decode_self_kernel<kXKind, DM, XL>, dim3((unsigned)plan.groups),
                      dim3(kSelfThreads), plan.lds_bytes, stream, packed, (int)g.panels,
                      g.panel_bytes, g.full_tiles, g.tail_bytes, x, (int)K, plan.kx, d, D, lhb,
                      norm, c, M, (int)g.L, nt, rec, row_scale, y, y_bf16 ? 1 : 0);
}

template <int kXKind, int XL>
hipError_t launch_self_d(const uint8_t* packed, const PackedGeom& g, const void* x, int64_t K,
                         int d, int D, int hb, const float* c, const float* M, int nt, int rec,
                         const float* row_scale, void* y, bool y_bf16, const SelfPlan& plan,
                         hipStream_t stream) {
  if (d <= 4)
    return launch_self_t<kXKind, 4, XL>(packed, g, x, K, d, D, hb, c, M, nt, rec, row_scale, y,
                                        y_bf16, plan, stream);
  if (d <= 10)
    return launch_self_t<kXKind, 10, XL>(packed, g, x, K, d, D, hb, c, M, nt, rec, row_scale, y,
                                         y_bf16, plan, stream);
  return launch_self_t<kXKind, 16, XL>(packed, g, x, K, d, D, hb, c, M, nt, rec, row_scale, y,
                                       y_bf16, plan, stream);
}

template <int kXKind>
hipError_t launch_self_x(const uint8_t* packed, const PackedGeom& g, const void* x, int64_t K,
                         int d, int D, int hb, const float* c, const float* M, int nt, int rec,
                         const float* row_scale, void* y, bool y_bf16, const SelfPlan& plan,
                         hipStream_t stream) {
  // 2 x values per thread per 1024 inputs (K rounded up to 1024)
  switch (plan.kx >> 9) {
    case 2: return launch_self_d<kXKind, 2>(packed, g, x, K, d, D, hb, c, M, nt, rec, row_scale, y,
                                            y_bf16, plan, stream);
    case 4: return launch_self_d<kXKind, 4>(packed, g, x, K, d, D, hb, c, M, nt, rec, row_scale, y,
                                            y_bf16, plan, stream);
    case 6:
    case 8: return launch_self_d<kXKind, 8>(packed, g, x, K, d, D, hb, c, M, nt, rec, row_scale, y,
                                            y_bf16, plan, stream);
    default: return launch_self_d<kXKind, 16>(packed, g, x, K, d, D, hb, c, M, nt, rec, row_scale,
                                              y, y_bf16, plan, stream);
  }
}

}  // namespace

SelfPlan plan_self(int64_t B, int64_t K, int d, int D, const PackedGeom& g, const OperandShape& s) {
  SelfPlan p{};
  p.ok = false;
  // One batch row; every slot of a panel held in registers; the input in one
  // round of loads; at least one full tile (the tail's slot load reads it).
  if (B != 1 || g.full_tiles > kSelfMaxTiles || g.full_tiles < 1 || s.cs != 1 || K > 8192 ||
      d > 16)
    return p;
  p.kx = (int)((K + 1023) / 1024) * 1024;
  p.pw = kSelfWaves / 2;
  p.groups = (int)((g.panels + p.pw - 1) / p.pw);
  const int dmr = d <= 4 ? 4 : (d <= 10 ? 12 : 16);      // padded M row of the instance
  p.lds_bytes = (size_t)g.ext_tiles * s.rec + (size_t)p.kx * 4 + (size_t)D * dmr * 4 +
                (size_t)g.ext_tiles * kTileCols * 4 + (size_t)p.pw * 64 * 5 * 4;
  if (p.lds_bytes > 160 * 1024) return p;
  p.ok = true;
  return p;
}

hipError_t launch_decode_self(const uint8_t* packed, const PackedGeom& g, const void* x,
                              bool x_bf16, int64_t K, int d, int D, int hb, const float* c,
                              const float* M, const OperandShape& s, const float* row_scale,
                              void* y, bool y_bf16, const SelfPlan& plan, hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
  if (!plan.ok || d > 16 || plan.pw != kSelfWaves / 2) return hipErrorInvalidValue;
  return x_bf16 ? launch_self_x<1>(packed, g, x, K, d, D, hb, c, M, s.nt, s.rec, row_scale, y,
                                   y_bf16, plan, stream)
                : launch_self_x<0>(packed, g, x, K, d, D, hb, c, M, s.nt, s.rec, row_scale, y,
                                   y_bf16, plan, stream);
}

}  // namespace lq
