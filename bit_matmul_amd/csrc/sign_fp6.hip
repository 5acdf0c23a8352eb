// Small-batch sign product (B <= 16) on the gfx950 matrix cores:
// v_mfma_scale_f32_16x16x128_f8f6f4 with the signs as the FP4 (E2M1) A
// operand and the lifted activations as the FP6 (E2M3) B operand, whose
// per-32-value E8M0 block scales ride in the instruction's scale operand.
//
// Sign operand. A lane of a 16x16x128 MFMA supplies 32 reduction indices of
// one row: k = 32g + n for lane group g, in nibble n = 8j + i of its 4-dword
// A operand. A packed word u of slot (g, r) holds row r's signs for tile
// columns 128u + 32g + b. One word becomes one whole A operand with four
// bit operations and no shifts, by splitting its bits into the four planes
// b = 4i + j:
//   dword 0 = w & 0x11111111   nibble 0x1 = 0.5 where the bit is set, else 0
//   dword 1 = w & 0x22222222   nibble 0x2 = 1.0
//   dword 2 = w & 0x44444444   nibble 0x4 = 2.0
//   dword 3 = (w & 0x88888888) | 0x22222222   nibble = +1.0 or -1.0 (0xA)
// so nibble 8j + i meets packed column 128u + 32g + 4i + j. With the sign
// s = 1 - 2*bit, sum_j s_j z_j = sum_{plane 3} s z + sum_{planes 0-2} z
// - 2 sum_{planes 0-2} bit z: the activation operand carries z on plane 3
// and -4z, -2z, -z on planes 0, 1, 2, and the plane-0..2 column sums of z
// (stored with the operand) are added once per batch row.
//
// Activation operand (written by the preparation kernel, layout in
// lq_internal.h): per tile one record holding, for every MFMA column
// (batch row b, term t), the FP6 codes of the t-th residual term of
// 32-value blocks, the blocks' E8M0 scales, and the per-row plane sums.
//
// Work split. A workgroup owns P 16-row panels over the whole reduction
// length (no communication between workgroups), for layers whose
// activation records all fit LDS (the chunked variant in
// sign_fp6_chunked.hip streams them for the others). Every wavefront takes
// the row's tiles round-robin, keeping DEPTH tiles of slots (P 16-byte
// loads per tile) requested: no barrier couples the wavefronts until the
// end, so the weight stream never waits for another wavefront. One
// activation-operand read from LDS feeds P panels' MFMAs. Records:
//   - copied first: at entry the records go to LDS with global_load_lds,
//     with the row scales and the tail tile's packed bytes, and land before
//     any weight is requested (requested together with the weight stream
//     they would queue behind it: a compute unit returns its vector-memory
//     requests roughly in order, and the stream fills every memory queue;
//     with no copy in flight the compiler's waits for the slot loads also
//     stay exact);
//   - streamed, where that copy is long (records of at most 1 KB, as at
//     batch 1 with bf16 activations, but more than 64 KB of them: the long
//     reductions): each tile's record is requested with its slots, 16 bytes
//     per lane, into the wavefront's registers, and copied to the
//     wavefront's own 1 KB of LDS just before the tile's MFMAs read it. No
//     copy precedes the first weight request, and the waits stay exact
//     (every request is a plain load into registers).
// The wavefronts' accumulators are added in LDS in a fixed order, the terms
// and plane sums combined, the row scale applied and y written.
// Deterministic: fixed summation orders, no floating-point atomics.
#include <algorithm>

#include "lq_fp6_mma.h"

namespace lq {
namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void lds_dma16(const void* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

template <int P, int CS, int W, int DEPTH, bool kStream>
__global__ __launch_bounds__(64 * W) void sign_fp6_kernel(SignTable tab, int rec, int ncv, int B,
                                                          int red_off, int y_bf16) {
  extern __shared__ __align__(16) uint8_t smem[];
  // this workgroup's layer (a wave-uniform choice among at most kMultiMax)
  int li = 0;
#pragma unroll
  for (int i = 1; i < kMultiMax; ++i)
    if (i < tab.n && (int)blockIdx.x >= tab.l[i].group_begin) li = i;
  const SignLayer& ly = tab.l[li];
  const uint8_t* __restrict__ packed = ly.packed;
  const uint8_t* __restrict__ aop = ly.aop;
  const float* __restrict__ row_scale = ly.row_scale;
  const int64_t panel_bytes = ly.panel_bytes;
  const int panels = ly.panels, full_tiles = ly.full_tiles, tail_bytes = ly.tail_bytes;
  const int N = ly.N;
  const int ext_tiles = full_tiles + (tail_bytes > 0 ? 1 : 0);
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int g = lane >> 4, r = lane & 15;
  const int pbase = ((int)blockIdx.x - ly.group_begin) * P;
  const bool has_tail = tail_bytes > 0;
  const int nfull = full_tiles;
  // this wavefront's full tiles: t0 + wave + j W, j < nk
  const int nk = wave < nfull ? (nfull - wave + W - 1) / W : 0;

  // LDS: row scales (1 KB), the row's records (red_off - 1024 bytes, a
  // whole number of KB; streamed: 1 KB per wavefront), the tail tile's slots
  // (P KB); the final reduction reuses everything after the row scales.
  float* rs_lds = reinterpret_cast<float*>(smem);
  uint8_t* rec_lds = smem + 1024;
  uint8_t* tslot_lds = smem + red_off;
  uint8_t* wrec = rec_lds + 1024 * wave;           // streamed: this wavefront's record

  // This lane's MFMA column in each column set; unused columns read the
  // set's last column (their products are never read).
  int boff[CS], soff[CS], u_str[CS];
#pragma unroll
  for (int cs = 0; cs < CS; ++cs) {
    const int ncs = max(1, min(16, ncv - 16 * cs));
    const int col = min(r, ncs - 1);
    boff[cs] = aop_data_offset(cs, 0, g, col, ncs);
    soff[cs] = aop_scale_offset(ncv, cs, g, col, ncs);
    u_str[cs] = aop_u_stride(ncs);
  }
  const int tpoff = aop_tpart_offset(ncv) + 4 * min(lane, B - 1);

  const uint8_t* prow[P];
#pragma unroll
  for (int p = 0; p < P; ++p) prow[p] = packed + (int64_t)min(pbase + p, panels - 1) * panel_bytes;

  const int tail_wave = nfull % W;                 // takes the tail tile first
  const int tb = kPanelRows * tail_bytes;           // tail bytes of a panel: a multiple of 16, <= 1008
  const int tail_o = min(16 * lane, max(tb, 16) - 16);
  v4u rsv = {0u, 0u, 0u, 0u};                       // streamed: row scales (wavefront 0)
  v4u tr_rec = {0u, 0u, 0u, 0u}, tr_raw[P];         // streamed: the tail tile's record and bytes
  if (!kStream) {
    // ---- 1. the activation records, the row scales and the tail tile's
    // packed bytes into LDS, requested before any weight (a compute unit
    // returns vector-memory requests about in order, so they land first)
    const uint8_t* src = aop + 16 * lane;
    const int bytes = ext_tiles * rec;
    for (int off = wave * 1024; off < bytes; off += W * 1024) lds_dma16(src + off, rec_lds + off);
    if (wave == 0) {
      const int n4 = min(pbase * kPanelRows + 4 * lane, N - 4);   // rows past N: never used
      lds_dma16(row_scale + n4, reinterpret_cast<uint8_t*>(rs_lds));
    }
    if (has_tail && wave == W - 1) {
#pragma unroll
      for (int p = 0; p < P; ++p)
        lds_dma16(prow[p] + (int64_t)full_tiles * kTileBytes + tail_o, tslot_lds + 1024 * p);
    }
  } else {
    // ---- 1'. requested ahead of the weights, into registers: the row
    // scales (used after the loop) and the tail tile's record and bytes
    if (wave == 0) {
      const int n4 = min(pbase * kPanelRows + 4 * lane, N - 4);
      rsv = *reinterpret_cast<const v4u*>(row_scale + n4);
    }
    if (has_tail && wave == tail_wave) {
      tr_rec = *reinterpret_cast<const v4u*>(aop + (int64_t)nfull * rec + 16 * lane);
#pragma unroll
      for (int p = 0; p < P; ++p)
        tr_raw[p] = *reinterpret_cast<const v4u*>(prow[p] + (int64_t)full_tiles * kTileBytes + tail_o);
    }
  }

  // ---- 2. packed slots, DEPTH tiles ahead (streamed: with the tile's
  // record). Loads are issued on every path (past the wavefront's last tile
  // every lane reads the panel's first 16 bytes and the first record,
  // unused), so that the count of loads issued after any given one is fixed
  // and the waits are exact.
  uint4 A[DEPTH][P];
  v4u R[DEPTH];
  auto issue = [&](int j, uint4 (&S)[P], v4u& Rj) {
    const int tile = j < nk ? wave + j * W : 0;
    const int off = j < nk ? tile * kTileBytes + 16 * lane : 0;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      // each weight byte is read once per call: non-temporal
      const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(prow[p] + off));
      S[p] = make_uint4(v.x, v.y, v.z, v.w);
    }
    // (a record of <= 1 KB: the 1 KB read from its start stays within the
    // operand's slack)
    if (kStream) Rj = *reinterpret_cast<const v4u*>(aop + (int64_t)tile * rec + 16 * lane);
  };
  // the copies above stay ahead of these requests
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) issue(d, A[d], R[d]);
  if (!kStream) {
    // The copies have landed once no more than the DEPTH tiles' P loads
    // each are outstanding; those stay in flight across the barrier.
    constexpr int n = DEPTH * P;
    static_assert(n <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8) | (n & 15) | ((n >> 4) << 14));
    wg_barrier();
  }

  f32x4 acc[P][CS];
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) acc[p][cs] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  float tacc = 0.0f;
  // The MFMAs of one tile whose activation record starts at `recp` (LDS).
  auto tile_mfma = [&](const uint8_t* recp, const uint4 (&S)[P]) {
    i32x8 bop[CS][4];
    uint32_t sc[CS];
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) {
      sc[cs] = *reinterpret_cast<const uint32_t*>(recp + soff[cs]);
#pragma unroll
      for (int u = 0; u < 4; ++u) bop[cs][u] = lds_b_operand(recp + boff[cs] + u * u_str[cs]);
    }
    tacc += *reinterpret_cast<const float*>(recp + tpoff);
    // Word u of every panel before word u + 1: consecutive MFMAs go to
    // different accumulators, so none waits for the one before it.
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int cs = 0; cs < CS; ++cs) acc[p][cs] = mfma_fp4_fp6<0>(S[p].x, bop[cs][0], sc[cs], acc[p][cs]);
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int cs = 0; cs < CS; ++cs) acc[p][cs] = mfma_fp4_fp6<1>(S[p].y, bop[cs][1], sc[cs], acc[p][cs]);
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int cs = 0; cs < CS; ++cs) acc[p][cs] = mfma_fp4_fp6<2>(S[p].z, bop[cs][2], sc[cs], acc[p][cs]);
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int cs = 0; cs < CS; ++cs) acc[p][cs] = mfma_fp4_fp6<3>(S[p].w, bop[cs][3], sc[cs], acc[p][cs]);
  };


  // ---- 3. the tail tile first (its slots from the row-major tail bytes),
  // by the wavefront whose turn it would be, then the full tiles
  if (has_tail && wave == tail_wave) {
    if (kStream) {
      // the wavefront's own LDS: its later reads follow these writes
      *reinterpret_cast<v4u*>(wrec + 16 * lane) = tr_rec;
#pragma unroll
      for (int p = 0; p < P; ++p) *reinterpret_cast<v4u*>(tslot_lds + 1024 * p + 16 * lane) = tr_raw[p];
    }
    uint4 TS[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      // slot (g, r): bytes 16u + 4g .. + 3 of row r, zero past the row's tail
      const uint8_t* row = tslot_lds + 1024 * p + r * tail_bytes;
      uint32_t w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint32_t v = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int t = 16 * u + 4 * g + k;
          const uint32_t byte = row[min(t, tail_bytes - 1)];      // unconditional read
          v |= (byte & (t < tail_bytes ? 0xFFu : 0u)) << (8 * k);
        }
        w[u] = v;
      }
      TS[p] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    tile_mfma(kStream ? wrec : rec_lds + nfull * rec, TS);
  }
  // While a later block of tiles follows, each tile's slots are replaced by
  // those DEPTH tiles on; the last block requests nothing, so that no load
  // is issued after the wavefront's last MFMAs (a request there would be
  // waited for, a whole memory round trip, before the epilogue).
  auto block = [&](int j0) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int j = j0 + d;
      if (kStream) *reinterpret_cast<v4u*>(wrec + 16 * lane) = R[d];
      tile_mfma(kStream ? wrec : rec_lds + (wave + j * W) * rec, A[d]);
      // the tile's MFMAs read A[d] before the next request overwrites it,
      // and the request goes out before the next tile's work (the scheduler
      // would otherwise hold it back to spare registers)
      __builtin_amdgcn_sched_barrier(0);
      issue(j + DEPTH, A[d], R[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  int j0 = 0;
  if (DEPTH < nk) {
    // The first block apart from the loop: the compiler cannot tell that the
    // LDS copies have landed, and waits for every load once, here, before
    // the first record read; the loop, entered only after it, keeps exact
    // waits.
    block(0);
    for (j0 = DEPTH; j0 + DEPTH < nk; j0 += DEPTH) block(j0);
  }
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    const int j = j0 + d;
    if (j < nk) {
      if (kStream) *reinterpret_cast<v4u*>(wrec + 16 * lane) = R[d];
      tile_mfma(kStream ? wrec : rec_lds + (wave + j * W) * rec, A[d]);
    }
    // one tile's operands live at a time, as in the loop
    __builtin_amdgcn_sched_barrier(0);
  }
  if (kStream && wave == 0) *reinterpret_cast<v4u*>(smem + 16 * lane) = rsv;   // rs_lds
  __builtin_amdgcn_s_waitcnt(0);                     // loads of tiles past the last, unused
  wg_barrier();                                      // records are no longer read

  // ---- 4. add the wavefronts' accumulators in a fixed order. Compact
  // layout: only the columns that hold a (batch row, term).
  const int NC = min(16, ncv);
  f32x4* red = reinterpret_cast<f32x4*>(smem + 1024);               // [W][P][CS][4][NC]
  float* tred = reinterpret_cast<float*>(smem + 1024 + W * P * CS * 4 * NC * 16);   // [W][16]
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int cs = 0; cs < CS; ++cs)
      if (r < min(16, ncv - 16 * cs)) red[(((wave * P + p) * CS + cs) * 4 + g) * NC + r] = acc[p][cs];
  if (lane < 16) tred[wave * 16 + lane] = tacc;
  wg_barrier();

  // One output (panel p, row, batch row b) per thread and pass, the terms'
  // columns read unconditionally (a term index past nt repeats the last,
  // weighted 0), summed in a fixed order: wavefronts, then terms.
  const int nt = ncv / B;                           // terms per batch row, 2..4
  void* __restrict__ y = ly.y;
  const int items = P * B * 16;
  for (int item = threadIdx.x; item < items; item += 64 * W) {
    const int row = item & 15;
    const int pb = item >> 4;
    const int p = pb / B, b = pb - (pb / B) * B;
    const int gi = row >> 2, ri = row & 3;
    float v[W][4], tv[W];
#pragma unroll
    for (int w = 0; w < W; ++w) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int cc = b * nt + min(t, nt - 1);
        v[w][t] = red[(((w * P + p) * CS + (cc >> 4)) * 4 + gi) * NC + (cc & 15)][ri];
      }
      tv[w] = tred[w * 16 + b];
    }
    float acc_s = 0.0f, tp = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float keep = t < nt ? 1.0f : 0.0f;
#pragma unroll
      for (int w = 0; w < W; ++w) acc_s = fmaf(v[w][t], keep, acc_s);
    }
#pragma unroll
    for (int w = 0; w < W; ++w) tp += tv[w];
    const float out = rs_lds[p * kPanelRows + row] * (acc_s + tp);
    const int n = (pbase + p) * kPanelRows + row;
    if (pbase + p < panels) {
      if (y_bf16)
        reinterpret_cast<uint16_t*>(y)[(int64_t)b * N + n] = (uint16_t)f32_to_bf16_bits(out);
      else
        reinterpret_cast<float*>(y)[(int64_t)b * N + n] = out;
    }
  }
}

constexpr int kRecLdsMax = 128 * 1024;             // LDS for the records of a row

// Wavefronts per workgroup, and the slot tiles each keeps requested (P
// 16-byte loads per tile). Eight wavefronts (two per SIMD, 256 registers
// each) while the slot, accumulator and operand registers fit 256: up to 11
// panels of one 16-column set, 7 of two; four (one per SIMD, 512) beyond.
constexpr int waves_for(int p, int cs, bool) { return (cs == 1 ? p >= 12 : p >= 8) ? 4 : 8; }
// Two tiles of slots in flight per wavefront at every width: on the 70B
// batch-1 step (one box, interleaved runs) 65.3 µs per step against 67.1
// with three and 67.7 with two to four chosen by width.
constexpr int depth_for(int) { return 2; }

template <int P, int CS, bool kStream>
hipError_t launch_fp6_t(const SignTable& tab, int groups, const OperandShape& s, int64_t B,
                        bool y_bf16, const Fp6Plan& plan, hipStream_t stream) {
  constexpr int W = waves_for(P, CS, kStream), DEPTH = depth_for(P);
  if (plan.w != W) return hipErrorInvalidValue;
  if (kStream && s.rec > 1024) return hipErrorInvalidValue;
  const dim3 grid((unsigned)groups);
  const dim3 block(64 * W);
  if (plan.lds_bytes > 160 * 1024) return hipErrorInvalidValue;   // a compute unit's LDS
  // Dynamic LDS beyond the default 64 KB limit has to be allowed per kernel.
  static size_t allowed = 0;
  if (plan.lds_bytes > allowed) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&sign_fp6_kernel<P, CS, W, DEPTH, kStream>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)plan.lds_bytes);
    if (e != hipSuccess) return e;
    allowed = plan.lds_bytes;
  }
  return launch_timed(sign_fp6_kernel<P, CS, W, DEPTH, kStream>, grid, block, plan.lds_bytes, stream, tab,
                      s.rec, s.ncv, (int)B, plan.red_off, y_bf16 ? 1 : 0);
}

// Panels per workgroup instantiated for each count of 16-column sets
// (registers: P x CS accumulator quads, DEPTH x P slot quads).
constexpr int kPanelsCS1[] = {1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 14, 16};
constexpr int kPanelsCS2[] = {1, 2, 3, 4, 6, 8, 12};
constexpr int kPanelsCS3[] = {1, 2, 3, 4};

}  // namespace

// LDS and workgroups of a plan of P panels per workgroup for one layer.
constexpr int kStreamRecordsAbove = 64 * 1024;     // records streamed beyond this copy

// Whether a layer's records are streamed (decided once for a group of layers
// sharing one launch, on its longest rows).
static bool stream_records(const PackedGeom& g, const OperandShape& s) {
  return s.rec <= 1024 && (int64_t)g.ext_tiles * s.rec > kStreamRecordsAbove;
}

// LDS, wavefronts and workgroups of a plan of P panels per workgroup (and
// the record mode pl->stream) for one layer.
static void fill_resident(Fp6Plan* pl, const PackedGeom& g, const OperandShape& s) {
  pl->w = waves_for(pl->p, s.cs, pl->stream);
  const int recs = pl->stream ? 1024 * pl->w : ((g.ext_tiles * s.rec + 1023) / 1024) * 1024;
  const int nc = std::min(16, s.ncv);
  const size_t red = (size_t)pl->w * pl->p * s.cs * 4 * nc * 16 + (size_t)pl->w * 16 * 4;
  pl->red_off = 1024 + recs;
  pl->lds_bytes = std::max((size_t)pl->red_off + (size_t)1024 * pl->p, 1024 + red);
  pl->pgroups = (int)((g.panels + pl->p - 1) / pl->p);
  pl->groups = pl->pgroups;
}

bool fp6_records_fit(const PackedGeom& g, const OperandShape& s) {
  return (int64_t)g.ext_tiles * s.rec <= kRecLdsMax;
}

Fp6Plan plan_fp6(int64_t B, const PackedGeom& g, const OperandShape& s, int device_cus,
                 int panels_per_group) {
  (void)B;
  if (!fp6_records_fit(g, s) && !stream_records(g, s))
    return plan_fp6_chunked(g, s, device_cus, panels_per_group);
  const int64_t cus = device_cus > 0 ? device_cus : 256;
  const int* cand = s.cs == 1 ? kPanelsCS1 : (s.cs == 2 ? kPanelsCS2 : kPanelsCS3);
  const int ncand = s.cs == 1 ? 12 : (s.cs == 2 ? 7 : 4);
  // The panels per workgroup that minimise the kilobytes the busiest
  // compute unit streams (workgroups beyond one per unit queue behind it):
  // its packed weights from memory, plus its activation records from the L2
  // cache weighted 1/4 (a compute unit's share of L2 bandwidth is several
  // times its share of HBM's); then the most panels (each operand read from
  // LDS feeds them all).
  Fp6Plan best{};
  int64_t best_load = -1;
  for (int ci = 0; ci < ncand; ++ci) {
    const int P = cand[ci];
    if (panels_per_group > 0 && P != panels_per_group) continue;
    const int64_t wgs = (g.panels + P - 1) / P;
    const int64_t load = ((wgs + cus - 1) / cus) * g.ext_tiles * (4 * P + s.rec / 1024) / 4;
    if (best_load < 0 || load < best_load || (load == best_load && P > best.p)) {
      best_load = load;
      best.p = P;
    }
  }
  if (best_load < 0) best.p = 1;
  best.stream = stream_records(g, s);
  fill_resident(&best, g, s);
  return best;
}

Fp6Plan plan_fp6_group(int64_t B, const PackedGeom* gs, int n, const OperandShape& s,
                       int device_cus) {
  // The layers' panels as one matrix of the longest rows: one kernel and one
  // count of panels per workgroup for all of them.
  PackedGeom all = gs[0];
  int64_t panels = 0;
  for (int i = 0; i < n; ++i) {
    panels += gs[i].panels;
    if (gs[i].ext_tiles > all.ext_tiles) all = gs[i];
  }
  all.panels = panels;
  return plan_fp6(B, all, s, device_cus);
}

Fp6Plan plan_fp6_layer(const Fp6Plan& group, const PackedGeom& g, const OperandShape& s) {
  Fp6Plan pl = group;
  if (pl.chunked) fill_chunks(&pl, g, s);
  else fill_resident(&pl, g, s);
  return pl;
}

namespace {

SignLayer sign_layer(const uint8_t* packed, const PackedGeom& g, const uint8_t* aop,
                     const float* row_scale, void* y, const Fp6Plan& plan, int group_begin) {
  SignLayer l;
  l.packed = packed;
  l.aop = aop;
  l.row_scale = row_scale;
  l.y = y;
  l.panel_bytes = g.panel_bytes;
  l.panels = (int)g.panels;
  l.full_tiles = (int)g.full_tiles;
  l.tail_bytes = (int)g.tail_bytes;
  l.N = (int)g.N;
  l.nch = plan.chunked ? plan.nch : 0;
  l.group_begin = group_begin;
  return l;
}

hipError_t launch_fp6_table(const SignTable& tab, int groups, const OperandShape& s, int64_t B,
                            bool y_bf16, const Fp6Plan& plan, hipStream_t stream) {
  if (plan.chunked) return launch_fp6_chunked_table(tab, groups, s, B, y_bf16, plan, stream);
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
#define LQ_FP6_CASE(P_, CS_)                                                            \
  if (plan.p == P_ && s.cs == CS_) return launch_fp6_t<P_, CS_, false>(tab, groups, s, B, y_bf16, plan, stream);
#define LQ_FP6_CASE_S(P_)                                                                \
  if (plan.p == P_ && s.cs == 1)                                                         \
    return plan.stream ? launch_fp6_t<P_, 1, true>(tab, groups, s, B, y_bf16, plan, stream) \
                       : launch_fp6_t<P_, 1, false>(tab, groups, s, B, y_bf16, plan, stream);
  LQ_FP6_CASE_S(1) LQ_FP6_CASE_S(2) LQ_FP6_CASE_S(3) LQ_FP6_CASE_S(4) LQ_FP6_CASE_S(5)
  LQ_FP6_CASE_S(6) LQ_FP6_CASE_S(7) LQ_FP6_CASE_S(8) LQ_FP6_CASE_S(10) LQ_FP6_CASE_S(12)
  LQ_FP6_CASE_S(14) LQ_FP6_CASE_S(16)
  LQ_FP6_CASE(1, 2) LQ_FP6_CASE(2, 2) LQ_FP6_CASE(3, 2) LQ_FP6_CASE(4, 2) LQ_FP6_CASE(6, 2)
  LQ_FP6_CASE(8, 2) LQ_FP6_CASE(12, 2)
  LQ_FP6_CASE(1, 3) LQ_FP6_CASE(2, 3) LQ_FP6_CASE(3, 3) LQ_FP6_CASE(4, 3)
#undef LQ_FP6_CASE
#undef LQ_FP6_CASE_S
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_sign_fp6(const uint8_t* packed, const PackedGeom& g, const OperandPlan& op,
                           int64_t B, const float* row_scale, void* y, bool y_bf16,
                           const Fp6Plan& plan, hipStream_t stream) {
  SignTable tab;
  tab.n = 1;
  tab.l[0] = sign_layer(packed, g, op.aop, row_scale, y, plan, 0);
  for (int i = 1; i < kMultiMax; ++i) tab.l[i] = tab.l[0];
  return launch_fp6_table(tab, plan.groups, op.s, B, y_bf16, plan, stream);
}

bool fp6_plans_match(const Fp6Plan& a, const Fp6Plan& b) {
  return a.chunked == b.chunked && a.stream == b.stream && a.p == b.p && a.w == b.w &&
         (!a.chunked || (a.tpc == b.tpc && a.chunk_bytes == b.chunk_bytes));
}

hipError_t launch_sign_fp6_multi(int n, const SignLayerDesc* layers, const OperandShape& s,
                                 int64_t B, bool y_bf16, hipStream_t stream) {
  if (n < 1 || n > kMultiMax) return hipErrorInvalidValue;
  SignTable tab;
  tab.n = n;
  Fp6Plan plan = layers[0].plan;
  int groups = 0;
  for (int i = 0; i < n; ++i) {
    const SignLayerDesc& l = layers[i];
    if (!fp6_plans_match(l.plan, plan)) return hipErrorInvalidValue;
    plan.lds_bytes = std::max(plan.lds_bytes, l.plan.lds_bytes);
    plan.red_off = std::max(plan.red_off, l.plan.red_off);
    tab.l[i] = sign_layer(l.packed, l.g, l.aop, l.row_scale, l.y, l.plan, groups);
    groups += l.plan.groups;
  }
  for (int i = n; i < kMultiMax; ++i) tab.l[i] = tab.l[n - 1];
  // every layer's records, tail slots and reduction must fit the LDS given
  if (!plan.chunked)
    plan.lds_bytes = std::max(plan.lds_bytes, (size_t)plan.red_off + (size_t)1024 * plan.p);
  return launch_fp6_table(tab, groups, s, B, y_bf16, plan, stream);
}

}  // namespace lq
