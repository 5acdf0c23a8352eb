// Fused single-launch decode of one quantized layer for small batches:
// whitening, lift, FP6 activation operand and the FP4 x FP6 sign product in
// one kernel ([paper] §3 introduction: T and the lift fold into the one
// operator that multiplies the packed signs).
//
// Every workgroup is a product workgroup (P panels over the whole reduction
// length, as in sign_fp6.hip: 7 compute wavefronts and a loader). The first
// E = tiles x B of them (in start order) are also producers: before their
// product work they compute the activation record of one (tile, batch row)
// and publish it. The loader wavefront of every workgroup waits until all
// records are published before it copies the first chunk into LDS; the
// compute wavefronts request the packed slots of their first two chunks at
// kernel entry, so the weight stream overlaps the preparation.
//
// Ordering and progress. Roles follow a ticket taken at workgroup start
// (an agent-scope atomic counter), so the E producers are the first E
// workgroups to start; a producer publishes before it waits for anything,
// and the host only picks this kernel when E is at most the number of
// compute units (one workgroup fits on every compute unit), so all producers
// can be resident together and every wait ends. A record is published with
// device-scope stores, a release fence and a per-(tile, batch row) flag set to
// this launch's epoch; consumers poll the flags with device-scope loads and
// issue an acquire fence before reading records, so no stale cached line of
// a record is read. The polls are bounded: after about a second a consumer
// gives up and sets an error word instead of hanging. The epoch is read from
// the control words at entry; the last workgroup to finish resets the ticket
// and finish counters and advances the epoch. The control words and flags
// must be zero before the first launch that uses them.
#include <algorithm>
#include <atomic>

#include "lq_fp6_mma.h"
#include "lq_prep.h"

namespace lq {
namespace {

constexpr int kW = 7;                  // compute wavefronts (plus one loader)
constexpr int kFusedThreads = 64 * (kW + 1);
static_assert(kFusedThreads == kTileCols, "the lift gives one column to every thread");
constexpr unsigned kMaxPolls = 1u << 20;

// Control words (separate 128-byte lines), then flags [tiles][16].
constexpr int kCtlEpoch = 0, kCtlTicket = 32, kCtlDone = 64, kCtlError = kFusedErrorWord;
constexpr int kCtlWords = kFusedCtlWords;

__device__ __forceinline__ void store_coherent_u32(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned load_coherent_u32(const unsigned* p) {
  return __hip_atomic_load(const_cast<unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LDS of the preparation (producers). It overlays the chunk buffers: every
// workgroup copies its first chunk only after all records are published,
// and a producer publishes (reading its record from here) before that.
struct PrepLds {
  float xs[kSpanMax];        // x * c, then its Hadamard transform
  float zt[kTileCols];       // the tile's lifted values
  float Ms[64 * 64];         // M / sqrt(hb)
};

template <int P, int TPC, int kXKind>
__global__ __launch_bounds__(kFusedThreads) void decode_fused_kernel(
    const uint8_t* __restrict__ packed, int panels, int64_t panel_bytes, int full_tiles,
    int tail_bytes, const void* __restrict__ x, int B, int K, int d, int D, int lhb, float norm,
    const float* __restrict__ c, const float* __restrict__ M, int L, uint8_t* aop, int rec,
    int ncv, unsigned* ctl, int nch, int chunk_bytes, int producers,
    const float* __restrict__ row_scale, void* __restrict__ y, int y_bf16, int N,
    unsigned max_polls, unsigned wait_skew) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int W = kW;
  constexpr int CT = W * TPC;
  unsigned* flags = ctl + kCtlWords;
  const int tid = threadIdx.x;
  const int wave = wave_id(), lane = tid & 63;
  const int g = lane >> 4, r = lane & 15;
  const bool loader = wave == W;
  const int nt = ncv / B;
  const int ext_tiles = full_tiles + (tail_bytes > 0 ? 1 : 0);

  // ---- ticket and epoch (nothing is in flight yet)
  __shared__ unsigned s_role, s_epoch;
  if (tid == 0) {
    s_role = __hip_atomic_fetch_add(ctl + kCtlTicket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) %
             gridDim.x;
    s_epoch = load_coherent_u32(ctl + kCtlEpoch) + 1u;
  }
  __syncthreads();
  const int role = (int)s_role;
  const unsigned epoch = s_epoch;
  const bool producer = role < producers;
  const int pq = role / B, pb = role % B;           // the producer's (tile, batch row)
  const int pbase = role * P;

  // LDS: row scales, chunk buffers (first holding the preparation area), the
  // tail tile.
  float* rs_lds = reinterpret_cast<float*>(smem);
  uint8_t* buf0 = smem + 1024;
  uint8_t* buf1 = buf0 + chunk_bytes;
  uint8_t* trec_lds = buf1 + chunk_bytes;
  uint8_t* tslot_lds = trec_lds + ((rec + 1023) / 1024) * 1024;
  PrepLds& pl = *reinterpret_cast<PrepLds*>(buf0);
  uint8_t* prec = reinterpret_cast<uint8_t*>(&pl + 1);       // the producer's record

  const int ncs = max(1, min(16, ncv));
  const int col = min(r, ncs - 1);
  const int boff = aop_data_offset(0, 0, g, col, ncs);
  const int soff = aop_scale_offset(ncv, 0, g, col, ncs);
  const int u_str = aop_u_stride(ncs);
  const int tpoff = aop_tpart_offset(ncv) + 4 * min(lane, B - 1);

  const uint8_t* prow[P];
#pragma unroll
  for (int p = 0; p < P; ++p) prow[p] = packed + (int64_t)min(pbase + p, panels - 1) * panel_bytes;

  f32x4 acc[P];
#pragma unroll
  for (int p = 0; p < P; ++p) acc[p] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  float tacc = 0.0f;

  uint4 A0[TPC][P], A1[TPC][P];
  const int last_full = max(full_tiles - 1, 0);
  auto issue_A = [&](int cc, uint4 (&A)[TPC][P]) {
    const bool live = cc < nch;
#pragma unroll
    for (int q = 0; q < TPC; ++q) {
      const int t = min(cc * CT + wave * TPC + q, last_full);
      const int off = live ? t * kTileBytes + 16 * lane : 0;
#pragma unroll
      for (int p = 0; p < P; ++p) A[q][p] = *reinterpret_cast<const uint4*>(prow[p] + off);
    }
  };
  auto tile_mfma = [&](const uint8_t* recp, const uint4 (&S)[P]) {
    i32x8 bop[4];
    const uint32_t sc = *reinterpret_cast<const uint32_t*>(recp + soff);
#pragma unroll
    for (int u = 0; u < 4; ++u) bop[u] = lds_b_operand(recp + boff + u * u_str);
    tacc += *reinterpret_cast<const float*>(recp + tpoff);
#pragma unroll
    for (int p = 0; p < P; ++p) {
      acc[p] = mfma_fp4_fp6<0>(S[p].x, bop[0], sc, acc[p]);
      acc[p] = mfma_fp4_fp6<1>(S[p].y, bop[1], sc, acc[p]);
      acc[p] = mfma_fp4_fp6<2>(S[p].z, bop[2], sc, acc[p]);
      acc[p] = mfma_fp4_fp6<3>(S[p].w, bop[3], sc, acc[p]);
    }
  };
  // Copy `bytes` (a multiple of 16) from global to LDS, 1 KB per
  // instruction, without reading past the end (the last lanes repeat the
  // final 16 bytes).
  auto dma = [&](const uint8_t* src, uint8_t* dst, int bytes) {
    for (int off = 0; off < bytes; off += 1024)
      __builtin_amdgcn_global_load_lds((const void*)(src + min(off + 16 * lane, bytes - 16)),
                                       (__attribute__((address_space(3))) void*)(dst + off), 16, 0, 0);
  };
  // Loader: wait until every (tile, batch row) of tiles [t0, t1) is
  // published in this launch's epoch. Bounded: on time-out the error word is
  // set and the product goes on with whatever the records hold.
  auto wait_tiles = [&](int t0, int t1) {
    const int n = (t1 - t0) * B;
    for (unsigned it = 0;; ++it) {
      bool ok = true;
      for (int i = lane; i < n; i += 64) {
        const int t = t0 + i / B, b = i % B;
        ok = ok && (load_coherent_u32(flags + t * 16 + b) == epoch + wait_skew);
      }
      if (__all(ok)) break;
      if (it >= max_polls) {
        if (lane == 0) store_coherent_u32(ctl + kCtlError, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
  };

  // ---- preparation phases of a producer: the lift (one column per thread
  // of all 8 wavefronts, written in the FP6 conversion's slot order with the
  // plane factors applied) and the FP6 blocks (lane h < 16 of wavefront 0
  // converts block h of the tile into this producer's record columns).
  auto lift_phase = [&](const TileSpan& ts) {
    const int jj = tid;                               // kTileCols threads
    const float z = jj < ts.width ? lift_column(pl.Ms, pl.xs, pq * kTileCols + jj, d, D, K, ts.h_lo)
                                  : 0.0f;
    float f;
    const int slot = fp6_slot(jj, f);
    pl.zt[slot] = f * z;
  };
  auto quant_phase = [&]() {
    if (tid >= 16) return;
    const int u = tid >> 2, gg = tid & 3;
    Fp6LaneTerms rt;
    float tp = fp6_lane_block(pl.zt, tid, nt, rt);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < nt) {
        const int cc = pb * nt + t;
        aop_store_block(prec + aop_data_offset(0, u, gg, cc, ncs), rt.dw[t]);
        prec[aop_scale_offset(ncv, 0, gg, cc, ncs) + u] = (uint8_t)(127 + rt.e[t]);
      }
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) tp += __shfl_xor(tp, o, 16);
    if (tid == 0) *reinterpret_cast<float*>(prec + aop_tpart_offset(ncv) + 4 * pb) = tp;
  };

  if (loader) {
    // ---- preparation inputs of a producer: x and c over the covering
    // Hadamard blocks, and M, into LDS
    // Every load is issued before the first is waited for (one memory round
    // trip, not one per element).
    if (producer) {
      const TileSpan ts = tile_span(pq, K, d, D, lhb, L);
      const int64_t xrow = (int64_t)pb * K;
      constexpr int kIt = kSpanMax / 64;
      float xv[kIt], cv[kIt];
#pragma unroll
      for (int it = 0; it < kIt; ++it) {
        const int i = lane + 64 * it;
        const int k = ts.h_lo + (i < ts.span ? i : 0);
        if (kXKind == 1) xv[it] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(x)[xrow + k]);
        else xv[it] = reinterpret_cast<const float*>(x)[xrow + k];
        cv[it] = c[k];
      }
      const int dD = d * D;
      constexpr int kMIt = 8;
      float mv[kMIt];
#pragma unroll
      for (int u = 0; u < kMIt; ++u) mv[u] = M[min(lane + 64 * u, dD - 1)];
#pragma unroll
      for (int it = 0; it < kIt; ++it) pl.xs[lane + 64 * it] = xv[it] * cv[it];
#pragma unroll
      for (int u = 0; u < kMIt; ++u)
        if (lane + 64 * u < dD) pl.Ms[lane + 64 * u] = mv[u] * norm;
      for (int base = 64 * kMIt; base < dD; base += 64 * kMIt) {     // d * D > 512
#pragma unroll
        for (int u = 0; u < kMIt; ++u) mv[u] = M[min(base + lane + 64 * u, dD - 1)];
#pragma unroll
        for (int u = 0; u < kMIt; ++u)
          if (base + lane + 64 * u < dD) pl.Ms[base + lane + 64 * u] = mv[u] * norm;
      }
    }
    wg_barrier();                                     // B1: inputs in LDS
    if (producer) {
      const TileSpan ts = tile_span(pq, K, d, D, lhb, L);
      wg_barrier();                                   // m1: transformed
      lift_phase(ts);
      wg_barrier();                                   // m2: lifted
    }
    wg_barrier();                                     // B2: record in LDS
    if (producer) {
      // Publish this producer's parts of the record: its nt columns' data
      // blocks, their scale dwords, its plane sum; then, after a release
      // fence, the flag.
      uint8_t* grec = aop + (int64_t)pq * rec;
      const int items = nt * 16 * 6 + nt * 4 + 1;
      for (int i = lane; i < items; i += 64) {
        int off;
        if (i < nt * 96) {
          const int t = i / 96, blk = (i % 96) / 6, k = i % 6;
          off = aop_data_offset(0, blk >> 2, blk & 3, pb * nt + t, ncs) + 4 * k;
        } else if (i < nt * 96 + nt * 4) {
          const int j = i - nt * 96, t = j >> 2, gg = j & 3;
          off = aop_scale_offset(ncv, 0, gg, pb * nt + t, ncs);
        } else {
          off = aop_tpart_offset(ncv) + 4 * pb;
        }
        store_coherent_u32(reinterpret_cast<unsigned*>(grec + off),
                           *reinterpret_cast<const uint32_t*>(prec + off));
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      if (lane == 0) store_coherent_u32(flags + pq * 16 + pb, epoch);
    }
    // ---- product: row scales; then, once every record is published (an
    // acquire fence after the flags so that no stale cached line of a
    // record is read), chunks 0 and 1 and the tail
    {
      const int n4 = min(pbase * kPanelRows + 4 * lane, N - 4);
      __builtin_amdgcn_global_load_lds((const void*)(row_scale + n4),
                                       (__attribute__((address_space(3))) void*)rs_lds, 16, 0, 0);
    }
    wait_tiles(0, ext_tiles);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const bool tail = tail_bytes > 0;
    for (int cc = 0; cc < min(nch, 2); ++cc) {
      const int t0 = cc * CT, t1 = min(full_tiles, t0 + CT);
      dma(aop + (int64_t)t0 * rec, cc == 0 ? buf0 : buf1, (t1 - t0) * rec);
    }
    if (tail) {
      dma(aop + (int64_t)full_tiles * rec, trec_lds, rec);
      const int tb = kPanelRows * tail_bytes;         // a multiple of 16, at most 1008
#pragma unroll
      for (int p = 0; p < P; ++p)
        dma(prow[p] + (int64_t)full_tiles * kTileBytes, tslot_lds + 1024 * p, tb);
    }
    __builtin_amdgcn_s_waitcnt(0);
    wg_barrier();                                     // Y0: chunks 0, 1 in LDS
    for (int c0 = 0; c0 < nch; c0 += 2) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {                   // step c0 + k
        __builtin_amdgcn_s_waitcnt(0);                // chunk c0 + k + 1 is in LDS
        wg_barrier();
        const int cn = c0 + k + 2;
        if (cn < nch) {
          const int t0 = cn * CT, t1 = min(full_tiles, t0 + CT);
          dma(aop + (int64_t)t0 * rec, k == 0 ? buf0 : buf1, (t1 - t0) * rec);
        }
        wg_barrier();
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    if (tail) {
      uint4 TS[P];
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const uint8_t* row = tslot_lds + 1024 * p + r * tail_bytes;
        uint32_t w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          uint32_t v = 0;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int t = 16 * u + 4 * g + k;
            const uint32_t byte = row[min(t, tail_bytes - 1)];
            v |= (byte & (t < tail_bytes ? 0xFFu : 0u)) << (8 * k);
          }
          w[u] = v;
        }
        TS[p] = make_uint4(w[0], w[1], w[2], w[3]);
      }
      tile_mfma(trec_lds, TS);
    }
  } else {
    // The packed slots of chunks 0 and 1 go out first.
    issue_A(0, A0);
    issue_A(1, A1);
    wg_barrier();                                     // B1
    if (producer) {
      // ---- preparation of (tile pq, batch row pb); the loader wavefront
      // joins the lift
      const TileSpan ts = tile_span(pq, K, d, D, lhb, L);
      if (1024 * wave < ts.span) wave_fwht_1024(pl.xs + 1024 * wave, lhb, lane);
      wg_barrier();                                   // m1
      lift_phase(ts);
      wg_barrier();                                   // m2
      quant_phase();
    }
    wg_barrier();                                     // B2
    wg_barrier();                                     // Y0
    auto step = [&](int cc, uint4 (&A)[TPC][P], uint8_t* cur) {
#pragma unroll
      for (int q = 0; q < TPC; ++q) {
        const int jt = wave * TPC + q;
        if (cc * CT + jt < full_tiles) tile_mfma(cur + jt * rec, A[q]);
      }
      wg_barrier();
      wg_barrier();
      issue_A(cc + 2, A);
    };
    for (int c0 = 0; c0 < nch; c0 += 2) {
      step(c0, A0, buf0);
      step(c0 + 1, A1, buf1);
    }
  }
  wg_barrier();

  // ---- add the wavefronts' accumulators in a fixed order and write y.
  f32x4* red = reinterpret_cast<f32x4*>(buf0);                       // [W+1][P][64]
  float* tred = reinterpret_cast<float*>(buf0 + (W + 1) * P * 64 * 16);   // [W+1][16]
#pragma unroll
  for (int p = 0; p < P; ++p) red[(wave * P + p) * 64 + lane] = acc[p];
  if (lane < 16) tred[wave * 16 + lane] = tacc;
  wg_barrier();
  const int items = P * B * 16;
  for (int item = tid; item < items; item += kFusedThreads) {
    const int row = item & 15;
    const int b = (item >> 4) % B;
    const int p = (item >> 4) / B;
    float v[W + 1][4], tv[W + 1];
#pragma unroll
    for (int w = 0; w <= W; ++w) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int cc = b * nt + min(t, nt - 1);
        const int l = 16 * (row >> 2) + (cc & 15);
        v[w][t] = red[(w * P + p) * 64 + l][row & 3];
      }
      tv[w] = tred[w * 16 + b];
    }
    const float rs = rs_lds[p * kPanelRows + row];
    float acc_s = 0.0f, tp = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < nt) {
#pragma unroll
        for (int w = 0; w <= W; ++w) acc_s += v[w][t];
      }
    }
#pragma unroll
    for (int w = 0; w <= W; ++w) tp += tv[w];
    const float out = rs * (acc_s + tp);
    const int n = (pbase + p) * kPanelRows + row;
    if (pbase + p < panels) {
      if (y_bf16)
        reinterpret_cast<uint16_t*>(y)[(int64_t)b * N + n] = (uint16_t)f32_to_bf16_bits(out);
      else
        reinterpret_cast<float*>(y)[(int64_t)b * N + n] = out;
    }
  }

  // ---- the last workgroup to finish resets the counters for the next launch
  __syncthreads();
  if (tid == 0) {
    const unsigned done =
        __hip_atomic_fetch_add(ctl + kCtlDone, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == gridDim.x - 1) {
      store_coherent_u32(ctl + kCtlDone, 0u);
      store_coherent_u32(ctl + kCtlTicket, 0u);
      store_coherent_u32(ctl + kCtlEpoch, epoch);
    }
  }
}

// The test aid: an epoch offset no producer writes (epochs count launches
// from zero) and a short bound on the polls.
std::atomic<bool> g_forced_timeout{false};
constexpr unsigned kForcedPolls = 4;
constexpr unsigned kForcedSkew = 0x40000000u;

template <int P, int TPC, int kXKind>
hipError_t launch_fused_t(const uint8_t* packed, const PackedGeom& g, const void* x, int64_t B,
                          int64_t K, int d, int D, int hb, const float* c, const float* M,
                          const OperandPlan& op, unsigned* ctl, const float* row_scale, void* y,
                          bool y_bf16, const FusedPlan& plan, hipStream_t stream) {
  int lhb = 0;
  while ((1 << lhb) < hb) ++lhb;
  const float norm = (lhb % 2 == 0) ? ldexpf(1.0f, -lhb / 2) : (float)(1.0 / sqrt((double)hb));
  if (plan.lds_bytes > 160 * 1024) return hipErrorInvalidValue;
  const bool forced = g_forced_timeout.load(std::memory_order_relaxed);
  static size_t allowed = 0;
  if (plan.lds_bytes > allowed) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&decode_fused_kernel<P, TPC, kXKind>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)plan.lds_bytes);
    if (e != hipSuccess) return e;
    allowed = plan.lds_bytes;
  }
  return launch_timed(decode_fused_kernel<P, TPC, kXKind>, dim3((unsigned)plan.groups),
                      dim3(kFusedThreads), plan.lds_bytes, stream, packed, (int)g.panels,
                      g.panel_bytes, g.full_tiles, g.tail_bytes, x, (int)B, (int)K, d, D, lhb, norm,
                      c, M, (int)g.L, op.aop, op.s.rec, op.s.ncv, ctl, plan.nch, plan.chunk_bytes,
                      plan.producers, row_scale, y, y_bf16 ? 1 : 0, (int)g.N,
                      forced ? kForcedPolls : kMaxPolls, forced ? kForcedSkew : 0u);
}

}  // namespace

void set_fused_forced_timeout(bool on) { g_forced_timeout.store(on, std::memory_order_relaxed); }

FusedPlan plan_fused(int64_t B, const PackedGeom& g, const OperandShape& s, int cus) {
  FusedPlan p{};
  p.ok = false;
  if (s.cs != 1 || B > 16 || g.ext_tiles > kMaxFusedTiles) return p;
  p.p = 1;
  for (int cand : {8, 4, 2}) {
    if ((g.panels + cand - 1) / cand >= 200) { p.p = cand; break; }
  }
  p.groups = (int)((g.panels + p.p - 1) / p.p);
  p.producers = g.ext_tiles * (int)B;
  // Every producer is also a product workgroup, and all producers must be
  // able to run at once (one workgroup fits on every compute unit).
  if (p.producers > p.groups || p.producers > cus) return p;
  const size_t prep = sizeof(PrepLds) + (size_t)s.rec;
  auto lds_for = [&](int tpc) {
    const int ct = kW * tpc;
    const int chunk = ((ct * s.rec + 1023) / 1024) * 1024;
    const size_t tail = (size_t)((s.rec + 1023) / 1024) * 1024 + (size_t)1024 * p.p;
    const size_t red = (size_t)(kW + 1) * p.p * 64 * 16 + (size_t)(kW + 1) * 64;
    return std::make_pair(chunk, 1024 + std::max(std::max((size_t)2 * chunk + tail, prep), red));
  };
  p.tpc = (p.p <= 4 && lds_for(3).second <= 150 * 1024) ? 3 : 1;
  const auto l = lds_for(p.tpc);
  p.chunk_bytes = l.first;
  p.lds_bytes = l.second;
  if (p.lds_bytes > 160 * 1024 - 256) return p;    // (plus the kernel's static words)
  p.nch = (g.full_tiles + kW * p.tpc - 1) / (kW * p.tpc);
  p.ok = true;
  return p;
}

hipError_t launch_decode_fused(const uint8_t* packed, const PackedGeom& g, const void* x,
                               bool x_bf16, int64_t B, int64_t K, int d, int D, int hb,
                               const float* c, const float* M, const OperandPlan& op,
                               unsigned* ctl, const float* row_scale, void* y, bool y_bf16,
                               const FusedPlan& plan, hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
#define LQ_FUSED_CASE(P_, TPC_)                                                                  \
  if (plan.p == P_ && plan.tpc == TPC_)                                                          \
    return x_bf16 ? launch_fused_t<P_, TPC_, 1>(packed, g, x, B, K, d, D, hb, c, M, op, ctl,    \
                                                 row_scale, y, y_bf16, plan, stream)            \
                  : launch_fused_t<P_, TPC_, 0>(packed, g, x, B, K, d, D, hb, c, M, op, ctl,    \
                                                 row_scale, y, y_bf16, plan, stream);
  LQ_FUSED_CASE(1, 3) LQ_FUSED_CASE(2, 3) LQ_FUSED_CASE(4, 3)
  LQ_FUSED_CASE(1, 1) LQ_FUSED_CASE(2, 1) LQ_FUSED_CASE(4, 1) LQ_FUSED_CASE(8, 1)
#undef LQ_FUSED_CASE
  return hipErrorInvalidValue;
}

}  // namespace lq
