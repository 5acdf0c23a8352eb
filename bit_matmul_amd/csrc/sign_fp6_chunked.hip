// Small-batch sign product, chunked variant: the same FP4 x FP6 arithmetic
// and operand records as sign_fp6.hip (which documents them), for layers
// whose activation records do not fit LDS at once (longer rows, more batch
// rows). A workgroup owns P 16-row panels over the whole reduction length
// (no communication between workgroups). Its W compute wavefronts take the
// full tiles in chunks of W*TPC tiles, TPC consecutive tiles each, all P
// panels per tile, so one activation-operand read from LDS feeds P MFMAs.
// An extra loader wavefront copies each chunk's activation records into LDS
// with global_load_lds (double-buffered, one chunk ahead) and multiplies
// the partial tail tile. The compute wavefronts keep the packed slots of two
// chunks in flight; since a wavefront waits for its loads in issue order
// and it issues nothing else, every tile's MFMAs start as soon as that
// tile's 16-byte slots have arrived. The two roles run separate code with
// the same sequence of barriers, so the compute wavefronts' waits on their
// slot loads never include the loader's copies. The wavefronts'
// accumulators are added in LDS in a fixed order, the terms and plane sums
// combined, and y written: deterministic, no atomics.
#include <algorithm>
#include <type_traits>

#include "lq_fp6_mma.h"

namespace lq {
namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Loader wavefronts (kChunkLoaders): each copies every kLoaders-th kilobyte
// of a chunk, so that a chunk is requested by that many wavefronts at once.
// Measured on the 70B down projection at B = 16: one loader 42.8 us, two
// 40.8, four 34.5, eight 34.4 (and register spills where the compute
// wavefronts need many).
constexpr int kLoaders = kChunkLoaders;

template <int P, int CS, int W, int TPC>
__global__ __launch_bounds__(64 * (W + kLoaders)) void sign_fp6_chunked_kernel(SignTable tab, int rec, int ncv,
                                                                int B, int chunk_bytes, int y_bf16) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int CT = W * TPC;                       // full tiles per chunk
  // this workgroup's layer (a wave-uniform choice among at most kMultiMax)
  int li = 0;
#pragma unroll
  for (int i = 1; i < kMultiMax; ++i)
    if (i < tab.n && (int)blockIdx.x >= tab.l[i].group_begin) li = i;
  const SignLayer& ly = tab.l[li];
  const uint8_t* __restrict__ packed = ly.packed;
  const uint8_t* __restrict__ aop = ly.aop;
  const float* __restrict__ row_scale = ly.row_scale;
  void* __restrict__ y = ly.y;
  const int64_t panel_bytes = ly.panel_bytes;
  const int panels = ly.panels, full_tiles = ly.full_tiles, tail_bytes = ly.tail_bytes;
  const int nch = ly.nch, N = ly.N;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int g = lane >> 4, r = lane & 15;
  const bool loader = wave >= W;
  const int lw = wave - W;                          // loader index (when loader)
  const int pbase = ((int)blockIdx.x - ly.group_begin) * P;

  // This lane's MFMA column in each column set; unused columns read the
  // set's last column (their products are never read).
  int boff[CS], soff[CS];
#pragma unroll
  for (int cs = 0; cs < CS; ++cs) {
    const int ncs = max(1, min(16, ncv - 16 * cs));
    const int col = min(r, ncs - 1);
    boff[cs] = aop_data_offset(cs, 0, g, col, ncs);
    soff[cs] = aop_scale_offset(ncv, cs, g, col, ncs);
  }
  int u_str[CS];                                    // bytes between the u blocks of a set
#pragma unroll
  for (int cs = 0; cs < CS; ++cs) u_str[cs] = aop_u_stride(max(1, min(16, ncv - 16 * cs)));
  const int tpoff = aop_tpart_offset(ncv) + 4 * min(lane, B - 1);

  const uint8_t* prow[P];
#pragma unroll
  for (int p = 0; p < P; ++p) prow[p] = packed + (int64_t)min(pbase + p, panels - 1) * panel_bytes;

  f32x4 acc[P][CS];
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) acc[p][cs] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  float tacc = 0.0f;

  uint4 A0[TPC][P], A1[TPC][P];
  const int last_full = max(full_tiles - 1, 0);
  // Packed slots of chunk c. Past the last chunk every lane reads the same
  // 16 bytes instead (one cache line; the registers are not used): the loads
  // are issued on every path, so that no register ever merges two values (a
  // merge would make the compiler wait for the loads in flight).
  auto issue_A = [&](int c, uint4 (&A)[TPC][P]) {
    const bool live = c < nch;
#pragma unroll
    for (int q = 0; q < TPC; ++q) {
      const int t = min(c * CT + wave * TPC + q, last_full);
      const int off = live ? t * kTileBytes + 16 * lane : 0;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        // Each weight byte is read once per call: a non-temporal load keeps
        // the stream from displacing the activation records in the caches.
        const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(prow[p] + off));
        A[q][p] = make_uint4(v.x, v.y, v.z, v.w);
      }
    }
  };
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
    // word u of every panel before word u + 1 (independent accumulators)
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
  auto dma_chunk = [&](int c, uint8_t* dst) {
    const int t0 = c * CT;
    const int bytes = min(CT, full_tiles - t0) * rec;
    const uint8_t* src = aop + (int64_t)t0 * rec + 16 * lane;
    for (int off = lw * 1024; off < bytes; off += kLoaders * 1024)
      __builtin_amdgcn_global_load_lds((const void*)(src + off),
                                       (__attribute__((address_space(3))) void*)(dst + off), 16, 0, 0);
  };

  // LDS: row scales (1 KB), chunk buffers 0 and 1, the tail tile's record
  // and slots; the final reduction reuses everything after the row scales.
  float* rs_lds = reinterpret_cast<float*>(smem);
  uint8_t* buf0 = smem + 1024;
  uint8_t* buf1 = buf0 + chunk_bytes;

  // ---- Pipeline. A compute unit serves its vector-memory requests roughly
  // in order, so the activation records (L2 hits) must be requested before
  // the HBM traffic that would otherwise delay them: the loader requests
  // chunks 0 and 1, the tail tile and the row scales first; a barrier then
  // releases the compute wavefronts' requests for the packed slots of chunks
  // 0 and 1. After multiplying chunk c, the loader requests chunk c + 2 into
  // the freed buffer before a barrier that releases the slot requests of
  // chunk c + 2, so each compute wavefront keeps two chunks of slots
  // requested and each copy lands a chunk ahead of its use.
  // The two roles run separate code with the same sequence of barriers, so
  // the compute wavefronts' waits on their slot loads never include the
  // loader's copies (which the compiler would otherwise have to assume may
  // still be in flight). The tail tile (its record and the P panels'
  // row-major tail bytes) is multiplied by the loader while the compute
  // wavefronts work on the first chunk.
  const bool tail = tail_bytes > 0;
  uint8_t* trec_lds = buf1 + chunk_bytes;
  uint8_t* tslot_lds = trec_lds + ((rec + 1023) / 1024) * 1024;

  if (loader) {
    // Row scales of the workgroup's rows (16 bytes per lane, clamped to N),
    // by the first loader, as are the tail tile's copies and MFMAs.
    if (lw == 0) {
      const int n4 = min(pbase * kPanelRows + 4 * lane, N - 4);
      __builtin_amdgcn_global_load_lds((const void*)(row_scale + n4),
                                       (__attribute__((address_space(3))) void*)rs_lds, 16, 0, 0);
    }
    if (nch > 0) dma_chunk(0, buf0);
    if (nch > 1) dma_chunk(1, buf1);
    if (tail && lw == 0) {
      const uint8_t* trec = aop + (int64_t)full_tiles * rec + 16 * lane;
      for (int off = 0; off < rec; off += 1024)
        __builtin_amdgcn_global_load_lds((const void*)(trec + off),
                                         (__attribute__((address_space(3))) void*)(trec_lds + off), 16, 0, 0);
      const int tb = kPanelRows * tail_bytes;         // a multiple of 16, at most 1008
      const int o = min(16 * lane, tb - 16);
#pragma unroll
      for (int p = 0; p < P; ++p)
        __builtin_amdgcn_global_load_lds((const void*)(prow[p] + (int64_t)full_tiles * kTileBytes + o),
                                         (__attribute__((address_space(3))) void*)(tslot_lds + 1024 * p), 16, 0, 0);
    }
    wg_barrier();
    __builtin_amdgcn_s_waitcnt(0);                    // chunks 0, 1, the tail, the row scales
    wg_barrier();
    // The tail tile while the compute wavefronts multiply the first chunk
    // (its record and slots landed with chunk 0): at the end it would delay
    // the final reduction.
    if (tail && lw == 0) {
      // Slot (g, r) of the tail: bytes 16u + 4g .. + 3 of row r (zero past
      // the row's tail_bytes), as in load_tail_slot.
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
            const uint32_t byte = row[min(t, tail_bytes - 1)];       // unconditional read
            v |= (byte & (t < tail_bytes ? 0xFFu : 0u)) << (8 * k);
          }
          w[u] = v;
        }
        TS[p] = make_uint4(w[0], w[1], w[2], w[3]);
      }
      tile_mfma(trec_lds, TS);
    }
    for (int c = 0; c < nch; c += 2) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {                   // step c + k
        __builtin_amdgcn_s_waitcnt(0);                // chunk c + k + 1 is in LDS
        wg_barrier();
        if (c + k + 2 < nch) dma_chunk(c + k + 2, k == 0 ? buf0 : buf1);
        wg_barrier();
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
  } else {
    wg_barrier();
    issue_A(0, A0);
    issue_A(1, A1);
    wg_barrier();
    // Step c: chunk c is in LDS (`cur`), its slots (A) are requested; the
    // slots of chunk c + 2 are requested after its MFMAs unless it is one
    // of the last two steps (a request there would be waited for, a whole
    // memory round trip, before the epilogue).
    auto step = [&](int c, uint4 (&A)[TPC][P], uint8_t* cur, auto more) {
#pragma unroll
      for (int q = 0; q < TPC; ++q) {
        const int j = wave * TPC + q;                 // tile within the chunk
        if (c * CT + j < full_tiles) tile_mfma(cur + j * rec, A[q]);
      }
      wg_barrier();                                   // `cur` and A are free
      wg_barrier();                                   // chunk c + 2 requested
      if constexpr (decltype(more)::value) issue_A(c + 2, A);
    };
    // Unrolled by two for the two register sets; an odd chunk count ends
    // with one empty step (no tiles). As many steps as the loader's loop.
    int c = 0;
    for (; c + 2 < nch; c += 2) {
      step(c, A0, buf0, std::true_type{});
      step(c + 1, A1, buf1, std::true_type{});
    }
    if (c < nch) {
      step(c, A0, buf0, std::false_type{});
      step(c + 1, A1, buf1, std::false_type{});
    }
  }
  wg_barrier();                                      // LDS past the row scales is reused below

  // ---- add the wavefronts' accumulators in a fixed order and write y.
  uint8_t* red_base = buf0;
  f32x4* red = reinterpret_cast<f32x4*>(red_base);                   // [W+1][P][CS][64]
  float* tred = reinterpret_cast<float*>(red_base + (W + 1) * P * CS * 64 * 16);   // [W+1][16]
  // the compute wavefronts and the first loader (the others hold no products)
  if (wave <= W) {
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int cs = 0; cs < CS; ++cs) red[((wave * P + p) * CS + cs) * 64 + lane] = acc[p][cs];
    if (lane < 16) tred[wave * 16 + lane] = tacc;
  }
  wg_barrier();

  // One output (panel p, row, batch row b) per thread and pass: every LDS
  // read is issued before the sums (fixed order: terms, then wavefronts).
  const int nt = ncv / B;                           // 1..4
  const int items = P * B * 16;
  for (int item = threadIdx.x; item < items; item += 64 * (W + kLoaders)) {
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
        v[w][t] = red[((w * P + p) * CS + (cc >> 4)) * 64 + l][row & 3];
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
}

template <int P, int CS, int W, int TPC>
hipError_t launch_chunked_t(const SignTable& tab, int groups, const OperandShape& s, int64_t B,
                            bool y_bf16, const Fp6Plan& plan, hipStream_t stream) {
  const dim3 grid((unsigned)groups);
  const dim3 block(64 * (W + kLoaders));
  if (plan.lds_bytes > 160 * 1024) return hipErrorInvalidValue;   // a compute unit's LDS
  // Dynamic LDS beyond the default 64 KB limit has to be allowed per kernel.
  static size_t allowed = 0;
  if (plan.lds_bytes > allowed) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&sign_fp6_chunked_kernel<P, CS, W, TPC>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)plan.lds_bytes);
    if (e != hipSuccess) return e;
    allowed = plan.lds_bytes;
  }
  return launch_timed(sign_fp6_chunked_kernel<P, CS, W, TPC>, grid, block, plan.lds_bytes, stream,
                      tab, s.rec, s.ncv, (int)B, plan.chunk_bytes, y_bf16 ? 1 : 0);
}

}  // namespace

// Compute wavefronts and tiles per wavefront per chunk for each column-set
// count: wider operands take fewer tiles per chunk so that two chunks of
// activation records fit in LDS. (Registers: with W + 4 wavefronts a SIMD
// runs up to ceil((W + 4) / 4) of them, each with 512 / that many VGPRs.)
int chunked_waves(int p, int cs) { return cs == 1 ? (p >= 4 ? 4 : 8) : (cs == 2 && p < 8 ? 4 : 2); }
int chunked_tiles(int p, int cs) { return cs == 1 && p <= 4 ? 3 : 1; }

Fp6Plan plan_fp6_chunked(const PackedGeom& g, const OperandShape& s, int device_cus,
                         int panels_per_group) {
  // Panels per workgroup: the fewest that still give at most one workgroup
  // per compute unit (so that none streams more than its share), which also
  // lets as many panels as possible share each activation-operand read.
  const int64_t cus = device_cus > 0 ? device_cus : 256;
  const int most = s.cs >= 3 ? 4 : 8;          // register budget
  Fp6Plan p{};
  p.chunked = true;
  p.p = panels_per_group > 0
            ? panels_per_group
            : (int)std::min<int64_t>(most, std::max<int64_t>(1, (g.panels + cus - 1) / cus));
  p.w = chunked_waves(p.p, s.cs);
  const int budget = 112 * 1024;               // two chunks of activation records
  p.tpc = 1;
  const int tpc = chunked_tiles(p.p, s.cs);
  if (tpc > 1 && 2 * p.w * tpc * s.rec + 2048 <= budget) p.tpc = tpc;
  fill_chunks(&p, g, s);
  return p;
}

void fill_chunks(Fp6Plan* p, const PackedGeom& g, const OperandShape& s) {
  const int ct = p->w * p->tpc;
  p->nch = (g.full_tiles + ct - 1) / ct;
  p->chunk_bytes = ((ct * s.rec + 1023) / 1024) * 1024;
  const size_t red = (size_t)(p->w + 1) * p->p * s.cs * 64 * 16 + (size_t)(p->w + 1) * 16 * 4;
  const size_t tail = (size_t)((s.rec + 1023) / 1024) * 1024 + (size_t)1024 * p->p;
  p->lds_bytes = 1024 + std::max((size_t)2 * p->chunk_bytes + tail, red);
  p->pgroups = (int)((g.panels + p->p - 1) / p->p);
  p->groups = p->pgroups;
}

hipError_t launch_fp6_chunked_table(const SignTable& tab, int groups, const OperandShape& s,
                                    int64_t B, bool y_bf16, const Fp6Plan& plan,
                                    hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
#define LQ_FP6C_CASE(P_, CS_, TPC_)                                                         \
  if (plan.p == P_ && s.cs == CS_ && plan.tpc == TPC_ && plan.w == chunked_waves(P_, CS_))  \
    return launch_chunked_t<P_, CS_, (CS_ == 1 ? (P_ >= 4 ? 4 : 8) : (CS_ == 2 && P_ < 8 ? 4 : 2)), TPC_>( \
        tab, groups, s, B, y_bf16, plan, stream);
  LQ_FP6C_CASE(1, 1, 3) LQ_FP6C_CASE(2, 1, 3) LQ_FP6C_CASE(3, 1, 3) LQ_FP6C_CASE(4, 1, 3)
  LQ_FP6C_CASE(1, 1, 1) LQ_FP6C_CASE(2, 1, 1) LQ_FP6C_CASE(3, 1, 1) LQ_FP6C_CASE(4, 1, 1)
  LQ_FP6C_CASE(5, 1, 1) LQ_FP6C_CASE(6, 1, 1) LQ_FP6C_CASE(7, 1, 1) LQ_FP6C_CASE(8, 1, 1)
  LQ_FP6C_CASE(1, 2, 1) LQ_FP6C_CASE(2, 2, 1) LQ_FP6C_CASE(3, 2, 1) LQ_FP6C_CASE(4, 2, 1)
  LQ_FP6C_CASE(5, 2, 1) LQ_FP6C_CASE(6, 2, 1) LQ_FP6C_CASE(7, 2, 1) LQ_FP6C_CASE(8, 2, 1)
  LQ_FP6C_CASE(1, 3, 1) LQ_FP6C_CASE(2, 3, 1) LQ_FP6C_CASE(3, 3, 1) LQ_FP6C_CASE(4, 3, 1)
#undef LQ_FP6C_CASE
  return hipErrorInvalidValue;
}

}  // namespace lq
