// W-space large-batch product: y = diag(r) W xt^T with the dense weights
// W[n][b d + i] = sum_e M[i][e] s[n][b][e] rebuilt on the fly from the packed
// signs, so the matrix cores reduce over the K' = d Kb inputs instead of the
// L = D Kb lifted columns: D / d times fewer MACs than the lifted product
// ([paper] §3: the lifted form is the same linear map; the weights it
// represents are M times each block's sign vector).
//
// Operand construction (gfx950 v_mfma_f32_16x16x32_bf16, lane l = 16 g + r
// supplies row r of A and column r of B for the reduction indices of lane
// group g). For D dividing 32 the packed word u of slot (g, r) holds row r's
// sign bits of 32 / D whole blocks (tile columns 128 u + 32 g + [0, 32)), so
// lane (g, r) builds its W values from its own bits: the D-bit pattern of a
// block indexes a table of the 2^D possible weight vectors (4 bf16 each,
// positions i >= d zero), computed per workgroup in LDS from M (fp32 sums in
// order of e, then rounded to bf16 once). One A operand = two blocks, 8 bf16;
// a 128-column step gives F = 16 / D of them (sub-steps). The B operand of
// lane (g, r) in sub-step s carries the matching inputs: xt[16 jb + r][d b + i]
// for the same two blocks b, i < 4 (zero for i >= d and past K).
//
// xt is first written in that order ("xp", bf16): per 16 batch rows and
// 128-column step an F KB block of 16-byte units [s][g][r]; the whitening
// itself writes it (xt never goes to memory). The pipeline is
// that of the lifted large-batch product (four LDS stages filled by DMA three
// steps ahead, slots DMA-copied per tile, B operands and table reads of the
// next sub-step issued before this sub-step's MFMAs).
#include "lq_internal.h"
#include "lq_prep.h"

namespace lq {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ------------------------------------------------------------ whitening + xp
// Workgroup (chunk h of 1024 inputs, 16 batch rows jb): x * c of the rows'
// chunk into LDS, the Walsh-Hadamard transform of every hb block (a
// wavefront per row), then the xp units of every block with inputs in the
// chunk. Slot (block b, position i) belongs to the chunk holding input
// min(b d + min(i, d - 1), K - 1): a unit whose eight slots all belong to
// this chunk is stored whole, one that straddles two chunks slot by slot (2
// bytes each; the other chunk's workgroup stores the rest). The last chunk
// also covers the virtual pad and the blocks past L up to the end of the
// last tile (zeros).
constexpr int kXpwStride = 1028;   // LDS row stride (floats): 16-byte aligned, rows 4 banks apart

template <int D, bool kXBF16>
__global__ __launch_bounds__(256) void xpw_kernel(const void* __restrict__ x,
                                                  const float* __restrict__ c, int64_t B,
                                                  int64_t K, int d, int lhb, float norm,
                                                  int64_t steps, int64_t blk_end, int64_t jb_base,
                                                  uint4* __restrict__ xp) {
  constexpr int F = 16 / D;
  __shared__ __align__(16) float xs[16 * kXpwStride];
  const int h = blockIdx.x;
  const int64_t jb = jb_base + blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t k_lo = (int64_t)h * 1024;
  const int n = (int)min((int64_t)1024, K - k_lo);

  // x * c: thread t takes inputs 4t .. 4t + 3 of every row
  const int k4 = 4 * tid;
  float cv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) cv[i] = k4 + i < n ? c[k_lo + k4 + i] : 0.0f;
#pragma unroll 4
  for (int rr = 0; rr < 16; ++rr) {
    const int64_t b = 16 * jb + rr;
    float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (b < B) {
      const int64_t at = b * K + k_lo + k4;
      if (k4 + 3 < n && (at & 3) == 0) {
        if (kXBF16) {
          const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(x) + at);
          v[0] = bf16_bits_to_f32(w.x & 0xFFFFu); v[1] = bf16_bits_to_f32(w.x >> 16);
          v[2] = bf16_bits_to_f32(w.y & 0xFFFFu); v[3] = bf16_bits_to_f32(w.y >> 16);
        } else {
          const float4 w = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + at);
          v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (k4 + i < n)
            v[i] = kXBF16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(x)[at + i])
                          : reinterpret_cast<const float*>(x)[at + i];
      }
    }
    *reinterpret_cast<float4*>(xs + rr * kXpwStride + k4) =
        make_float4(v[0] * cv[0], v[1] * cv[1], v[2] * cv[2], v[3] * cv[3]);
  }
  __syncthreads();
  // (every hb block lies inside the chunk: hb divides 1024 and K; past n
  // the values are zero and stay zero)
  for (int rr = wave; rr < 16; rr += 4) wave_fwht_1024(xs + rr * kXpwStride, lhb, lane);
  __syncthreads();

  const bool last = k_lo + 1024 >= K;
  const int64_t b_first = k_lo / d;
  const int64_t b_last = last ? blk_end - 1 : (k_lo + 1023) / d;
  const int64_t u_lo = b_first / 2, nu = b_last / 2 - u_lo + 1;
  auto owner = [&](int64_t bb, int i) -> int64_t {
    return min(bb * d + min(i, d - 1), K - 1) >> 10;
  };
  for (int64_t idx = tid; idx < nu * 16; idx += 256) {
    const int64_t U = u_lo + (idx >> 4);
    const int r = (int)(idx & 15);
    const int64_t b0 = 2 * U;
    const int64_t col = b0 * D;
    const int64_t q = col >> 9;
    const int cu = (int)((col >> 7) & 3), g = (int)((col >> 5) & 3), s = (int)((col & 31) / D) >> 1;
    uint4* dst = xp + ((jb * steps + 4 * q + cu) * F + s) * 64 + 16 * g + r;
    const float* xr = xs + r * kXpwStride;
    uint32_t hv[8];
    bool own[8];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t k = (b0 + hh) * d + i;
        const bool o = owner(b0 + hh, i) == h;
        own[4 * hh + i] = o;
        hv[4 * hh + i] = f32_to_bf16_bits(o && i < d && k < K ? xr[k - k_lo] * norm : 0.0f);
      }
    if (own[0] && own[7]) {
      *dst = make_uint4(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16), hv[4] | (hv[5] << 16),
                        hv[6] | (hv[7] << 16));
    } else {
      uint16_t* p = reinterpret_cast<uint16_t*>(dst);
#pragma unroll
      for (int m = 0; m < 8; ++m)
        if (own[m]) p[m] = (uint16_t)hv[m];
    }
  }
}

// ------------------------------------------------------------ product
// Workgroup: 4 wavefronts; tile 4 PW panels x 16 JB batch rows; wavefront w
// owns panels w PW .. w PW + PW - 1 and all JB batch tiles.
template <int D, int PW, int JB, bool kYBF16>
__global__ __launch_bounds__(256) void wspace_kernel(
    const uint8_t* __restrict__ packed, int64_t panels, int64_t panel_bytes, int full_tiles,
    int ext_tiles, const uint4* __restrict__ xp, int64_t B16, int64_t B,
    const uint4* __restrict__ tail_slots, const float* __restrict__ M, int d,
    const float* __restrict__ row_scale, void* __restrict__ y, int64_t N) {
  constexpr int F = 16 / D;                       // sub-steps per step
  constexpr int kChunks = JB * F;                 // 1 KB chunks of a step's B operands
  constexpr int kStageUnits = kChunks * 64;       // [jb][s][g][r]
  constexpr int kSlotUnits = 4 * PW * 64;         // [wave][panel][lane]
  constexpr int kLut = 1 << D;
  __shared__ uint4 stage0[kStageUnits];
  __shared__ uint4 stage1[kStageUnits];
  __shared__ uint4 stage2[kStageUnits];
  __shared__ uint4 stage3[kStageUnits];
  __shared__ uint4 slotA[kSlotUnits];
  __shared__ uint4 slotB[kSlotUnits];
  __shared__ uint2 lut[kLut];
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int64_t steps = 4 * (int64_t)ext_tiles;
  const int64_t last = steps - 1;
  const int64_t jb0 = (int64_t)blockIdx.y * JB;
  const int64_t pbase = (int64_t)blockIdx.x * 4 * PW + wave * PW;

  // The weight vector of every sign pattern: entry p, value i = sum over e
  // of M[i][e] times (bit e of p ? -1 : +1), in order of e, rounded to bf16.
  for (int p = threadIdx.x; p < kLut; p += 256) {
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float a = 0.0f;
      if (i < d) {
#pragma unroll
        for (int e = 0; e < D; ++e) a = fmaf(M[i * D + e], ((p >> e) & 1) ? -1.0f : 1.0f, a);
      }
      h[i] = f32_to_bf16_bits(a);
    }
    lut[p] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  }

  auto dma = [&](const void* src, uint4* dst) {
    __builtin_amdgcn_global_load_lds(
        (const void*)(reinterpret_cast<const uint8_t*>(src) + 16 * lane),
        (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
  };
  // The B operands of one step: kChunks copies of 1 KB spread over the four
  // wavefronts (clamped: a repeated copy writes the same bytes again).
  constexpr int kCopies = (kChunks + 3) / 4;
  auto copy_step = [&](int64_t t, uint4* dst) {
#pragma unroll
    for (int k = 0; k < kCopies; ++k) {
      const int ch = min(wave + 4 * k, kChunks - 1);
      const int c = ch / F, s = ch % F;
      const int64_t jb = min(jb0 + c, B16 - 1);
      dma(xp + ((jb * steps + t) * F + s) * 64, dst + ch * 64);
    }
  };
  auto copy_slots = [&](int q, uint4* dst) {
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int64_t pnl = min(pbase + i, panels - 1);
      const void* src = q < full_tiles
                            ? (const void*)(packed + pnl * panel_bytes + (int64_t)q * kTileBytes)
                            : (const void*)(tail_slots + pnl * 64);
      dma(src, dst + (wave * PW + i) * 64);
    }
  };
  // A operand of sub-step s from word w: the table entries of blocks 2 s and
  // 2 s + 1 of the word.
  auto a_operand = [&](uint32_t w, int s) -> u32x4 {
    const uint2 e0 = lut[(w >> (2 * s * D)) & (kLut - 1)];
    const uint2 e1 = lut[(w >> ((2 * s + 1) * D)) & (kLut - 1)];
    return (u32x4){e0.x, e0.y, e1.x, e1.y};
  };

  f32x4 acc[PW][JB];
#pragma unroll
  for (int i = 0; i < PW; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j) acc[i][j] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

  // One step: F sub-steps. The B operands and table reads of the next
  // sub-step (for the last one, sub-step 0 of the next step, whose stage is
  // complete by then) are issued before the MFMAs of this one. At the last
  // sub-step of a tile the next tile's words are not loaded yet: its first A
  // operands are read at the start of the next step.
  auto mult = [&](const uint4* st, const uint4* st_next, const uint32_t (&w)[PW][4], int u,
                  uint4 (&bcur)[JB], u32x4 (&acur)[PW]) {
    uint4 bnext[JB];
    u32x4 anext[PW];
#pragma unroll
    for (int s = 0; s < F; ++s) {
#pragma unroll
      for (int c = 0; c < JB; ++c)
        bnext[c] = s < F - 1 ? st[(c * F + s + 1) * 64 + lane] : st_next[(c * F) * 64 + lane];
      if (s < F - 1 || u < 3) {
#pragma unroll
        for (int i = 0; i < PW; ++i) anext[i] = a_operand(w[i][s < F - 1 ? u : u + 1], (s + 1) % F);
      }
      // Keep those reads here: the scheduler would otherwise sink each one
      // next to its first use.
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < PW; ++i) {
#pragma unroll
        for (int c = 0; c < JB; ++c) {
          const u32x4 bop = {bcur[c].x, bcur[c].y, bcur[c].z, bcur[c].w};
          acc[i][c] = mfma_bf16(acur[i], bop, acc[i][c]);
        }
      }
#pragma unroll
      for (int c = 0; c < JB; ++c) bcur[c] = bnext[c];
      if (s < F - 1 || u < 3) {
#pragma unroll
        for (int i = 0; i < PW; ++i) acur[i] = anext[i];
      }
    }
  };

  // Copies are issued unconditionally (past the last step, the last step
  // again), so kCopies copy instructions follow those of step t + 1 when step
  // t begins: waiting until at most that many are outstanding means step
  // t + 1's copies, and everything issued before them, have landed.
  constexpr int kWait1 = (7 << 4) | (15 << 8) | (kCopies & 15) | ((kCopies >> 4) << 14);
  static_assert(kCopies <= 63, "vmcnt range");
  copy_slots(0, slotA);
  copy_step(0, stage0);
  copy_step(min((int64_t)1, last), stage1);
  copy_step(min((int64_t)2, last), stage2);
  uint4 bcur[JB];
  u32x4 acur[PW];

  auto tile = [&](int q, const uint4* slot_cur, uint4* slot_next) {
    uint32_t w[PW][4];
    const int64_t t0 = 4 * (int64_t)q;
#pragma unroll
    for (int u = 0; u < 4; ++u) {                // step t = t0 + u, stage u
      __builtin_amdgcn_s_waitcnt(kWait1);
      wg_barrier();                              // (the first one also publishes the table)
      if (u == 0) {
#pragma unroll
        for (int i = 0; i < PW; ++i) {
          const uint4 v = slot_cur[(wave * PW + i) * 64 + lane];
          w[i][0] = v.x; w[i][1] = v.y; w[i][2] = v.z; w[i][3] = v.w;
        }
        if (q == 0) {
#pragma unroll
          for (int c = 0; c < JB; ++c) bcur[c] = stage0[(c * F) * 64 + lane];
        }
#pragma unroll
        for (int i = 0; i < PW; ++i) acur[i] = a_operand(w[i][0], 0);
      }
      copy_step(min(t0 + u + 3, last), u == 0 ? stage3 : (u == 1 ? stage0 : (u == 2 ? stage1 : stage2)));
      if (u == 0) copy_slots(min(q + 1, ext_tiles - 1), slot_next);
      mult(u == 0 ? stage0 : (u == 1 ? stage1 : (u == 2 ? stage2 : stage3)),
           u == 0 ? stage1 : (u == 1 ? stage2 : (u == 2 ? stage3 : stage0)), w, u, bcur, acur);
    }
  };
  for (int q = 0; q < ext_tiles; q += 2) {
    tile(q, slotA, slotB);
    if (q + 1 < ext_tiles) tile(q + 1, slotB, slotA);
  }

  // No copy may still be writing LDS when the workgroup ends.
  __builtin_amdgcn_s_waitcnt(0);
  // Epilogue: lane (g, r) of tile (i, j) holds rows 4g..4g+3 of panel
  // pbase + i for batch row 16 (jb0 + j) + r.
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int64_t pnl = pbase + i;
    if (pnl >= panels) continue;
    const int64_t n0 = pnl * kPanelRows + 4 * g;
    const float4 rs = *reinterpret_cast<const float4*>(row_scale + n0);
#pragma unroll
    for (int j = 0; j < JB; ++j) {
      const int64_t b = 16 * (jb0 + j) + r;
      if (b >= B) continue;
      const float v0 = rs.x * acc[i][j][0], v1 = rs.y * acc[i][j][1];
      const float v2 = rs.z * acc[i][j][2], v3 = rs.w * acc[i][j][3];
      if (kYBF16) {
        uint16_t* yp = reinterpret_cast<uint16_t*>(y) + b * N + n0;
        const uint32_t lo = f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16);
        const uint32_t hi = f32_to_bf16_bits(v2) | (f32_to_bf16_bits(v3) << 16);
        *reinterpret_cast<uint2*>(yp) = make_uint2(lo, hi);
      } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + b * N + n0) = make_float4(v0, v1, v2, v3);
      }
    }
  }
}

template <int D, int PW, int JB, bool kYBF16>
hipError_t launch_ws_t(const uint8_t* packed, const PackedGeom& g, const uint4* xp, int64_t B,
                       const uint4* tail_slots, const float* M, int d, const float* row_scale,
                       void* y, hipStream_t stream) {
  const int64_t B16 = (B + 15) / 16;
  const dim3 grid((unsigned)((g.panels + 4 * PW - 1) / (4 * PW)), (unsigned)((B16 + JB - 1) / JB));
  return launch_timed(wspace_kernel<D, PW, JB, kYBF16>, grid, dim3(256), 0, stream, packed,
                      g.panels, g.panel_bytes, g.full_tiles, g.ext_tiles, xp, B16, B, tail_slots,
                      M, d, row_scale, y, g.N);
}

template <int D, bool kYBF16>
hipError_t launch_ws_y(const uint8_t* packed, const PackedGeom& g, const uint4* xp, int64_t B,
                       const uint4* tail_slots, const float* M, int d, const float* row_scale,
                       void* y, const LargePlan& p, hipStream_t stream) {
  // (D = 4: at most 4 batch tiles, or the four stages would not fit LDS)
#define LQ_WS_CASE(PW_, JB_)                                                                       \
  if constexpr ((16 / D) * JB_ <= 16) {                                                            \
    if (p.ppw == PW_ && p.jb == JB_)                                                               \
      return launch_ws_t<D, PW_, JB_, kYBF16>(packed, g, xp, B, tail_slots, M, d, row_scale, y,   \
                                              stream);                                             \
  }
  LQ_WS_CASE(8, 4) LQ_WS_CASE(8, 2) LQ_WS_CASE(8, 1)
  LQ_WS_CASE(4, 8) LQ_WS_CASE(4, 4) LQ_WS_CASE(4, 2) LQ_WS_CASE(4, 1)
  LQ_WS_CASE(2, 4) LQ_WS_CASE(2, 2) LQ_WS_CASE(2, 1)
  LQ_WS_CASE(1, 4) LQ_WS_CASE(1, 2) LQ_WS_CASE(1, 1)
#undef LQ_WS_CASE
  return hipErrorInvalidValue;
}

}  // namespace

bool wspace_supported(int d, int D) { return (D == 4 || D == 8) && d >= 1 && d <= 4 && d <= D; }

XpGeom xp_geom(int64_t B, const PackedGeom& g, int D) {
  XpGeom x;
  x.B16 = (B + 15) / 16;
  x.steps = 4 * (int64_t)g.ext_tiles;
  x.bytes = (size_t)x.B16 * x.steps * (16 / D) * 1024;
  x.tail_bytes = g.tail_bytes ? (size_t)g.panels * kTileBytes : 0;
  return x;
}

LargePlan plan_wspace(int64_t B, const PackedGeom& g, int D) {
  LargePlan p;
  const int64_t B16 = (B + 15) / 16;
  if (D == 8 && B16 >= 8 && ((g.panels + 15) / 16) * ((B16 + 7) / 8) >= 512) {
    p.jb = 8;
    p.ppw = 4;
    return p;
  }
  p.jb = B16 >= 4 ? 4 : (B16 >= 2 ? 2 : 1);
  const int64_t bt = (B16 + p.jb - 1) / p.jb;
  p.ppw = 1;
  for (int c : {8, 4, 2}) {
    if (((g.panels + 4 * c - 1) / (4 * c)) * bt >= 512) { p.ppw = c; break; }
  }
  return p;
}

hipError_t launch_xpw(const void* x, bool x_bf16, int64_t B, int64_t K, int hb, const float* c,
                      int d, int D, const PackedGeom& g, void* xp, hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
  if (!wspace_supported(d, D) || hb < 1 || hb > 1024 || (hb & (hb - 1)) || K % hb) return hipErrorInvalidValue;
  const XpGeom xg = xp_geom(B, g, D);
  int lhb = 0;
  while ((1 << lhb) < hb) ++lhb;
  const float norm = (lhb % 2 == 0) ? ldexpf(1.0f, -lhb / 2) : (float)(1.0 / sqrt((double)hb));
  const int64_t blk_end = (int64_t)g.ext_tiles * (kTileCols / D);
  const unsigned chunks = (unsigned)((K + 1023) / 1024);
  uint4* out = reinterpret_cast<uint4*>(xp);
  for (int64_t jb0 = 0; jb0 < xg.B16; jb0 += 65535) {
    const dim3 grid(chunks, (unsigned)min(xg.B16 - jb0, (int64_t)65535));
#define LQ_XPW(D_, BF_)                                                                            \
    hipLaunchKernelGGL((xpw_kernel<D_, BF_>), grid, dim3(256), 0, stream, x, c, B, K, d, lhb, norm, \
                       xg.steps, blk_end, jb0, out)
    if (D == 8) {
      if (x_bf16) LQ_XPW(8, true); else LQ_XPW(8, false);
    } else {
      if (x_bf16) LQ_XPW(4, true); else LQ_XPW(4, false);
    }
#undef LQ_XPW
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_wspace(const uint8_t* packed, const PackedGeom& g, const void* xp,
                         void* tail_slots, int64_t B, const float* M, int d, int D,
                         const float* row_scale, void* y, bool y_bf16, hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
  if (!wspace_supported(d, D)) return hipErrorInvalidValue;
  const LargePlan p = plan_wspace(B, g, D);
  const uint4* x = reinterpret_cast<const uint4*>(xp);
  uint4* ts = reinterpret_cast<uint4*>(tail_slots);
  if (g.tail_bytes) {
    const hipError_t e = launch_tail_slots(packed, g, ts, stream);
    if (e != hipSuccess) return e;
  }
  if (D == 8)
    return y_bf16 ? launch_ws_y<8, true>(packed, g, x, B, ts, M, d, row_scale, y, p, stream)
                  : launch_ws_y<8, false>(packed, g, x, B, ts, M, d, row_scale, y, p, stream);
  return y_bf16 ? launch_ws_y<4, true>(packed, g, x, B, ts, M, d, row_scale, y, p, stream)
                : launch_ws_y<4, false>(packed, g, x, B, ts, M, d, row_scale, y, p, stream);
}

}  // namespace lq
