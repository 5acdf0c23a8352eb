// Large-batch sign product on the bf16 matrix cores (gfx950
// v_mfma_f32_16x16x32_bf16): a tiled GEMM y = diag(r) S z^T for B > 16.
//
// Operand construction. In a 16x16x32 MFMA, lane l = 16*g + r supplies row r
// of the A tile and column r of the B tile, each for the 8 reduction indices
// of lane group g. A packed slot gives lane (g, r) exactly row r's bits for
// 32 columns per word (word u of slot (g, r): tile columns 128u + 32g + b), so
// the sign operand is built in registers, with no data exchange: the bf16 pair
// of A-dword j in sub-step s takes bits p = 4s + j and p + 16 of the word,
//   ((w << (15 - p)) & 0x80008000) | 0x3F803F80     (+1 = 0x3F80, -1 = 0xBF80),
// so the B operand of lane (g, r) in sub-step s must hold, as bf16 pairs,
// (z[c + j], z[c + j + 16]) for j = 0..3, c = 128u + 32g + 4s. The pairing of
// reduction indices inside one MFMA is the same for A and B by construction.
//
// z is first rewritten into exactly that order ("zp", one pass: from z for
// lq_sign_gemm, or straight from the lift for lq_linear): for every 16 batch
// rows and every 128-column step, a 4 KB block of 16-byte units
// [s][g][r] = the B operand of lane (g, r) in sub-step s. One 1 KB DMA then
// fills 64 consecutive units of LDS, and every LDS read of the product is
// one conflict-free 1 KB wavefront read. fp32 z is carried as two bf16
// terms, hi = bf16(z) and lo = bf16(z - hi), in two zp planes; bf16 z as is.
// Accumulation is fp32.
#include <algorithm>

#include "lq_internal.h"
#include "lq_prep.h"

namespace lq {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kZpBlock = 4096;   // bytes of one (16 rows x 128 columns) zp block

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// A operand (8 bf16 +-1) of sub-step s (0..3) from one packed word: per
// dword one shift and one and-or of the two sign bits into 1.0. The mask and
// the 1.0 pair are passed in registers (mask, one): with them as constants
// the compiler emits a separate and and or, since these three-operand
// instructions take no literal constants on this target.
__device__ __forceinline__ u32x4 sign_operand(uint32_t w, int s, uint32_t mask, uint32_t one) {
  u32x4 a;
  const int p0 = 4 * s;
  a.x = ((w << (15 - p0)) & mask) | one;
  a.y = ((w << (14 - p0)) & mask) | one;
  a.z = ((w << (13 - p0)) & mask) | one;
  a.w = ((w << (12 - p0)) & mask) | one;
  return a;
}

// A 32-bit constant in a vector register, opaque to constant folding.
__device__ __forceinline__ uint32_t vreg_const(uint32_t v) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
  return r;
}

// ------------------------------------------------------------ zp
// Workgroup (tile q, jb): batch rows 16 jb .. 16 jb + 15 and the tile's 512
// columns, i.e. the 4 KB blocks of steps 4q .. 4q + 3. Thread (u, g, r)
// (u = step in the tile) makes the 32 values of row 16 jb + r, columns
// c = 128 (4q + u) + 32 g + [0, 32), and writes units (s, g, r) of step
// 4q + u for s = 0..3: unit s holds columns c + 4s + {0..3} and
// c + 16 + 4s + {0..3}. For a fixed s the 64 lanes of a wavefront write
// 1 KB of consecutive units.
// kSrc 0: z fp32, 1: z bf16 (B x L, row-major), 2: lift from xt (B x K fp32)
// with M (the lq_linear path: z is never written in row-major form). For the
// lift the workgroup stages M and the rows' original columns [k_lo, k_lo +
// span) (span <= (511 / D + 2) d <= 639) in LDS (dynamic: max(d D, 256) +
// 16 xstride floats).
template <int kSrc, int NTERM>
__global__ __launch_bounds__(256) void zp_kernel(const void* __restrict__ src, int64_t B, int64_t L,
                                                 int64_t K, int d, int D,
                                                 const float* __restrict__ M, int64_t steps,
                                                 int64_t B16, int64_t jb_base, int xstride,
                                                 uint4* __restrict__ zp) {
  extern __shared__ float lds_f[];
  const int64_t q = blockIdx.x, jb = jb_base + blockIdx.y;
  const int t = threadIdx.x;
  const int u = t >> 6, g = (t >> 4) & 3, r = t & 15;
  const int64_t b = 16 * jb + r;
  const int64_t c_lo = 512 * q + 128 * u + 32 * g;
  float v[32];
  if (kSrc == 2) {
    // LDS: M (at least 256 slots, one per thread), then the staged rows
    const int nm = d * D;
    float* Ms = lds_f;
    float* xs = lds_f + max(nm, 256);
    // (32-bit index arithmetic: L <= 2^28)
    const int tile_lo = 512 * (int)q;
    const int blk_lo = tile_lo / D;
    const int blk_hi = min(tile_lo + 511, (int)L - 1) / D;
    const int64_t k_lo = (int64_t)blk_lo * d;
    // The tile's blocks cover inputs [k_lo, k_lo + span); those past K (the
    // virtual pad) are staged as zeros, so every block has d inputs.
    const int span = (blk_hi + 1 - blk_lo) * d;
    // All 16 rows' loads go out before the first is stored (span <= 639 <
    // 3 x 256): loading and storing a row at a time cost one memory round
    // trip per row. Addresses are clamped (rows to B - 1, inputs to the
    // span and to K - 1) and no load depends on a condition, so none is
    // put under a branch (a branch joins only after its load has landed).
    // Rows past B hold row B - 1's values; their outputs are zeroed below.
    const float* __restrict__ xsrc = reinterpret_cast<const float*>(src);
    const float m0 = M[min(t, nm - 1)];          // M's first 256 entries, before x
    float xv[16][3];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const float* xrow = xsrc + min(16 * jb + rr, B - 1) * K;
#pragma unroll
      for (int j = 0; j < 3; ++j) xv[rr][j] = xrow[min(k_lo + min(t + 256 * j, span - 1), K - 1)];
    }
    Ms[t] = m0;                                   // (slots past d D unused)
    for (int i = t + 256; i < nm; i += 256) Ms[i] = M[i];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int k = t + 256 * j;
        if (k < span) xs[xstride * rr + k] = k_lo + k < K ? xv[rr][j] : 0.0f;
      }
    __syncthreads();
    // Column c_lo + k is element eo[k] of the block whose inputs start at
    // xo[k] in the row's staged span (clamped for columns past L, whose
    // values are replaced by 0 below).
    const float* xr = xs + xstride * r;
    int xo[32], eo[32];
    {
      const int blk = (int)c_lo / D;
      int e = (int)c_lo - blk * D;
      int xoff = (blk - blk_lo) * d;
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        xo[k] = min(xoff, span - d);
        eo[k] = e;
        if (++e == D) {
          e = 0;
          xoff += d;
        }
      }
    }
    // z = sum_i M[i][e] xt[block d + i], in order of i for every column.
#pragma unroll
    for (int k = 0; k < 32; ++k) v[k] = 0.0f;
    for (int i = 0; i < d; ++i) {
      // all 64 reads of this i before its multiply-adds (interleaved, each
      // read would be waited for on its own)
      float mv[32], xx[32];
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        mv[k] = Ms[i * D + eo[k]];
        xx[k] = xr[xo[k] + i];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < 32; ++k) v[k] = fmaf(mv[k], xx[k], v[k]);
    }
#pragma unroll
    for (int k = 0; k < 32; ++k) v[k] = b < B && c_lo + k < L ? v[k] : 0.0f;
  } else {
    // 32 consecutive values (L % 8 == 0: every 8-value chunk is in or out).
#pragma unroll
    for (int k8 = 0; k8 < 4; ++k8) {
      const int64_t c = c_lo + 8 * k8;
      const bool in = b < B && c < L;
      if (kSrc == 1) {
        const uint4 w = in ? *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(src) + b * L + c)
                           : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          v[8 * k8 + 2 * h] = __uint_as_float(ww[h] << 16);
          v[8 * k8 + 2 * h + 1] = __uint_as_float(ww[h] & 0xFFFF0000u);
        }
      } else {
        const float* zr = reinterpret_cast<const float*>(src) + b * L + c;
        const float4 lo = in ? *reinterpret_cast<const float4*>(zr) : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 hi = in ? *reinterpret_cast<const float4*>(zr + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
        v[8 * k8 + 0] = lo.x; v[8 * k8 + 1] = lo.y; v[8 * k8 + 2] = lo.z; v[8 * k8 + 3] = lo.w;
        v[8 * k8 + 4] = hi.x; v[8 * k8 + 5] = hi.y; v[8 * k8 + 6] = hi.z; v[8 * k8 + 7] = hi.w;
      }
    }
  }
  const int64_t step = 4 * q + u;
  const int64_t base = (jb * steps + step) * (kZpBlock / 16) + g * 16 + r;
  const int64_t plane = B16 * steps * (kZpBlock / 16);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a0 = v[4 * s + j], a1 = v[16 + 4 * s + j];
      const uint32_t h0 = f32_to_bf16_bits(a0), h1 = f32_to_bf16_bits(a1);
      hi[j] = h0 | (h1 << 16);
      if (NTERM == 2) {
        const uint32_t l0 = f32_to_bf16_bits(a0 - bf16_bits_to_f32(h0));
        const uint32_t l1 = f32_to_bf16_bits(a1 - bf16_bits_to_f32(h1));
        lo[j] = l0 | (l1 << 16);
      }
    }
    zp[base + s * 64] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    if (NTERM == 2) zp[plane + base + s * 64] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
}

// ------------------------------------------------------------ tail slots
// The slots of the partial tail tile of every panel, assembled once into
// full-tile form (1 KB per panel), so that the product loads every tile's
// slot with one 16-byte load from one of two addresses. Thread = (panel, lane).
__global__ __launch_bounds__(256) void tail_slots_kernel(const uint8_t* __restrict__ packed,
                                                         int64_t panels, int64_t panel_bytes,
                                                         int full_tiles, int tail_bytes,
                                                         uint4* __restrict__ out) {
  const int64_t pnl = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (pnl >= panels) return;
  out[pnl * 64 + lane] =
      load_tail_slot(packed + pnl * panel_bytes, full_tiles, tail_bytes, lane >> 4, lane & 15);
}

// ------------------------------------------------------------ product
// Workgroup: 4 wavefronts; tile 4 PW panels (64 PW rows) x 16 JB batch rows.
// Wavefront w owns panels w PW .. w PW + PW - 1 and all JB batch tiles:
// each B operand read from LDS feeds PW MFMAs, each sign operand built in
// registers feeds JB (times the z terms). Four LDS stages, one per step of
// a 512-column tile: at step t the four wavefronts copy the zp blocks of
// step t + 3 into the stage of step t - 1 while they multiply step t. The
// stages are separate LDS arrays, so the compiler knows a copy into one
// does not alias the reads of another and does not make those reads wait
// for it. One barrier per step: every wavefront has waited for its own
// copies of step t (its copies of steps t + 1 and t + 2, issued later, may
// still be in flight: memory operations complete in order) and is done
// with step t - 1, whose stage the next copy overwrites. The packed slots
// go from memory straight into registers, one tile (4 steps) ahead.
// Reduction ranges: workgroup z takes tiles [z tps, min((z + 1) tps,
// ext_tiles)); with more than one range (a layer with too few panel and
// batch groups to fill the chip), each writes its fp32 sums, unscaled, to
// partial[z][b][n] and large_reduce_kernel adds the ranges in order.
template <int NTERM, int PW, int JB, bool kYBF16>
__global__ __launch_bounds__(256) void sign_mfma_large_kernel(
    const uint8_t* __restrict__ packed, int64_t panels, int64_t panel_bytes, int full_tiles,
    int tail_bytes, int ext_tiles, const uint4* __restrict__ zp, int64_t B16, int64_t B,
    const uint4* __restrict__ tail_slots, const float* __restrict__ row_scale,
    void* __restrict__ y, int64_t N, int tps, float* __restrict__ partial) {
  constexpr int kStageUnits = NTERM * JB * (kZpBlock / 16);   // [term][jb][s][g][r]
  constexpr int kSlotUnits = 4 * PW * 64;                      // [wave][panel][lane]
  __shared__ uint4 stage0[kStageUnits];
  __shared__ uint4 stage1[kStageUnits];
  __shared__ uint4 stage2[kStageUnits];
  __shared__ uint4 stage3[kStageUnits];
  __shared__ uint4 slotA[kSlotUnits];
  __shared__ uint4 slotB[kSlotUnits];
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int64_t steps = 4 * (int64_t)ext_tiles;
  const int q_lo = (int)blockIdx.z * tps;
  const int q_hi = min(q_lo + tps, ext_tiles);    // never empty (checked on the host)
  const int64_t last = 4 * (int64_t)q_hi - 1;      // the last step of this range
  const int64_t jb0 = (int64_t)blockIdx.y * JB;
  const int64_t pbase = (int64_t)blockIdx.x * 4 * PW + wave * PW;

  // A copy is a uniform base plus the lane's 16 bytes (a 32-bit offset).
  const uint32_t lane16 = 16u * (uint32_t)lane;
  auto dma = [&](const void* src, uint4* dst) {
    __builtin_amdgcn_global_load_lds((const void*)(reinterpret_cast<const uint8_t*>(src) + lane16),
                                     (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
  };
  // zp blocks of one step: NTERM * JB blocks of 4 KB, i.e. 4 NTERM JB
  // wavefront copies of 1 KB, spread over the 4 wavefronts. Copy c of step
  // t reads zp + ((term * B16 + jb) * steps + t) * kZpBlock + 1 KB * wave:
  // a base fixed for the workgroup plus t blocks.
  const uint8_t* cbase[NTERM * JB];
#pragma unroll
  for (int c = 0; c < NTERM * JB; ++c) {
    const int term = c / JB, j = c % JB;
    const int64_t jb = min(jb0 + j, B16 - 1);
    cbase[c] = reinterpret_cast<const uint8_t*>(zp) + (term * B16 + jb) * steps * kZpBlock + 1024 * wave;
  }
  auto copy_step = [&](int64_t t, uint4* dst) {
    const int64_t off = t * kZpBlock;
#pragma unroll
    for (int c = 0; c < NTERM * JB; ++c) dma(cbase[c] + off, dst + (c * kZpBlock + 1024 * wave) / 16);
  };
  // The slots (1 KB per panel: the tile itself, or its assembled tail) of
  // tile q for this wavefront's panels.
  const uint8_t* sbase[PW];
  const uint4* tbase[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int64_t pnl = min(pbase + i, panels - 1);
    sbase[i] = packed + pnl * panel_bytes;
    tbase[i] = tail_slots + pnl * 64;
  }
  auto copy_slots = [&](int q, uint4* dst) {
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const void* src = q < full_tiles ? (const void*)(sbase[i] + (int64_t)q * kTileBytes)
                                       : (const void*)tbase[i];
      dma(src, dst + (wave * PW + i) * 64);
    }
  };

  f32x4 acc[PW][JB];
#pragma unroll
  for (int i = 0; i < PW; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j) acc[i][j] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

  const uint32_t kMask = vreg_const(0x80008000u), kOne = vreg_const(0x3F803F80u);
  // One step: 4 sub-steps. The B operands of the next sub-step (for the last
  // one, sub-step 0 of the next step, whose stage is complete by then) are
  // read from LDS before the MFMAs of this one are issued, so that the LDS
  // latency hides behind them; the sign operands of the next sub-step are
  // built into other registers while these MFMAs run (building them into the
  // registers the MFMAs still read would stall on those reads). At the last
  // sub-step of a tile the next tile's words are not loaded yet: its first
  // sign operands are built at the start of the next step.
  constexpr int NB = NTERM * JB;
  auto mult = [&](const uint4* st, const uint4* st_next, const uint32_t (&w)[PW][4], int u,
                  uint4 (&bcur)[NB], u32x4 (&acur)[PW]) {
    uint4 bnext[NB];
    u32x4 anext[PW];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int c = 0; c < NB; ++c)
        bnext[c] = s < 3 ? st[(c * 4 + s + 1) * 64 + lane] : st_next[(c * 4) * 64 + lane];
      // Keep those reads here: the scheduler would otherwise sink each one
      // next to its first use.
      __builtin_amdgcn_sched_barrier(0);
      if (s < 3 || u < 3) {
#pragma unroll
        for (int i = 0; i < PW; ++i)
          anext[i] = sign_operand(w[i][s < 3 ? u : u + 1], (s + 1) & 3, kMask, kOne);
      }
#pragma unroll
      for (int i = 0; i < PW; ++i) {
#pragma unroll
        for (int c = 0; c < NB; ++c) {
          const u32x4 bop = {bcur[c].x, bcur[c].y, bcur[c].z, bcur[c].w};
          acc[i][c % JB] = mfma_bf16(acur[i], bop, acc[i][c % JB]);
        }
      }
#pragma unroll
      for (int c = 0; c < NB; ++c) bcur[c] = bnext[c];
      if (s < 3 || u < 3) {
#pragma unroll
        for (int i = 0; i < PW; ++i) acur[i] = anext[i];
      }
    }
  };

  // Every step issues its copies unconditionally (past the last step, the
  // last step again, into a stage no later step reads), so that at least
  // kCopies copy instructions follow those of step t + 1 when step t
  // begins: waiting until at most that many are outstanding means the copies
  // of step t + 1, and every copy issued before them (the slots of the
  // current tile among them), have landed. After the barrier, stages t and
  // t + 1 are complete.
  constexpr int kCopies = NTERM * JB;
  constexpr int kWait1 = (7 << 4) | (15 << 8) | (kCopies & 15) | ((kCopies >> 4) << 14);
  static_assert(kCopies <= 63, "vmcnt range");
  const int64_t t_lo = 4 * (int64_t)q_lo;
  copy_slots(q_lo, slotA);
  copy_step(t_lo, stage0);
  copy_step(min(t_lo + 1, last), stage1);
  copy_step(min(t_lo + 2, last), stage2);
  uint4 bcur[NB];
  u32x4 acur[PW];

  auto tile = [&](int q, const uint4* slot_cur, uint4* slot_next) {
    uint32_t w[PW][4];
    const int64_t t0 = 4 * (int64_t)q;
#pragma unroll
    for (int u = 0; u < 4; ++u) {                // step t = t0 + u, stage u
      __builtin_amdgcn_s_waitcnt(kWait1);
      wg_barrier();
      if (u == 0) {
#pragma unroll
        for (int i = 0; i < PW; ++i) {
          const uint4 v = slot_cur[(wave * PW + i) * 64 + lane];
          w[i][0] = v.x; w[i][1] = v.y; w[i][2] = v.z; w[i][3] = v.w;
        }
        if (q == q_lo) {
#pragma unroll
          for (int c = 0; c < NB; ++c) bcur[c] = stage0[(c * 4) * 64 + lane];
        }
#pragma unroll
        for (int i = 0; i < PW; ++i) acur[i] = sign_operand(w[i][0], 0, kMask, kOne);
      }
      copy_step(min(t0 + u + 3, last), u == 0 ? stage3 : (u == 1 ? stage0 : (u == 2 ? stage1 : stage2)));
      if (u == 0) copy_slots(min(q + 1, q_hi - 1), slot_next);
      mult(u == 0 ? stage0 : (u == 1 ? stage1 : (u == 2 ? stage2 : stage3)),
           u == 0 ? stage1 : (u == 1 ? stage2 : (u == 2 ? stage3 : stage0)), w, u, bcur, acur);
    }
  };
  for (int q = q_lo; q < q_hi; q += 2) {
    tile(q, slotA, slotB);
    if (q + 1 < q_hi) tile(q + 1, slotB, slotA);
  }

  // No copy may still be writing LDS when the workgroup ends.
  __builtin_amdgcn_s_waitcnt(0);
  // Epilogue: lane (g, r) of tile (i, j) holds rows 4g..4g+3 of panel
  // pbase + i for batch row 16 (jb0 + j) + r.
  const int g = lane >> 4, r = lane & 15;
  if (gridDim.z > 1) {
    float* part = partial + (int64_t)blockIdx.z * B * N;
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int64_t pnl = pbase + i;
      if (pnl >= panels) continue;
      const int64_t n0 = pnl * kPanelRows + 4 * g;
#pragma unroll
      for (int j = 0; j < JB; ++j) {
        const int64_t b = 16 * (jb0 + j) + r;
        if (b >= B) continue;
        *reinterpret_cast<float4*>(part + b * N + n0) =
            make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      }
    }
    return;
  }
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

// y[b][n] = r[n] * (the reduction ranges' partial sums added in order), four
// outputs per thread (N is a multiple of 16).
__global__ __launch_bounds__(256) void large_reduce_kernel(const float* __restrict__ partial,
                                                           int ksplit, int64_t B, int64_t N,
                                                           const float* __restrict__ row_scale,
                                                           void* __restrict__ y, int y_bf16) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;   // b * N + n
  if (i >= B * N) return;
  const int64_t n = i % N;
  float4 s = *reinterpret_cast<const float4*>(partial + i);
  for (int k = 1; k < ksplit; ++k) {
    const float4 v = *reinterpret_cast<const float4*>(partial + (int64_t)k * B * N + i);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  const float4 rs = *reinterpret_cast<const float4*>(row_scale + n);
  const float v0 = rs.x * s.x, v1 = rs.y * s.y, v2 = rs.z * s.z, v3 = rs.w * s.w;
  if (y_bf16) {
    const uint32_t lo = f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16);
    const uint32_t hi = f32_to_bf16_bits(v2) | (f32_to_bf16_bits(v3) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + i) = make_uint2(lo, hi);
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + i) = make_float4(v0, v1, v2, v3);
  }
}

template <int NTERM, int PW, int JB, bool kYBF16>
hipError_t launch_large_t(const uint8_t* packed, const PackedGeom& g, const uint4* zp, int64_t B,
                          const uint4* tail_slots, const float* row_scale, void* y,
                          const LargePlan& p, float* partial, hipStream_t stream) {
  const int64_t B16 = (B + 15) / 16;
  const dim3 grid((unsigned)((g.panels + 4 * PW - 1) / (4 * PW)), (unsigned)((B16 + JB - 1) / JB),
                  (unsigned)p.ksplit);
  if (p.ksplit > 1 && partial == nullptr) return hipErrorInvalidValue;
  if ((int64_t)(p.ksplit - 1) * p.tps >= g.ext_tiles) return hipErrorInvalidValue;   // an empty range
  // Timed as one product: the first kernel records the start event, the
  // reduction the stop.
  LaunchEvents& ev = launch_events();
  const LaunchEvents taken = ev;
  if (p.ksplit > 1) ev.stop = nullptr;
  const hipError_t e = launch_timed(sign_mfma_large_kernel<NTERM, PW, JB, kYBF16>, grid, dim3(256), 0,
                                    stream, packed, g.panels, g.panel_bytes, g.full_tiles,
                                    g.tail_bytes, g.ext_tiles, zp, B16, B, tail_slots, row_scale, y,
                                    g.N, p.tps, partial);
  if (e != hipSuccess || p.ksplit == 1) return e;
  const int64_t quads = B * g.N / 4;
  const dim3 rgrid((unsigned)((quads + 255) / 256));
  if (taken.start != nullptr)
    hipExtLaunchKernelGGL(large_reduce_kernel, rgrid, dim3(256), 0u, stream, nullptr, taken.stop, 0u,
                          (const float*)partial, p.ksplit, B, g.N, row_scale, y, kYBF16 ? 1 : 0);
  else
    hipLaunchKernelGGL(large_reduce_kernel, rgrid, dim3(256), 0, stream, (const float*)partial,
                       p.ksplit, B, g.N, row_scale, y, kYBF16 ? 1 : 0);
  return hipGetLastError();
}

template <int NTERM, bool kYBF16>
hipError_t launch_large_y(const uint8_t* packed, const PackedGeom& g, const uint4* zp, int64_t B,
                          const uint4* tail_slots, const float* row_scale, void* y,
                          const LargePlan& p, float* partial, hipStream_t stream) {
  // (fp32 z: at most 2 batch tiles, or the LDS stages would not fit)
#define LQ_LARGE_CASE(PW_, JB_)                                                                    \
  if constexpr (NTERM * JB_ <= 4 || (NTERM == 1 && JB_ == 8 && PW_ == 4)) {                        \
    if (p.ppw == PW_ && p.jb == JB_)                                                               \
      return launch_large_t<NTERM, PW_, JB_, kYBF16>(packed, g, zp, B, tail_slots, row_scale, y,  \
                                                     p, partial, stream);                          \
  }
  LQ_LARGE_CASE(8, 4) LQ_LARGE_CASE(8, 2) LQ_LARGE_CASE(8, 1)
  LQ_LARGE_CASE(4, 8) LQ_LARGE_CASE(4, 4) LQ_LARGE_CASE(4, 2) LQ_LARGE_CASE(4, 1)
  LQ_LARGE_CASE(2, 4) LQ_LARGE_CASE(2, 2) LQ_LARGE_CASE(2, 1)
  LQ_LARGE_CASE(1, 4) LQ_LARGE_CASE(1, 2) LQ_LARGE_CASE(1, 1)
#undef LQ_LARGE_CASE
  return hipErrorInvalidValue;
}

}  // namespace

ZpGeom zp_geom(int64_t B, const PackedGeom& g, bool z_bf16) {
  ZpGeom z;
  z.B16 = (B + 15) / 16;
  z.steps = 4 * (int64_t)g.ext_tiles;
  z.nterm = z_bf16 ? 1 : 2;
  z.bytes = (size_t)z.nterm * z.B16 * z.steps * kZpBlock;
  z.tail_bytes = g.tail_bytes ? (size_t)g.panels * kTileBytes : 0;
  return z;
}

LargePlan plan_large(int64_t B, const PackedGeom& g, bool z_bf16) {
  LargePlan p;
  p.ksplit = 1;
  p.tps = g.ext_tiles;
  p.partial_bytes = 0;
  const int64_t B16 = (B + 15) / 16;
  // bf16 z with >= 128 batch rows: 4 panels x 8 batch tiles per wavefront
  // (each sign operand feeds 8 MFMAs), when that still gives >= 512
  // workgroups; the four stages of 32 KB and the slots then fill LDS.
  if (z_bf16 && B16 >= 8 && ((g.panels + 15) / 16) * ((B16 + 7) / 8) >= 512) {
    p.jb = 8;
    p.ppw = 4;
    return p;
  }
  // fp32 z (two bf16 planes): at most 2 batch tiles, or the stages would
  // not fit LDS.
  p.jb = B16 >= 4 && z_bf16 ? 4 : (B16 >= 2 ? 2 : 1);
  const int64_t bt = (B16 + p.jb - 1) / p.jb;
  // The most panels per wavefront that still give >= 512 workgroups.
  p.ppw = 1;
  for (int c : {8, 4, 2}) {
    if (((g.panels + 4 * c - 1) / (4 * c)) * bt >= 512) { p.ppw = c; break; }
  }
  // None does, with 4 batch tiles: 2 panels per wavefront (each B operand
  // read from LDS then feeds twice the MFMAs) if, with the reduction split
  // below, the launch still has a workgroup for every compute unit
  // (Qwen-2.5-32B up / down at B = 64: product 59 -> 55 us).
  if (p.ppw == 1 && p.jb == 4) {
    const int64_t w2 = ((g.panels + 7) / 8) * bt;
    const int64_t k2 = std::min<int64_t>(512 / std::max<int64_t>(w2, 1), g.ext_tiles / 8);
    if (w2 * std::max<int64_t>(k2, 1) >= 256) p.ppw = 2;
  }
  // Still fewer than 512 (two per compute unit fit its LDS at these
  // tilings): split the reduction into ranges of at least 8 tiles, as many
  // as keep the workgroups within 512.
  const int64_t wgs = ((g.panels + 4 * p.ppw - 1) / (4 * p.ppw)) * bt;
  const int64_t ks = std::min<int64_t>(512 / std::max<int64_t>(wgs, 1), g.ext_tiles / 8);
  if (ks >= 2) {
    p.tps = (int)((g.ext_tiles + ks - 1) / ks);
    p.ksplit = (int)((g.ext_tiles + p.tps - 1) / p.tps);    // no empty range
    p.partial_bytes = (size_t)p.ksplit * (size_t)B * (size_t)g.N * sizeof(float);
  }
  return p;
}

hipError_t launch_zp(const void* src, int kind, int64_t B, int64_t L, int64_t K, int d, int D,
                     const float* M, const PackedGeom& g, void* zp, hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
  const ZpGeom z = zp_geom(B, g, kind == 1 || kind == 3);
  uint4* out = reinterpret_cast<uint4*>(zp);
  // Lift: LDS for M and 16 rows of the tile's original columns (odd stride).
  const int span_max = kind >= 2 ? (int)((511 / D + 2) * d) : 0;
  const int xstride = span_max | 1;
  const size_t lds = kind >= 2 ? (size_t)(std::max(d * D, 256) + 16 * xstride) * sizeof(float) : 0;
  // Batch tiles map to grid.y, at most 65535 per launch.
  for (int64_t jb0 = 0; jb0 < z.B16; jb0 += 65535) {
    const dim3 grid((unsigned)g.ext_tiles, (unsigned)min(z.B16 - jb0, (int64_t)65535));
    switch (kind) {
      case 0: hipLaunchKernelGGL((zp_kernel<0, 2>), grid, dim3(256), lds, stream, src, B, L, K, d, D, M, z.steps, z.B16, jb0, xstride, out); break;
      case 1: hipLaunchKernelGGL((zp_kernel<1, 1>), grid, dim3(256), lds, stream, src, B, L, K, d, D, M, z.steps, z.B16, jb0, xstride, out); break;
      case 2: hipLaunchKernelGGL((zp_kernel<2, 2>), grid, dim3(256), lds, stream, src, B, L, K, d, D, M, z.steps, z.B16, jb0, xstride, out); break;
      case 3: hipLaunchKernelGGL((zp_kernel<2, 1>), grid, dim3(256), lds, stream, src, B, L, K, d, D, M, z.steps, z.B16, jb0, xstride, out); break;
      default: return hipErrorInvalidValue;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_tail_slots(const uint8_t* packed, const PackedGeom& g, void* out,
                             hipStream_t stream) {
  hipLaunchKernelGGL(tail_slots_kernel, dim3((unsigned)((g.panels + 3) / 4)), dim3(256), 0, stream,
                     packed, g.panels, g.panel_bytes, g.full_tiles, g.tail_bytes,
                     reinterpret_cast<uint4*>(out));
  return hipGetLastError();
}

hipError_t launch_sign_mfma_large(const uint8_t* packed, const PackedGeom& g, const void* zp,
                                  void* tail_slots, bool z_bf16, int64_t B,
                                  const float* row_scale, void* y, bool y_bf16, float* partial,
                                  hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
  const LargePlan p = plan_large(B, g, z_bf16);
  const uint4* z = reinterpret_cast<const uint4*>(zp);
  uint4* ts = reinterpret_cast<uint4*>(tail_slots);
  if (g.tail_bytes) {
    const hipError_t e = launch_tail_slots(packed, g, ts, stream);
    if (e != hipSuccess) return e;
  }
  if (z_bf16)
    return y_bf16 ? launch_large_y<1, true>(packed, g, z, B, ts, row_scale, y, p, partial, stream)
                  : launch_large_y<1, false>(packed, g, z, B, ts, row_scale, y, p, partial, stream);
  return y_bf16 ? launch_large_y<2, true>(packed, g, z, B, ts, row_scale, y, p, partial, stream)
                : launch_large_y<2, false>(packed, g, z, B, ts, row_scale, y, p, partial, stream);
}

}  // namespace lq
