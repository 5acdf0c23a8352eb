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
// block indexes a table of the 2^D possible weight vectors (fp32 sums in
// order of e, rounded to bf16 once; 4 bf16 per entry, zero past d), computed
// per workgroup in LDS from M. A step is 8 blocks of every lane (D / 4 words:
// 256 tile columns for D = 8, 128 for D = 4); their 8 d weights, block after
// block, are exactly d A operands of 8 bf16 (sub-steps), no padding. The B
// operand of lane (g, r) in sub-step f carries the matching inputs:
// xt[16 jb + r][b d + i] for the same stream positions 8 f .. 8 f + 7 (zero
// past K).
//
// xt is first written in that order ("xp", bf16): per 16 batch rows and step
// a d KB block of 16-byte units [f][g][r]; the whitening itself writes it
// (xt never goes to memory). The pipeline is that of the lifted large-batch
// product (four LDS stages filled by DMA three steps ahead, slots
// DMA-copied per tile, B operands of the next sub-step read before this
// sub-step's MFMAs).
#include <type_traits>

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
// Workgroup (chunk h of 1024 inputs, 8 batch rows): wavefront w whitens rows
// w and w + 4 of the chunk (x * c, then the Walsh-Hadamard transform of every
// hb block, in registers with one pass through a per-wavefront LDS buffer),
// scales by 1/sqrt(hb) and keeps the bf16 results in LDS. Then every thread
// builds whole lane-steps (step t, lane group g, row r): the 8 d values of a
// step, which are BPW-block runs of consecutive inputs, and stores their d
// units. Input k belongs to the chunk holding min(k, K - 1): a lane-step
// whose values all lie in this chunk is stored whole, one that straddles
// chunks value by value (2 bytes each; the other chunk's workgroup stores
// the rest). The last chunk also covers the virtual pad and the blocks past
// L up to the end of the last tile (zeros).
constexpr int kXpwRows = 8;
constexpr int kXpwOut = 1040;      // bf16 per LDS row: rows 8 banks apart

// Stages 0..9 of the transform (those below lhb) of the 1024 values whose
// lane l holds 16 l + j in a[j], in the order of the shared wavefront
// transform; the scaled bf16 results go to out[0..1023].
__device__ __forceinline__ void fwht_row_to_bf16(float (&a)[16], float* buf, int lhb, int lane,
                                                 float norm, uint16_t* out) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s < lhb) {
      const int hs = 1 << s;
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if ((k & hs) == 0) {
          const float x0 = a[k], x1 = a[k | hs];
          a[k] = x0 + x1;
          a[k | hs] = x0 - x1;
        }
    }
  }
  if (lhb > 4) lane_stage<1>(a, lane);
  if (lhb > 5) lane_stage<2>(a, lane);
  float4* dst = reinterpret_cast<float4*>(buf + 16 * lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = make_float4(a[4 * i], a[4 * i + 1], a[4 * i + 2], a[4 * i + 3]);
  // The wavefront's own LDS writes are seen by its later reads.
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int k = 0; k < 16; ++k) a[k] = buf[lane + 64 * k];
#pragma unroll
  for (int s = 6; s < 10; ++s) {
    if (s < lhb) {
      const int hs = 1 << (s - 6);
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if ((k & hs) == 0) {
          const float x0 = a[k], x1 = a[k | hs];
          a[k] = x0 + x1;
          a[k | hs] = x0 - x1;
        }
    }
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) out[lane + 64 * k] = (uint16_t)f32_to_bf16_bits(a[k] * norm);
}

template <int D, int DD, bool kXBF16>
__global__ __launch_bounds__(256) void xpw_kernel(const void* __restrict__ x,
                                                  const float* __restrict__ c, int64_t B,
                                                  int64_t K, int lhb, float norm, int64_t steps,
                                                  int64_t blk_end, int64_t jr_base,
                                                  uint4* __restrict__ xp) {
  __shared__ __align__(16) float buf[4][1024];
  __shared__ __align__(16) uint16_t xo[kXpwRows * kXpwOut];
  const int h = blockIdx.x;
  const int64_t jr = jr_base + blockIdx.y;        // rows 8 jr .. 8 jr + 7
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t k_lo = (int64_t)h * 1024;
  const int n = (int)min((int64_t)1024, K - k_lo);
  const int k16 = 16 * lane;

  // x * c: lane l takes inputs 16 l .. 16 l + 15 of its wavefront's rows
  float cv[16], a[2][16];
  const bool full = k16 + 16 <= n;
  if (full && (reinterpret_cast<uintptr_t>(c) & 15) == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = *reinterpret_cast<const float4*>(c + k_lo + k16 + 4 * i);
      cv[4 * i] = v.x; cv[4 * i + 1] = v.y; cv[4 * i + 2] = v.z; cv[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) cv[j] = k16 + j < n ? c[k_lo + k16 + j] : 0.0f;
  }
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int64_t b = 8 * jr + wave + 4 * m;
    const int64_t at = b * K + k_lo + k16;
#pragma unroll
    for (int j = 0; j < 16; ++j) a[m][j] = 0.0f;
    if (b < B) {
      if (full && (at & 7) == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0) {
        if constexpr (kXBF16) {
          const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + at);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const uint4 w = p[i];
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              a[m][8 * i + 2 * e] = bf16_bits_to_f32(ww[e] & 0xFFFFu);
              a[m][8 * i + 2 * e + 1] = bf16_bits_to_f32(ww[e] >> 16);
            }
          }
        } else {
          const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + at);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float4 w = p[i];
            a[m][4 * i] = w.x; a[m][4 * i + 1] = w.y; a[m][4 * i + 2] = w.z; a[m][4 * i + 3] = w.w;
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (k16 + j < n)
            a[m][j] = kXBF16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(x)[at + j])
                             : reinterpret_cast<const float*>(x)[at + j];
      }
    }
  }
  // (every hb block lies inside the chunk: hb divides 1024 and K; past n
  // the values are zero and stay zero)
#pragma unroll
  for (int m = 0; m < 2; ++m) {
#pragma unroll
    for (int j = 0; j < 16; ++j) a[m][j] *= cv[j];
    fwht_row_to_bf16(a[m], buf[wave], lhb, lane, norm, xo + (wave + 4 * m) * kXpwOut);
  }
  __syncthreads();

  constexpr int BPT = 512 / D;                    // blocks per tile
  constexpr int WPS = D / 4;                      // packed words per step = runs per lane-step
  constexpr int SPT = 4 / WPS;                    // steps per tile
  constexpr int BPW = 32 / D;                     // blocks per word = per run
  constexpr int RUN = BPW * DD;                   // inputs per run (even)
  const int64_t k_hi = k_lo + n;                  // this chunk's inputs: [k_lo, k_hi)
  const bool last = k_lo + 1024 >= K;
  const int64_t b_first = k_lo / DD;
  const int64_t b_last = last ? blk_end - 1 : (k_lo + 1023) / DD;
  const int64_t q_lo = b_first / BPT, nq = b_last / BPT - q_lo + 1;
  const int64_t jb = jr >> 1;
  const int r16 = 8 * (int)(jr & 1);
  // items: (tile, step, lane group, row), row fastest
  const int64_t items = nq * SPT * 4 * kXpwRows;
  for (int64_t idx = tid; idx < items; idx += 256) {
    const int r = (int)(idx & 7);
    const int g = (int)((idx >> 3) & 3);
    const int64_t rest = idx >> 5;
    const int sg = (int)(rest % SPT);
    const int64_t q = q_lo + rest / SPT;
    const int64_t t = q * SPT + sg;
    uint4* dst = xp + (jb * steps + t) * DD * 64 + 16 * g + r16 + r;
    const uint16_t* row = xo + r * kXpwOut;
    int64_t k0[WPS];
    bool fast = true;
#pragma unroll
    for (int R = 0; R < WPS; ++R) {
      k0[R] = (q * BPT + (sg * WPS + R) * (BPT / 4) + g * BPW) * DD;
      fast = fast && k0[R] >= k_lo && k0[R] + RUN <= k_hi;
    }
    if (fast) {
      // the runs' RUN / 2 words each, in stream order, are the d units
      uint32_t wv[4 * DD];
#pragma unroll
      for (int R = 0; R < WPS; ++R) {
        const uint2* p = reinterpret_cast<const uint2*>(row + (k0[R] - k_lo));
#pragma unroll
        for (int i = 0; i < RUN / 4; ++i) {
          const uint2 v = p[i];
          wv[R * (RUN / 2) + 2 * i] = v.x;
          wv[R * (RUN / 2) + 2 * i + 1] = v.y;
        }
      }
#pragma unroll
      for (int f = 0; f < DD; ++f)
        dst[f * 64] = make_uint4(wv[4 * f], wv[4 * f + 1], wv[4 * f + 2], wv[4 * f + 3]);
    } else {
#pragma unroll
      for (int R = 0; R < WPS; ++R) {
#pragma unroll
        for (int e = 0; e < RUN; ++e) {
          const int64_t k = k0[R] + e;
          if ((min(k, K - 1) >> 10) != h) continue;
          const uint16_t v = k < K ? row[k - k_lo] : (uint16_t)0;
          const int p = R * RUN + e;                   // stream position
          reinterpret_cast<uint16_t*>(dst + (p >> 3) * 64)[p & 7] = v;
        }
      }
    }
  }
}

// ------------------------------------------------------------ product
// Workgroup: 4 wavefronts; tile 4 PW panels x 16 JB batch rows; wavefront w
// owns panels w PW .. w PW + PW - 1 and all JB batch tiles.
constexpr int kWsPW = kWsPanelsPerWave;

// The DD A operands of one step from the table entries e[0..7] of its 8
// blocks (entry j: dwords .x = v0 | v1 << 16, .y = v2 | v3 << 16, zero past
// DD): the stream of 8 DD weights, block after block, cut into operands of 8.
template <int DD>
__device__ __forceinline__ void pack_step(const uint2 (&e)[8], u32x4 (&a)[DD]) {
  if constexpr (DD == 4) {
#pragma unroll
    for (int f = 0; f < 4; ++f)
      a[f] = (u32x4){e[2 * f].x, e[2 * f].y, e[2 * f + 1].x, e[2 * f + 1].y};
  } else if constexpr (DD == 2) {
#pragma unroll
    for (int f = 0; f < 2; ++f)
      a[f] = (u32x4){e[4 * f].x, e[4 * f + 1].x, e[4 * f + 2].x, e[4 * f + 3].x};
  } else if constexpr (DD == 1) {
    a[0] = (u32x4){e[0].x | (e[1].x << 16), e[2].x | (e[3].x << 16), e[4].x | (e[5].x << 16),
                   e[6].x | (e[7].x << 16)};
  } else {
    // three bf16 per block: a pair of blocks (x, y) fills three dwords
    uint32_t dw[12];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint2 x = e[2 * j], y = e[2 * j + 1];
      dw[3 * j] = x.x;
      dw[3 * j + 1] = x.y | (y.x << 16);
      dw[3 * j + 2] = __builtin_amdgcn_alignbit(y.y, y.x, 16);
    }
#pragma unroll
    for (int f = 0; f < 3; ++f) a[f] = (u32x4){dw[4 * f], dw[4 * f + 1], dw[4 * f + 2], dw[4 * f + 3]};
  }
}

template <int D, int DD, int JB>
__global__ __launch_bounds__(256) void wspace_kernel(
    const uint8_t* __restrict__ packed, int64_t panels, int64_t panel_bytes, int full_tiles,
    int ext_tiles, const uint4* __restrict__ xp, int64_t B16, int64_t B,
    const uint4* __restrict__ tail_slots, const float* __restrict__ M, int y_bf16,
    const float* __restrict__ row_scale, void* __restrict__ y, int64_t N) {
  constexpr int PW = kWsPW;
  constexpr int WPS = D / 4;                      // packed words per step
  constexpr int SPT = 4 / WPS;                    // steps per tile
  constexpr int BPW = 32 / D;                     // blocks per word of a lane
  constexpr int kChunks = JB * DD;                // 1 KB chunks of a step's B operands
  constexpr int kStageUnits = kChunks * 64;       // [jb][f][g][r]
  constexpr int kSlotUnits = 4 * PW * 64;         // [wave][panel][lane]
  constexpr int kLut = 1 << D;
  constexpr int kWaitLds0 = (3 << 14) | (7 << 4) | 15;   // lgkmcnt(0) alone
  __shared__ uint4 stage0[kStageUnits];
  __shared__ uint4 stage1[kStageUnits];
  __shared__ uint4 stage2[kStageUnits];
  __shared__ uint4 stage3[kStageUnits];
  // Each wavefront copies and reads only its own part of the slots, and
  // reads a tile's words (at the tile's last step) before it copies the next
  // tile's (at the first step of that tile), so one buffer serves.
  __shared__ uint4 slots[kSlotUnits];
  // (the most strictly aligned LDS object, so it is placed at address 0 and a
  // lookup's address is its index times 8, one shift of the packed byte)
  __shared__ __align__(2048) uint2 lut[kLut];
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int64_t steps = SPT * (int64_t)ext_tiles;
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
      if (i < DD) {
#pragma unroll
        for (int e = 0; e < D; ++e) a = fmaf(M[i * D + e], ((p >> e) & 1) ? -1.0f : 1.0f, a);
      }
      h[i] = f32_to_bf16_bits(a);
    }
    lut[p] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  }

  // A copy is a uniform base plus the lane's 16 bytes (a 32-bit offset).
  const uint32_t lane16 = 16u * (uint32_t)lane;
  auto dma = [&](const void* src, uint4* dst) __attribute__((always_inline)) {
    __builtin_amdgcn_global_load_lds((const void*)(reinterpret_cast<const uint8_t*>(src) + lane16),
                                     (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
  };
  // The B operands of one step: kChunks copies of 1 KB spread over the four
  // wavefronts (clamped: a repeated copy writes the same bytes again). Copy
  // k of step t reads chunk ch_k (batch tile c, sub-step f) at
  // xp + ((jb * steps + t) * DD + f) * 64: a base fixed for the workgroup
  // plus t * DD KB.
  constexpr int kCopies = (kChunks + 3) / 4;
  const uint4* cbase[kCopies];
  int cdst[kCopies];
#pragma unroll
  for (int k = 0; k < kCopies; ++k) {
    const int ch = min(wave + 4 * k, kChunks - 1);
    const int c = ch / DD, f = ch % DD;
    const int64_t jb = min(jb0 + c, B16 - 1);
    cbase[k] = xp + (jb * steps * DD + f) * 64;
    cdst[k] = ch * 64;
  }
  auto copy_step = [&](int64_t t, uint4* dst) __attribute__((always_inline)) {
    const int64_t off = t * (DD * 64);
#pragma unroll
    for (int k = 0; k < kCopies; ++k) dma(cbase[k] + off, dst + cdst[k]);
  };
  // The slots of tile q of this wavefront's panels: the panel's packed bytes
  // plus q KB, or past the full tiles the panel's rebuilt tail slots.
  const uint8_t* sbase[PW];
  const uint4* tbase[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int64_t pnl = min(pbase + i, panels - 1);
    sbase[i] = packed + pnl * panel_bytes;
    tbase[i] = tail_slots + pnl * 64;
  }
  auto copy_slots = [&](int q, uint4* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const void* src = q < full_tiles ? (const void*)(sbase[i] + (int64_t)q * kTileBytes)
                                       : (const void*)tbase[i];
      dma(src, dst + (wave * PW + i) * 64);
    }
  };
  // The table entries of step sg of the tiles whose words are w: 8 per panel.
  auto lut_step = [&](const uint32_t (&w)[PW][4], int sg, uint2 (&e)[PW][8])
                      __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PW; ++i)
#pragma unroll
      for (int lam = 0; lam < 8; ++lam) {
        const uint32_t word = w[i][sg * WPS + lam / BPW];
        e[i][lam] = lut[(word >> (D * (lam % BPW))) & (kLut - 1)];
      }
  };
  auto read_words = [&](const uint4* slot, uint32_t (&w)[PW][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const uint4 v = slot[(wave * PW + i) * 64 + lane];
      w[i][0] = v.x; w[i][1] = v.y; w[i][2] = v.z; w[i][3] = v.w;
    }
  };

  f32x4 acc[PW][JB];
#pragma unroll
  for (int i = 0; i < PW; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j) acc[i][j] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

  // One step: DD sub-steps. The B operands of the next sub-step (for the
  // last one, sub-step 0 of the next step, whose stage is complete by then)
  // are read before the MFMAs of this one; the A operands of the next step
  // are packed from its table entries e between the last sub-step's MFMAs.
  // The table entries of the next step are looked up in DD parts, part f
  // right after sub-step f's B-operand reads: a wait for those reads then
  // covers at most one part's lookups issued after them (the LDS counter
  // counts only 15), not all 8 PW.
  auto mult = [&](const uint4* st, const uint4* st_next, u32x4 (&a)[PW][DD], uint4 (&bcur)[JB],
                  const uint32_t (&w)[PW][4], int sg_next, uint2 (&e)[PW][8])
                  __attribute__((always_inline)) {
    uint4 bnext[JB];
#pragma unroll
    for (int f = 0; f < DD; ++f) {
#pragma unroll
      for (int c = 0; c < JB; ++c)
        bnext[c] = f < DD - 1 ? st[(c * DD + f + 1) * 64 + lane] : st_next[(c * DD) * 64 + lane];
      // this part's table entries: entries lam of every panel with
      // lam * DD / 8 == f
#pragma unroll
      for (int i = 0; i < PW; ++i)
#pragma unroll
        for (int lam = 0; lam < 8; ++lam)
          if ((lam * DD) / 8 == f) {
            const uint32_t word = w[i][sg_next * WPS + lam / BPW];
            e[i][lam] = lut[(word >> (D * (lam % BPW))) & (kLut - 1)];
          }
      // Keep those reads here: the scheduler would otherwise sink each one
      // next to its first use.
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < PW; ++i) {
#pragma unroll
        for (int c = 0; c < JB; ++c) {
          const u32x4 bop = {bcur[c].x, bcur[c].y, bcur[c].z, bcur[c].w};
          acc[i][c] = mfma_bf16(a[i][f], bop, acc[i][c]);
        }
      }
      if (f == DD - 1) {
        u32x4 an[PW][DD];
#pragma unroll
        for (int i = 0; i < PW; ++i) pack_step<DD>(e[i], an[i]);
        // one MFMA, then up to 4 VALU instructions, and so on
#pragma unroll
        for (int k = 0; k < PW * JB; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
#pragma unroll
        for (int i = 0; i < PW; ++i)
#pragma unroll
          for (int g = 0; g < DD; ++g) a[i][g] = an[i][g];
      }
#pragma unroll
      for (int c = 0; c < JB; ++c) bcur[c] = bnext[c];
    }
  };

  // Copies are issued unconditionally (past the last step, the last step
  // again), slots before stage, so kCopies copy instructions follow those of
  // step t + 1 when step t begins: waiting until at most that many are
  // outstanding means step t + 1's copies, and everything issued before them
  // (the next tile's slots too, from the second step of a tile on), have
  // landed.
  constexpr int kWait1 = (7 << 4) | (15 << 8) | (kCopies & 15) | ((kCopies >> 4) << 14);
  constexpr int kWait2 = (7 << 4) | (15 << 8) | ((2 * kCopies) & 15) | (((2 * kCopies) >> 4) << 14);
  static_assert(2 * kCopies <= 63, "vmcnt range");
  static_assert(SPT >= 2, "the next tile's words are read in a tile's second step or later");
  copy_slots(0, slots);
  copy_step(0, stage0);
  copy_step(min((int64_t)1, last), stage1);
  copy_step(min((int64_t)2, last), stage2);
  uint4 bcur[JB];
  u32x4 a[PW][DD];
  uint32_t w[PW][4];

  // Stage of step t: t mod 4, selected at compile time (the stages are
  // separate arrays, so the compiler knows a copy into one does not alias
  // the reads of another and makes those reads wait for nothing).
  auto stage_c = [&](auto ic) __attribute__((always_inline)) -> uint4* {
    constexpr int i = decltype(ic)::value & 3;
    if constexpr (i == 0) return stage0;
    else if constexpr (i == 1) return stage1;
    else if constexpr (i == 2) return stage2;
    else return stage3;
  };
  // Step sg of tile q, whose first step uses stage `off` (for D = 8 tiles
  // alternate between stages 0-1 and 2-3).
  // On entry a holds the step's A operands; the step looks up the next
  // step's table entries (in its last step, from the next tile's words).
  auto do_step = [&](auto sgc, auto offc, int q) __attribute__((always_inline)) {
    constexpr int sg = decltype(sgc)::value;
    constexpr int su = (decltype(offc)::value + sg) & 3;
    const int64_t t = (int64_t)q * SPT + sg;
    __builtin_amdgcn_s_waitcnt(kWait1);
    // The LDS wait as a builtin, not inline assembly: the compiler then
    // knows that the reads issued before the barrier have landed and does
    // not drain the next sub-step's reads to wait for them.
    __builtin_amdgcn_s_waitcnt(kWaitLds0);
    __builtin_amdgcn_s_barrier();
    uint2 e[PW][8];
    if constexpr (sg + 1 == SPT) read_words(slots, w);   // the next tile's words
    if constexpr (sg == 0) copy_slots(min(q + 1, ext_tiles - 1), slots);
    copy_step(min(t + 3, last), stage_c(std::integral_constant<int, su + 3>{}));
    mult(stage_c(std::integral_constant<int, su>{}), stage_c(std::integral_constant<int, su + 1>{}),
         a, bcur, w, sg + 1 < SPT ? sg + 1 : 0, e);
  };
  auto tile = [&](auto offc, int q) __attribute__((always_inline)) {
    do_step(std::integral_constant<int, 0>{}, offc, q);
    do_step(std::integral_constant<int, 1>{}, offc, q);
    if constexpr (SPT > 2) {
      do_step(std::integral_constant<int, 2>{}, offc, q);
      do_step(std::integral_constant<int, 3>{}, offc, q);
    }
  };
  // Before the loop: the first tile's words, step 0's A operands and
  // sub-step 0 of its B operands (steps 1 and 2 may still be in flight);
  // the barrier also publishes the table.
  __builtin_amdgcn_s_waitcnt(kWait2);
  __builtin_amdgcn_s_waitcnt(kWaitLds0);
  __builtin_amdgcn_s_barrier();
  {
    uint2 e[PW][8];
    read_words(slots, w);
    lut_step(w, 0, e);
#pragma unroll
    for (int i = 0; i < PW; ++i) pack_step<DD>(e[i], a[i]);
  }
#pragma unroll
  for (int c = 0; c < JB; ++c) bcur[c] = stage0[(c * DD) * 64 + lane];
  int q = 0;
  for (; q + 1 < ext_tiles; q += 2) {
    tile(std::integral_constant<int, 0>{}, q);
    tile(std::integral_constant<int, SPT & 3>{}, q + 1);
  }
  if (q < ext_tiles) tile(std::integral_constant<int, 0>{}, q);

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
      if (y_bf16) {
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

template <int D, int DD, int JB>
hipError_t launch_ws_t(const uint8_t* packed, const PackedGeom& g, const uint4* xp, int64_t B,
                       const uint4* tail_slots, const float* M, const float* row_scale, void* y,
                       bool y_bf16, hipStream_t stream) {
  const int64_t B16 = (B + 15) / 16;
  const dim3 grid((unsigned)((g.panels + 4 * kWsPW - 1) / (4 * kWsPW)), (unsigned)((B16 + JB - 1) / JB));
  return launch_timed(wspace_kernel<D, DD, JB>, grid, dim3(256), 0, stream, packed, g.panels,
                      g.panel_bytes, g.full_tiles, g.ext_tiles, xp, B16, B, tail_slots, M,
                      y_bf16 ? 1 : 0, row_scale, y, g.N);
}

template <int D, int DD>
hipError_t launch_ws_jb(const uint8_t* packed, const PackedGeom& g, const uint4* xp, int64_t B,
                        const uint4* tail_slots, const float* M, const float* row_scale, void* y,
                        bool y_bf16, int jb, hipStream_t stream) {
  switch (jb) {
    case 8:
      if constexpr (DD <= 3)
        return launch_ws_t<D, DD, 8>(packed, g, xp, B, tail_slots, M, row_scale, y, y_bf16, stream);
      else
        return hipErrorInvalidValue;
    case 4: return launch_ws_t<D, DD, 4>(packed, g, xp, B, tail_slots, M, row_scale, y, y_bf16, stream);
    case 2: return launch_ws_t<D, DD, 2>(packed, g, xp, B, tail_slots, M, row_scale, y, y_bf16, stream);
    case 1: return launch_ws_t<D, DD, 1>(packed, g, xp, B, tail_slots, M, row_scale, y, y_bf16, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_ws_d(const uint8_t* packed, const PackedGeom& g, const uint4* xp, int64_t B,
                       const uint4* tail_slots, const float* M, int d, const float* row_scale,
                       void* y, bool y_bf16, int jb, hipStream_t stream) {
  switch (d) {
    case 1: return launch_ws_jb<D, 1>(packed, g, xp, B, tail_slots, M, row_scale, y, y_bf16, jb, stream);
    case 2: return launch_ws_jb<D, 2>(packed, g, xp, B, tail_slots, M, row_scale, y, y_bf16, jb, stream);
    case 3: return launch_ws_jb<D, 3>(packed, g, xp, B, tail_slots, M, row_scale, y, y_bf16, jb, stream);
    case 4: return launch_ws_jb<D, 4>(packed, g, xp, B, tail_slots, M, row_scale, y, y_bf16, jb, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool wspace_supported(int d, int D) { return (D == 4 || D == 8) && d >= 1 && d <= 4 && d <= D; }

XpGeom xp_geom(int64_t B, const PackedGeom& g, int d, int D) {
  XpGeom x;
  x.B16 = (B + 15) / 16;
  x.steps = (16 / D) * (int64_t)g.ext_tiles;
  x.bytes = (size_t)x.B16 * x.steps * d * 1024;
  x.tail_bytes = g.tail_bytes ? (size_t)g.panels * kTileBytes : 0;
  return x;
}

int plan_wspace_jb(int64_t B, const PackedGeom& g, int d) {
  const int64_t B16 = (B + 15) / 16;
  const int64_t pgroups = (g.panels + 4 * kWsPW - 1) / (4 * kWsPW);
  // 8 batch tiles per workgroup (each A operand feeds 8 MFMAs) where that
  // still gives >= 512 workgroups and the stages fit LDS (d <= 3)
  if (d <= 3 && B16 >= 8 && pgroups * ((B16 + 7) / 8) >= 512) return 8;
  return B16 >= 4 ? 4 : (B16 >= 2 ? 2 : 1);
}

hipError_t launch_xpw(const void* x, bool x_bf16, int64_t B, int64_t K, int hb, const float* c,
                      int d, int D, const PackedGeom& g, void* xp, hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
  if (!wspace_supported(d, D) || hb < 1 || hb > 1024 || (hb & (hb - 1)) || K % hb) return hipErrorInvalidValue;
  const XpGeom xg = xp_geom(B, g, d, D);
  int lhb = 0;
  while ((1 << lhb) < hb) ++lhb;
  const float norm = (lhb % 2 == 0) ? ldexpf(1.0f, -lhb / 2) : (float)(1.0 / sqrt((double)hb));
  const int64_t blk_end = (int64_t)g.ext_tiles * (kTileCols / D);
  const unsigned chunks = (unsigned)((K + 1023) / 1024);
  const int64_t groups = 2 * xg.B16;             // 8-row groups
  uint4* out = reinterpret_cast<uint4*>(xp);
  for (int64_t jr0 = 0; jr0 < groups; jr0 += 65535) {
    const dim3 grid(chunks, (unsigned)min(groups - jr0, (int64_t)65535));
#define LQ_XPW(D_, DD_)                                                                          \
    if (x_bf16)                                                                                  \
      hipLaunchKernelGGL((xpw_kernel<D_, DD_, true>), grid, dim3(256), 0, stream, x, c, B, K,   \
                         lhb, norm, xg.steps, blk_end, jr0, out);                                \
    else                                                                                         \
      hipLaunchKernelGGL((xpw_kernel<D_, DD_, false>), grid, dim3(256), 0, stream, x, c, B, K,  \
                         lhb, norm, xg.steps, blk_end, jr0, out)
    switch (D * 8 + d) {
      case 8 * 8 + 1: LQ_XPW(8, 1); break;
      case 8 * 8 + 2: LQ_XPW(8, 2); break;
      case 8 * 8 + 3: LQ_XPW(8, 3); break;
      case 8 * 8 + 4: LQ_XPW(8, 4); break;
      case 4 * 8 + 1: LQ_XPW(4, 1); break;
      case 4 * 8 + 2: LQ_XPW(4, 2); break;
      case 4 * 8 + 3: LQ_XPW(4, 3); break;
      default: LQ_XPW(4, 4); break;
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
  const int jb = plan_wspace_jb(B, g, d);
  const uint4* x = reinterpret_cast<const uint4*>(xp);
  uint4* ts = reinterpret_cast<uint4*>(tail_slots);
  if (g.tail_bytes) {
    const hipError_t e = launch_tail_slots(packed, g, ts, stream);
    if (e != hipSuccess) return e;
  }
  if (D == 8) return launch_ws_d<8>(packed, g, x, B, ts, M, d, row_scale, y, y_bf16, jb, stream);
  return launch_ws_d<4>(packed, g, x, B, ts, M, d, row_scale, y, y_bf16, jb, stream);
}

}  // namespace lq
