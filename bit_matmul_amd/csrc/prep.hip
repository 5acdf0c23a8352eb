// Activation preparation for the small-batch sign products (B <= 16), fused
// into one launch per call: whitening xt = H_hb (c .* x), the lift
// z[j*D + e] = sum_i M[i][e] xt[j*d + i], and the operand format the sign
// product reads.
//
// One workgroup per (512-column lifted tile q, batch row b). The tile's
// lifted columns need the original columns [k_lo, k_hi) of its d-blocks;
// the workgroup loads the whole Hadamard blocks covering them into LDS,
// transforms them in place (at most 2048 values: a tile spans at most 640
// original columns), lifts, and writes either
//   - fp32 z (the VALU product's input), or
//   - the FP8 operand of the FP4 x FP8 matrix-core product: z is split into
//     NT fp8 (e4m3) terms, each 16x finer than the previous, after scaling the
//     tile by a power of two so that the largest |4 z| fits fp8's range. The
//     bytes are laid out exactly as the product's B operand (see sign_fp4.hip)
//     and pre-multiplied by the factor of the sign-bit plane they meet
//     (-4, -2, -1 or +1). Per tile and batch row it also stores the inverse
//     scale and the sum of z over the columns of planes 0..2.
// Workgroup (0, 0) also clears the split-K tickets of the product that
// follows on the same stream.
#include "lq_internal.h"
#include "lq_fp8.h"

namespace lq {
namespace {

// A tile's lifted columns come from at most 511/D + 2 d-blocks, i.e. at most
// 511 + 2D <= 639 original columns, which lie in at most 2 blocks of 1024,
// 3 of 512, 4 of 256, ...: never more than 2048 values.
constexpr int kSpanMax = 2048;

__device__ __forceinline__ float block_reduce_sum(float v, float* red) {
  // Fixed-order reduction: within waves by xor shuffles, then the 4 waves.
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  const float s = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return s;
}

__device__ __forceinline__ float block_reduce_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  const float s = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return s;
}

// kMode 0: write fp32 z. kMode 1: write the FP8 operand (NT terms).
// kXKind 0: x fp32, 1: x bf16, 2: input is already-lifted z in fp32,
// 3: already-lifted z in bf16 (whitening and lift skipped).
// Index arithmetic is 32-bit (K, L < 2^31 is checked on the host).
template <int kMode, int kXKind>
__global__ __launch_bounds__(256) void prep_kernel(
    const void* __restrict__ x, int B, int K, int d, int D, int hb, float norm,
    const float* __restrict__ c, const float* __restrict__ M, int L,
    float* __restrict__ zf32,                      // kMode 0: B x L
    uint4* __restrict__ zop, float* __restrict__ invscale, float* __restrict__ tpart,
    int nt, int rp, int cs_count, int ncv, unsigned* __restrict__ tickets, int n_tickets) {
  __shared__ float xs[kSpanMax];
  __shared__ float zt[kTileCols];
  __shared__ float Ms[64 * 64];
  __shared__ float red[4];
  const int q = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;

  if (q == 0 && b == 0)
    for (int i = tid; i < n_tickets; i += blockDim.x) tickets[i] = 0u;

  const int c_lo = q * kTileCols;
  const int width = min(kTileCols, L - c_lo);

  if (kXKind <= 1) {
    // Original columns [k_lo, k_hi) feed this tile's d-blocks; load the
    // whole Hadamard blocks that cover them.
    const int j_lo = c_lo / D, j_hi = (c_lo + width - 1) / D + 1;
    const int k_lo = j_lo * d;
    const int k_hi = min(j_hi * d, K);
    const int h_lo = k_lo < K ? (k_lo / hb) * hb : 0;
    const int span = k_lo < K ? ((k_hi - 1) / hb + 1) * hb - h_lo : 0;
    const int64_t xrow = (int64_t)b * K;
    // Every global load of the thread first (x, c and M), then the LDS stores.
    float xv[kSpanMax / 256], cv[kSpanMax / 256], mv[16];
#pragma unroll
    for (int j = 0; j < kSpanMax / 256; ++j) {
      const int i = tid + 256 * j;
      const int k = h_lo + (i < span ? i : 0);
      if (kXKind == 1) xv[j] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(x)[xrow + k]);
      else xv[j] = reinterpret_cast<const float*>(x)[xrow + k];
      cv[j] = c[k];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int i = tid + 256 * j;
      mv[j] = M[i < d * D ? i : 0];
    }
    // Unconditional stores (entries past span and d*D are never read).
#pragma unroll
    for (int j = 0; j < kSpanMax / 256; ++j) xs[tid + 256 * j] = xv[j] * cv[j];
#pragma unroll
    for (int j = 0; j < 16; ++j) Ms[tid + 256 * j] = mv[j] * norm;   // fold 1/sqrt(hb) into M
    __syncthreads();
    // In-place fast Walsh-Hadamard transform of each hb-block of the span.
    for (int h = 1; h < hb; h <<= 1) {
      for (int idx = tid; idx < span / 2; idx += 256) {
        const int i = (idx / h) * 2 * h + (idx % h);
        const float a0 = xs[i], a1 = xs[i + h];
        xs[i] = a0 + a1;
        xs[i + h] = a0 - a1;
      }
      __syncthreads();
    }
    // Lift the tile: 2 columns per thread, d multiply-adds each.
#pragma unroll
    for (int jr = 0; jr < kTileCols / 256; ++jr) {
      const int jj = tid + 256 * jr;
      float acc = 0.0f;
      if (jj < width) {
        const int col = c_lo + jj;
        const int blk = col / D;
        const int e = col - blk * D;
        const int kb = blk * d;
        for (int i = 0; i < d; ++i)
          if (kb + i < K) acc = fmaf(Ms[i * D + e], xs[kb + i - h_lo], acc);
      }
      zt[jj] = acc;
    }
  } else {
    const int64_t zrow = (int64_t)b * L + c_lo;
    float v[kTileCols / 256];
#pragma unroll
    for (int jr = 0; jr < kTileCols / 256; ++jr) {
      const int jj = tid + 256 * jr;
      const int jc = jj < width ? jj : 0;
      float t;
      if (kXKind == 3) t = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(x)[zrow + jc]);
      else t = reinterpret_cast<const float*>(x)[zrow + jc];
      v[jr] = jj < width ? t : 0.0f;
    }
#pragma unroll
    for (int jr = 0; jr < kTileCols / 256; ++jr) zt[tid + 256 * jr] = v[jr];
  }
  __syncthreads();

  if (kMode == 0) {
    const int64_t zrow = (int64_t)b * L + c_lo;
#pragma unroll
    for (int jr = 0; jr < kTileCols / 256; ++jr) {
      const int jj = tid + 256 * jr;
      if (jj < width) zf32[zrow + jj] = zt[jj];
    }
    return;
  }

  // ---- FP8 operand (kMode 1)
  float amax = 0.0f, tp = 0.0f;
#pragma unroll
  for (int jr = 0; jr < kTileCols / 256; ++jr) {
    const int jj = tid + 256 * jr;
    const float v = zt[jj];
    amax = fmaxf(amax, fabsf(v));
    if ((jj & 3) != 3) tp += v;
  }
  amax = block_reduce_max(amax, red);
  tp = block_reduce_sum(tp, red);
  // Scale 2^e with 32 <= amax * 2^e < 64, so |4 z| * 2^e < 256 <= 448.
  int e = 0;
  if (amax > 0.0f) {
    e = 5 - ilogbf(amax);
    e = e > 100 ? 100 : (e < -100 ? -100 : e);
  }
  const float s = ldexpf(1.0f, e);
  if (tid == 0) {
    invscale[q * B + b] = ldexpf(1.0f, -e);
    tpart[q * B + b] = tp;
  }
  // This (tile, batch row) owns MFMA columns cidx = (b % rp) * nt + t of
  // column set b / rp. Work item = one dword (4 bytes) of one 16-byte
  // operand slice: (t, u, h, gb, dw).
  const int cset = b / rp;
  const int cbase = (b % rp) * nt;
  uint32_t* zop32 = reinterpret_cast<uint32_t*>(zop);
  for (int item = tid; item < 128 * nt; item += 256) {
    const int t = item >> 7, rest = item & 127;
    const int u = rest >> 5, h = (rest >> 4) & 1, gb = (rest >> 2) & 3, dw = rest & 3;
    uint32_t word = 0u;
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      // Reduction index k of byte (h*16 + e16) of lane group gb; the sign
      // operand holds k = 32*gA + n at nibble n = 8*plane + i, which is
      // packed column 128u + 32*gA + 4*i + plane of the word.
      const int e16 = 4 * dw + e4;
      const int k = 64 * h + 16 * gb + e16;
      const int gA = k >> 5, n = k & 31;
      const int plane = n >> 3, i = n & 7;
      const float f = (plane == 3) ? 1.0f : (plane == 2 ? -1.0f : (plane == 1 ? -2.0f : -4.0f));
      const float v = zt[128 * u + 32 * gA + 4 * i + plane] * s * f;
      word |= fp8_term(v, t) << (8 * e4);
    }
    const int slot = (((q * 4 + u) * cs_count + cset) * 2 + h) * 4 + gb;
    zop32[(slot * ncv + cbase + t) * 4 + dw] = word;
  }
}

template <int kMode, int kXKind>
hipError_t launch_prep_t(const void* x, int64_t B, int64_t K, int d, int D, int hb, const float* c,
                         const float* M, int64_t L, float* zf32, const OperandPlan& op,
                         unsigned* tickets, int n_tickets, hipStream_t stream) {
  int k = 0;
  while ((1 << k) < hb) ++k;
  const float norm = (k % 2 == 0) ? ldexpf(1.0f, -k / 2) : (float)(1.0 / sqrt((double)hb));
  const int ext = (int)((L + kTileCols - 1) / kTileCols);
  hipLaunchKernelGGL((prep_kernel<kMode, kXKind>), dim3((unsigned)ext, (unsigned)B), dim3(256), 0,
                     stream, x, (int)B, (int)K, d, D, hb, norm, c, M, (int)L, zf32, op.zop,
                     op.invscale, op.tpart, op.nt, op.rp, op.cs, op.ncv, tickets, n_tickets);
  return hipGetLastError();
}

}  // namespace

OperandShape operand_shape(int64_t B, bool z_bf16) {
  OperandShape s;
  if (!z_bf16) { s.nt = 4; s.rp = 4; }
  else if (B <= 10) { s.nt = 3; s.rp = 5; }
  else { s.nt = 2; s.rp = 8; }
  s.cs = (int)((B + s.rp - 1) / s.rp);
  s.ncv = (s.cs == 1) ? (int)B * s.nt : s.rp * s.nt;
  return s;
}

size_t operand_bytes(int64_t B, int64_t L, const OperandShape& s) {
  const int64_t ext = (L + kTileCols - 1) / kTileCols;
  return (size_t)ext * 4 * s.cs * 2 * 4 * s.ncv * 16;
}

hipError_t launch_prep(const void* x, int xkind, int64_t B, int64_t K, int d, int D, int hb,
                       const float* c, const float* M, int64_t L, float* zf32,
                       const OperandPlan* op, unsigned* tickets, int n_tickets,
                       hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
  OperandPlan none{};
  const OperandPlan& o = op ? *op : none;
  if (op == nullptr) {
    switch (xkind) {
      case 0: return launch_prep_t<0, 0>(x, B, K, d, D, hb, c, M, L, zf32, o, tickets, n_tickets, stream);
      case 1: return launch_prep_t<0, 1>(x, B, K, d, D, hb, c, M, L, zf32, o, tickets, n_tickets, stream);
      case 2: return launch_prep_t<0, 2>(x, B, K, d, D, hb, c, M, L, zf32, o, tickets, n_tickets, stream);
      default: return launch_prep_t<0, 3>(x, B, K, d, D, hb, c, M, L, zf32, o, tickets, n_tickets, stream);
    }
  }
  switch (xkind) {
    case 0: return launch_prep_t<1, 0>(x, B, K, d, D, hb, c, M, L, zf32, o, tickets, n_tickets, stream);
    case 1: return launch_prep_t<1, 1>(x, B, K, d, D, hb, c, M, L, zf32, o, tickets, n_tickets, stream);
    case 2: return launch_prep_t<1, 2>(x, B, K, d, D, hb, c, M, L, zf32, o, tickets, n_tickets, stream);
    default: return launch_prep_t<1, 3>(x, B, K, d, D, hb, c, M, L, zf32, o, tickets, n_tickets, stream);
  }
}

}  // namespace lq
