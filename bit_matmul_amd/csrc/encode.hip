// Nearest-neighbour encoding of weight blocks, and one gradient step of the
// mapping matrix M on it ([paper] §3.1, Eq. (1): the inner minimisation over
// the sign vectors is the quantization step; the outer one trains M on
// Gaussian blocks).
//
// Search: every sign vector s in {+1,-1}^D is visited once, in Gray-code
// order, carrying the residual r = w - M s in fp64 (a flip of sign e moves it
// by +-2 M[:, e]: d adds and d fused multiply-adds for the squared distance
// per visit). The minimum is taken on (distance, pattern index), index bit e
// set meaning s_e = -1, so that equal distances go to the lowest index. For
// D <= 10 one lane walks all 2^D vectors of its block; beyond, a wavefront
// shares a block: lane l walks the 2^(D-6) vectors whose top six bits are l,
// and the wavefront reduces.
//
// Pseudo-inverse-initialised search (lq_encode_pinv): M = [M_a | M_f], the
// first d columns solved for, the other F = D - d enumerated. For each of the
// 2^F sign vectors s_f of M_f, visited in Gray-code order, the lane carries
// u = A (w - M_f s_f) (A = M_a^-1, computed on the host) and r_f = w - M_f s_f
// in fp64 (a flip moves them by +-2 A M_f[:, k] and +-2 M_f[:, k]); the
// solved signs are s_a = sgn(u) (+1 at 0), the candidate's residual
// r = r_f - M_a s_a (d^2 fused multiply-adds). The minimum is taken on
// (distance, index of the whole pattern). F <= 10: one lane per block;
// beyond, a wavefront per block, lane l walking the 2^(F-6) vectors whose
// top six free bits are l.
#include "lq_internal.h"

namespace lq {
namespace {

constexpr int kEncThreads = 256;

// 2 M[i][e] as doubles at [e][DM] (rows past d zero: they add exact zeros).
template <int DM>
__device__ __forceinline__ void stage_m2(double* m2, const float* __restrict__ M, int d, int D) {
  for (int j = threadIdx.x; j < D * DM; j += kEncThreads) {
    const int e = j / DM, i = j - e * DM;
    m2[j] = i < d ? 2.0 * (double)M[i * D + e] : 0.0;
  }
}

// The search over patterns p = prefix | q, q < 2^nfree, for one block.
// Returns the best (distance, index) of this lane. Pattern k of the walk is
// prefix | gray(k); step k flips bit ctz(k). Seven steps in eight flip bit
// 0, 1 or 2, whose columns are held in registers; the walk is unrolled by
// eight so those steps need no bit scan and no LDS read (the visiting order
// and the arithmetic of every step are those of the plain loop).
template <int DM>
__device__ __forceinline__ void walk(const double* m2, const double (&wv)[DM], int D,
                                     uint32_t prefix, int nfree, double& best, uint32_t& bidx) {
  // residual of the first pattern: r = w - M s, s_e = -1 where bit e is set
  double r[DM];
#pragma unroll
  for (int i = 0; i < DM; ++i) r[i] = wv[i];
  for (int e = 0; e < D; ++e) {
    const double sgn = ((prefix >> e) & 1) ? 0.5 : -0.5;   // - s_e / 2 (m2 holds 2 M)
#pragma unroll
    for (int i = 0; i < DM; ++i) r[i] = fma(sgn, m2[e * DM + i], r[i]);
  }
  double d0 = 0.0, d1 = 0.0;
#pragma unroll
  for (int i = 0; i < DM; ++i) {
    if (i & 1) d1 = fma(r[i], r[i], d1);
    else d0 = fma(r[i], r[i], d0);
  }
  best = d0 + d1;
  bidx = prefix;
  uint32_t pat = prefix;
  // One step: flip bit e (column col), update r and the distance, keep the
  // least (distance, pattern) — branch-free.
  auto step = [&](const auto& col, int e) __attribute__((always_inline)) {
    pat ^= 1u << e;
    // s_e became -1: M s lost 2 M[:, e], r gains it; became +1: r loses it
    const double sg = ((pat >> e) & 1) ? 1.0 : -1.0;
    // two partial sums: half the dependent chain
    double s0 = 0.0, s1 = 0.0;
#pragma unroll
    for (int i = 0; i < DM; ++i) {
      r[i] = fma(sg, col[i], r[i]);
      if (i & 1) s1 = fma(r[i], r[i], s1);
      else s0 = fma(r[i], r[i], s0);
    }
    const double dd = s0 + s1;
    const bool take = (dd < best) | ((dd == best) & (pat < bidx));   // no short circuit: no branch
    best = take ? dd : best;
    bidx = take ? pat : bidx;
  };
  const uint32_t count = 1u << nfree;
  if (nfree < 3) {
    for (uint32_t k = 1; k < count; ++k) {
      const int e = __builtin_ctz(k);
      step(m2 + e * DM, e);
    }
    return;
  }
  double c0[DM], c1[DM], c2[DM];
#pragma unroll
  for (int i = 0; i < DM; ++i) {
    c0[i] = m2[i];
    c1[i] = m2[DM + i];
    c2[i] = m2[2 * DM + i];
  }
  for (uint32_t k0 = 0; k0 < count; k0 += 8) {
    // steps k0 + 1 .. k0 + 7 flip bits 0 1 0 2 0 1 0
    step(c0, 0);
    step(c1, 1);
    step(c0, 0);
    step(c2, 2);
    step(c0, 0);
    step(c1, 1);
    step(c0, 0);
    // step k0 + 8 flips bit ctz(k0 + 8) >= 3 (none after the last pattern)
    const uint32_t k = k0 + 8;
    if (k < count) {
      const int e = __builtin_ctz(k);
      step(m2 + e * DM, e);
    }
  }
}

__device__ __forceinline__ void better(double& best, uint32_t& bidx, double ob, uint32_t oi) {
  if (ob < best || (ob == best && oi < bidx)) {
    best = ob;
    bidx = oi;
  }
}

// kWave: one wavefront per block (D > 10), else one lane per block.
// Writes signs[b][e] = +-1 and, if dist2 is not null, the squared distance.
template <int DM, bool kWave>
__global__ __launch_bounds__(kEncThreads) void encode_kernel(const float* __restrict__ w,
                                                             int64_t nblocks, int d, int D,
                                                             const float* __restrict__ M,
                                                             int8_t* __restrict__ signs,
                                                             float* __restrict__ dist2) {
  __shared__ double m2[32 * DM];
  stage_m2<DM>(m2, M, d, D);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t b = kWave ? (int64_t)blockIdx.x * (kEncThreads / 64) + (threadIdx.x >> 6)
                          : (int64_t)blockIdx.x * kEncThreads + threadIdx.x;
  if (b >= nblocks) return;                    // (after the only barrier)
  double wv[DM];
#pragma unroll
  for (int i = 0; i < DM; ++i) wv[i] = i < d ? (double)w[b * d + i] : 0.0;
  double best;
  uint32_t bidx;
  if (kWave) {
    const int nfree = D - 6;
    walk<DM>(m2, wv, D, (uint32_t)lane << nfree, nfree, best, bidx);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const double ob = __shfl_xor(best, o, 64);
      const uint32_t oi = (uint32_t)__shfl_xor((int)bidx, o, 64);
      better(best, bidx, ob, oi);
    }
    // lane e writes sign e
    if (lane < D) signs[b * D + lane] = ((bidx >> lane) & 1) ? (int8_t)-1 : (int8_t)1;
    if (lane == 0 && dist2 != nullptr) dist2[b] = (float)best;
  } else {
    walk<DM>(m2, wv, D, 0u, D, best, bidx);
    for (int e = 0; e < D; ++e) signs[b * D + e] = ((bidx >> e) & 1) ? (int8_t)-1 : (int8_t)1;
    if (dist2 != nullptr) dist2[b] = (float)best;
  }
}

// ------------------------------------------------- pseudo-inverse search
// LDS tables (doubles, rows past d zero): ma[e][DM] = column e of M_a,
// al[i][DM] = row i of A, b2[k][DM] = 2 (A M_f)[:, k], mf2[k][DM] = 2 M_f[:, k].
template <int DM>
struct PinvTables {
  double ma[DM * DM];
  double al[DM * DM];
  double b2[kEncodePinvMaxFree * DM];
  double mf2[kEncodePinvMaxFree * DM];
};

template <int DM>
__device__ __forceinline__ void stage_pinv(PinvTables<DM>& t, const float* __restrict__ M,
                                           const double* __restrict__ AB, int d, int D) {
  const int F = D - d;
  for (int j = threadIdx.x; j < DM * DM; j += kEncThreads) {
    const int e = j / DM, i = j - e * DM;
    t.ma[j] = (i < d && e < d) ? (double)M[i * D + e] : 0.0;
    t.al[j] = (i < d && e < d) ? AB[e * d + i] : 0.0;     // al[e][i] = A[e][i]
  }
  for (int j = threadIdx.x; j < kEncodePinvMaxFree * DM; j += kEncThreads) {
    const int k = j / DM, i = j - k * DM;
    const bool in = i < d && k < F;
    t.b2[j] = in ? 2.0 * AB[d * d + i * F + k] : 0.0;
    t.mf2[j] = in ? 2.0 * (double)M[i * D + d + k] : 0.0;
  }
}

// Zero, opaque to the compiler: a table address offset by it is a new
// address on every visit, so the d^2 M_a entries are read from LDS where they
// are used instead of being hoisted into (far too many) registers.
__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("s_mov_b32 %0, 0" : "=s"(z));
  return z;
}

// The candidate of free pattern q: s_a = sgn(u), r = r_f - M_a s_a.
template <int DM>
__device__ __forceinline__ void pinv_candidate(const PinvTables<DM>& t, const double (&u)[DM],
                                               const double (&rf)[DM], int d, uint32_t q,
                                               double& best, uint32_t& bidx, bool first) {
  const double* ma = t.ma + opaque_zero();
  double r[DM];
#pragma unroll
  for (int i = 0; i < DM; ++i) r[i] = rf[i];
  uint32_t sab = 0;
#pragma unroll
  for (int e = 0; e < DM; ++e) {
    const bool neg = u[e] < 0.0;                      // rows past d: u = 0, +1, a zero column
    sab |= (neg ? 1u : 0u) << e;
    const double ms = neg ? 1.0 : -1.0;               // -s_e
#pragma unroll
    for (int i = 0; i < DM; ++i) r[i] = fma(ms, ma[e * DM + i], r[i]);
  }
  double d0 = 0.0, d1 = 0.0;
#pragma unroll
  for (int i = 0; i < DM; ++i) {
    if (i & 1) d1 = fma(r[i], r[i], d1);
    else d0 = fma(r[i], r[i], d0);
  }
  const double dd = d0 + d1;
  const uint32_t idx = sab | (q << d);
  if (first || dd < best || (dd == best && idx < bidx)) {
    best = dd;
    bidx = idx;
  }
}

// The walk over free patterns q = prefix | g, g < 2^nfree, for one block.
template <int DM>
__device__ __forceinline__ void pinv_walk(const PinvTables<DM>& t, const double (&wv)[DM], int d,
                                          int F, uint32_t prefix, int nfree, double& best,
                                          uint32_t& bidx) {
  // u = A w - A M_f s_f and r_f = w - M_f s_f at the first pattern
  double u[DM], rf[DM];
#pragma unroll
  for (int i = 0; i < DM; ++i) {
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < DM; ++j) acc = fma(t.al[i * DM + j], wv[j], acc);
    u[i] = acc;
    rf[i] = wv[i];
  }
  for (int k = 0; k < F; ++k) {
    const double h = ((prefix >> k) & 1) ? 0.5 : -0.5;   // -s_k / 2 (the tables hold 2x)
#pragma unroll
    for (int i = 0; i < DM; ++i) {
      u[i] = fma(h, t.b2[k * DM + i], u[i]);
      rf[i] = fma(h, t.mf2[k * DM + i], rf[i]);
    }
  }
  uint32_t q = prefix;
  pinv_candidate<DM>(t, u, rf, d, q, best, bidx, true);
  const uint32_t count = 1u << nfree;
  for (uint32_t k = 1; k < count; ++k) {
    const int e = __builtin_ctz(k);
    q ^= 1u << e;
    // s_e became -1: M_f s_f lost 2 M_f[:, e], u and r_f gain it; became +1: they lose it
    const double sg = ((q >> e) & 1) ? 1.0 : -1.0;
#pragma unroll
    for (int i = 0; i < DM; ++i) {
      u[i] = fma(sg, t.b2[e * DM + i], u[i]);
      rf[i] = fma(sg, t.mf2[e * DM + i], rf[i]);
    }
    pinv_candidate<DM>(t, u, rf, d, q, best, bidx, false);
  }
}

template <int DM, bool kWave>
__global__ __launch_bounds__(kEncThreads) void encode_pinv_kernel(
    const float* __restrict__ w, int64_t nblocks, int d, int D, const float* __restrict__ M,
    const double* __restrict__ AB, int8_t* __restrict__ signs, float* __restrict__ dist2) {
  __shared__ PinvTables<DM> t;
  stage_pinv<DM>(t, M, AB, d, D);
  __syncthreads();
  const int F = D - d;
  const int lane = threadIdx.x & 63;
  const int64_t b = kWave ? (int64_t)blockIdx.x * (kEncThreads / 64) + (threadIdx.x >> 6)
                          : (int64_t)blockIdx.x * kEncThreads + threadIdx.x;
  if (b >= nblocks) return;                    // (after the only barrier)
  double wv[DM];
#pragma unroll
  for (int i = 0; i < DM; ++i) wv[i] = i < d ? (double)w[b * d + i] : 0.0;
  double best = 0.0;
  uint32_t bidx = 0;
  if (kWave) {
    const int nfree = F - 6;
    pinv_walk<DM>(t, wv, d, F, (uint32_t)lane << nfree, nfree, best, bidx);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const double ob = __shfl_xor(best, o, 64);
      const uint32_t oi = (uint32_t)__shfl_xor((int)bidx, o, 64);
      better(best, bidx, ob, oi);
    }
    if (lane < D) signs[b * D + lane] = ((bidx >> lane) & 1) ? (int8_t)-1 : (int8_t)1;
    if (lane == 0 && dist2 != nullptr) dist2[b] = (float)best;
  } else {
    pinv_walk<DM>(t, wv, d, F, 0u, F, best, bidx);
    for (int e = 0; e < D; ++e) signs[b * D + e] = ((bidx >> e) & 1) ? (int8_t)-1 : (int8_t)1;
    if (dist2 != nullptr) dist2[b] = (float)best;
  }
}

template <int DM>
hipError_t launch_encode_pinv_t(const float* w, int64_t nblocks, int d, int D, const float* M,
                                const double* AB, int8_t* signs, float* dist2, hipStream_t stream) {
  if (D - d > 10) {
    const int64_t groups = (nblocks + 3) / 4;
    hipLaunchKernelGGL((encode_pinv_kernel<DM, true>), dim3((unsigned)groups), dim3(kEncThreads), 0,
                       stream, w, nblocks, d, D, M, AB, signs, dist2);
  } else {
    const int64_t groups = (nblocks + kEncThreads - 1) / kEncThreads;
    hipLaunchKernelGGL((encode_pinv_kernel<DM, false>), dim3((unsigned)groups), dim3(kEncThreads),
                       0, stream, w, nblocks, d, D, M, AB, signs, dist2);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------ training step
// Workgroup g takes samples 256 g .. 256 g + 255. Phase 1, thread = sample:
// r = w - M s* and u = r / ||r|| (zero where r = 0) in fp64, into LDS with
// the signs. Phase 2, thread = entry (i, e) of the gradient: -sum over the
// workgroup's samples, in order, of u[i] s*[e]; thread d D sums ||r||. One
// (d D + 1)-double partial per workgroup; deterministic.
template <int DM>
__global__ __launch_bounds__(kEncThreads) void train_grad_kernel(
    const float* __restrict__ w, const int8_t* __restrict__ signs, int64_t n, int d, int D,
    const float* __restrict__ M, double* __restrict__ partial) {
  __shared__ double us[kEncThreads * DM];
  __shared__ double norms[kEncThreads];
  __shared__ int8_t ss[kEncThreads * 32];
  const int t = threadIdx.x;
  const int64_t b = (int64_t)blockIdx.x * kEncThreads + t;
  if (b < n) {
    double r[DM];
    double nrm = 0.0;
#pragma unroll
    for (int i = 0; i < DM; ++i) {
      double v = 0.0;
      if (i < d) {
        v = (double)w[b * d + i];
        for (int e = 0; e < D; ++e) v -= (double)M[i * D + e] * (double)signs[b * D + e];
      }
      r[i] = v;
      nrm = fma(v, v, nrm);
    }
    nrm = sqrt(nrm);
    norms[t] = nrm;
#pragma unroll
    for (int i = 0; i < DM; ++i) us[t * DM + i] = nrm > 0.0 ? r[i] / nrm : 0.0;
    for (int e = 0; e < D; ++e) ss[t * 32 + e] = signs[b * D + e];
  } else {
    norms[t] = 0.0;
#pragma unroll
    for (int i = 0; i < DM; ++i) us[t * DM + i] = 0.0;
    for (int e = 0; e < D; ++e) ss[t * 32 + e] = 0;
  }
  __syncthreads();
  const int width = d * D + 1;
  for (int j = t; j < width; j += kEncThreads) {
    double acc = 0.0;
    if (j < d * D) {
      const int i = j / D, e = j - i * D;
      for (int k = 0; k < kEncThreads; ++k) acc -= us[k * DM + i] * (double)ss[k * 32 + e];
    } else {
      for (int k = 0; k < kEncThreads; ++k) acc += norms[k];
    }
    partial[(int64_t)blockIdx.x * width + j] = acc;
  }
}

// One workgroup: the partials in workgroup order, the mean, the update
// M <- M - lr * grad (fp64, stored as fp32), the loss (the mean of ||r|| at
// the old M).
__global__ __launch_bounds__(kEncThreads) void train_update_kernel(const double* __restrict__ partial,
                                                                   int groups, int64_t n, int d,
                                                                   int D, float lr,
                                                                   float* __restrict__ M,
                                                                   float* __restrict__ loss) {
  const int width = d * D + 1;
  for (int j = threadIdx.x; j < width; j += kEncThreads) {
    double acc = 0.0;
    for (int g = 0; g < groups; ++g) acc += partial[(int64_t)g * width + j];
    acc /= (double)n;
    if (j < d * D) M[j] = (float)((double)M[j] - (double)lr * acc);
    else if (loss != nullptr) *loss = (float)acc;
  }
}

template <int DM>
hipError_t launch_encode_t(const float* w, int64_t nblocks, int d, int D, const float* M,
                           int8_t* signs, float* dist2, hipStream_t stream) {
  if (D > 10) {
    const int64_t groups = (nblocks + 3) / 4;
    hipLaunchKernelGGL((encode_kernel<DM, true>), dim3((unsigned)groups), dim3(kEncThreads), 0,
                       stream, w, nblocks, d, D, M, signs, dist2);
  } else {
    const int64_t groups = (nblocks + kEncThreads - 1) / kEncThreads;
    hipLaunchKernelGGL((encode_kernel<DM, false>), dim3((unsigned)groups), dim3(kEncThreads), 0,
                       stream, w, nblocks, d, D, M, signs, dist2);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_encode(const float* w, int64_t nblocks, int d, int D, const float* M,
                         int8_t* signs, float* dist2, hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
  if (d < 1 || d > D || D > kEncodeMaxD || d > kEncodeMaxSmallD) return hipErrorInvalidValue;
  if (nblocks == 0) return hipSuccess;
  // d in registers, padded with zeros to the next width instantiated (the
  // pages' configurations, d = 2, 3, 10 and 16, run unpadded)
  if (d <= 2) return launch_encode_t<2>(w, nblocks, d, D, M, signs, dist2, stream);
  if (d <= 3) return launch_encode_t<3>(w, nblocks, d, D, M, signs, dist2, stream);
  if (d <= 4) return launch_encode_t<4>(w, nblocks, d, D, M, signs, dist2, stream);
  if (d <= 8) return launch_encode_t<8>(w, nblocks, d, D, M, signs, dist2, stream);
  if (d <= 10) return launch_encode_t<10>(w, nblocks, d, D, M, signs, dist2, stream);
  if (d <= 12) return launch_encode_t<12>(w, nblocks, d, D, M, signs, dist2, stream);
  return launch_encode_t<16>(w, nblocks, d, D, M, signs, dist2, stream);
}

hipError_t launch_encode_pinv(const float* w, int64_t nblocks, int d, int D, const float* M,
                              const double* AB, int8_t* signs, float* dist2, hipStream_t stream) {
  (void)hipGetLastError();
  if (d < 1 || d > D || D > kEncodePinvMaxD || D - d > kEncodePinvMaxFree || d > kEncodeMaxSmallD)
    return hipErrorInvalidValue;
  if (nblocks == 0) return hipSuccess;
  if (d <= 2) return launch_encode_pinv_t<2>(w, nblocks, d, D, M, AB, signs, dist2, stream);
  if (d <= 3) return launch_encode_pinv_t<3>(w, nblocks, d, D, M, AB, signs, dist2, stream);
  if (d <= 4) return launch_encode_pinv_t<4>(w, nblocks, d, D, M, AB, signs, dist2, stream);
  if (d <= 8) return launch_encode_pinv_t<8>(w, nblocks, d, D, M, AB, signs, dist2, stream);
  if (d <= 10) return launch_encode_pinv_t<10>(w, nblocks, d, D, M, AB, signs, dist2, stream);
  if (d <= 12) return launch_encode_pinv_t<12>(w, nblocks, d, D, M, AB, signs, dist2, stream);
  return launch_encode_pinv_t<16>(w, nblocks, d, D, M, AB, signs, dist2, stream);
}

int train_groups(int64_t n) { return (int)((n + kEncThreads - 1) / kEncThreads); }

size_t train_workspace_bytes(int64_t n, int d, int D) {
  // signs (n D bytes, 16-byte aligned), then the partials
  const size_t sb = ((size_t)n * D + 15) / 16 * 16;
  return sb + (size_t)train_groups(n) * (d * D + 1) * sizeof(double);
}

hipError_t launch_train_step(float* M, const float* w, int64_t n, int d, int D, float lr,
                             float* loss, void* ws, hipStream_t stream) {
  (void)hipGetLastError();
  if (d < 1 || d > D || D > kTrainMaxD || d > kEncodeMaxSmallD) return hipErrorInvalidValue;
  int8_t* signs = reinterpret_cast<int8_t*>(ws);
  double* partial = reinterpret_cast<double*>(reinterpret_cast<char*>(ws) +
                                              ((size_t)n * D + 15) / 16 * 16);
  hipError_t e = launch_encode(w, n, d, D, M, signs, nullptr, stream);
  if (e != hipSuccess) return e;
  const int groups = train_groups(n);
#define LQ_TRAIN(DM_)                                                                             \
  hipLaunchKernelGGL(train_grad_kernel<DM_>, dim3((unsigned)groups), dim3(kEncThreads), 0, stream, \
                     w, signs, n, d, D, M, partial)
  if (d <= 4) LQ_TRAIN(4);
  else if (d <= 8) LQ_TRAIN(8);
  else if (d <= 12) LQ_TRAIN(12);
  else LQ_TRAIN(16);
#undef LQ_TRAIN
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(train_update_kernel, dim3(1), dim3(kEncThreads), 0, stream, partial, groups,
                     n, d, D, lr, M, loss);
  return hipGetLastError();
}

}  // namespace lq
