// Lift: z[b][j*D + e] = sum_{i<d} M[i][e] * xt[b][j*d + i], xt = 0 past K.
// One thread per lifted value; M (d x D <= 64 x 64) and the needed xt values
// are staged in LDS. The sum runs i = 0..d-1 with fused multiply-adds, so
// results are deterministic.
#include "lq_internal.h"

namespace lq {
namespace {

// Workgroup = 256 consecutive lifted columns of one batch row. Their d-blocks
// use at most (255/D + 2) * d <= 383 original columns, loaded into LDS with
// one coalesced round trip before the multiply-adds.
template <bool kBF16>
__global__ __launch_bounds__(256) void lift_kernel(const float* __restrict__ xt, int64_t K, int d,
                                                   int D, const float* __restrict__ M,
                                                   void* __restrict__ z, int64_t L) {
  __shared__ float Ms[64 * 64];
  __shared__ float xs[384];
  const int64_t b = blockIdx.y;
  const int64_t j0 = (int64_t)blockIdx.x * 256;
  const int64_t k_lo = (j0 / D) * d;
  const int64_t j_last = (j0 + 255 < L) ? j0 + 255 : L - 1;
  int64_t k_hi = (j_last / D + 1) * d;
  if (k_hi > K) k_hi = K;
  const int span = k_hi > k_lo ? (int)(k_hi - k_lo) : 0;
  for (int i = threadIdx.x; i < d * D; i += blockDim.x) Ms[i] = M[i];
  for (int i = threadIdx.x; i < span; i += blockDim.x) xs[i] = xt[b * K + k_lo + i];
  __syncthreads();
  const int64_t j = j0 + threadIdx.x;
  if (j >= L) return;
  const int64_t blk = j / D;
  const int e = (int)(j - blk * D);
  const int64_t kb = blk * d;
  float acc = 0.0f;
  for (int i = 0; i < d; ++i) {
    const int64_t k = kb + i;
    if (k < K) acc = fmaf(Ms[i * D + e], xs[k - k_lo], acc);
  }
  if (kBF16)
    reinterpret_cast<uint16_t*>(z)[b * L + j] = (uint16_t)f32_to_bf16_bits(acc);
  else
    reinterpret_cast<float*>(z)[b * L + j] = acc;
}

}  // namespace

hipError_t launch_lift(const float* xt, int64_t B, int64_t K, int d, int D, const float* M,
                       void* z, bool z_bf16, hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
  const int64_t L = ((K + d - 1) / d) * D;
  const int64_t bx = (L + 255) / 256;
  // Batch rows map to grid.y (at most 65535 per launch).
  for (int64_t b0 = 0; b0 < B; b0 += 65535) {
    const int64_t nb = (B - b0 < 65535) ? (B - b0) : 65535;
    const float* xs = xt + b0 * K;
    void* zs = z_bf16 ? (void*)(reinterpret_cast<uint16_t*>(z) + b0 * L)
                      : (void*)(reinterpret_cast<float*>(z) + b0 * L);
    if (z_bf16)
      hipLaunchKernelGGL(lift_kernel<true>, dim3((unsigned)bx, (unsigned)nb), dim3(256), 0, stream,
                         xs, K, d, D, M, zs, L);
    else
      hipLaunchKernelGGL(lift_kernel<false>, dim3((unsigned)bx, (unsigned)nb), dim3(256), 0, stream,
                         xs, K, d, D, M, zs, L);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lq
