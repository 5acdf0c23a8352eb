// Lift: z[b][j*D + e] = sum_{i<d} M[i][e] * xt[b][j*d + i], xt = 0 past K.
// One thread per lifted value; M (d x D <= 64 x 64) is staged in LDS. The sum
// runs i = 0..d-1 with fused multiply-adds, so results are deterministic.
#include "lq_internal.h"

namespace lq {
namespace {

template <bool kBF16>
__global__ __launch_bounds__(256) void lift_kernel(const float* __restrict__ xt, int64_t K, int d,
                                                   int D, const float* __restrict__ M,
                                                   void* __restrict__ z, int64_t L) {
  __shared__ float Ms[64 * 64];
  for (int i = threadIdx.x; i < d * D; i += blockDim.x) Ms[i] = M[i];
  __syncthreads();
  const int64_t b = blockIdx.y;
  const float* xr = xt + b * K;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < L;
       j += (int64_t)gridDim.x * blockDim.x) {
    const int64_t blk = j / D;
    const int e = (int)(j - blk * D);
    const int64_t k0 = blk * d;
    float acc = 0.0f;
    for (int i = 0; i < d; ++i) {
      const int64_t k = k0 + i;
      if (k < K) acc = fmaf(Ms[i * D + e], xr[k], acc);
    }
    if (kBF16)
      reinterpret_cast<uint16_t*>(z)[b * L + j] = (uint16_t)f32_to_bf16_bits(acc);
    else
      reinterpret_cast<float*>(z)[b * L + j] = acc;
  }
}

}  // namespace

hipError_t launch_lift(const float* xt, int64_t B, int64_t K, int d, int D, const float* M,
                       void* z, bool z_bf16, hipStream_t stream) {
  const int64_t L = ((K + d - 1) / d) * D;
  int64_t bx = (L + 255) / 256;
  if (bx > 4096) bx = 4096;
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
