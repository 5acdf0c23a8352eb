// Whitening xt = H_hb (c .* x) per run of hb channels: a fast Walsh-Hadamard
// transform (Sylvester order, orthonormal) after the per-channel scales.
//
// The flattened B*K activations are cut into chunks of 1024 values, one chunk
// per 256-thread workgroup; hb divides both K and 1024, so every chunk holds
// whole Hadamard blocks and the butterflies of stride h < hb never leave it.
// Thread t first holds chunk elements 4t..4t+3: strides 1 and 2 are done in
// registers, strides 4..128 with cross-lane shuffles inside the 64-wide
// wavefront. One LDS transpose then gives thread t the elements t + 256j, so
// strides 256 and 512 are again in registers. Stages commute, so their order
// does not matter. fp32 arithmetic throughout.
#include "lq_internal.h"

namespace lq {
namespace {

__device__ __forceinline__ void butterfly(float& a, float& b) {
  const float s = a + b, d = a - b;
  a = s;
  b = d;
}

template <bool kBF16>
__device__ __forceinline__ float load_x(const void* x, int64_t i) {
  if (kBF16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(x)[i]);
  return reinterpret_cast<const float*>(x)[i];
}

template <bool kBF16>
__global__ __launch_bounds__(256) void hadamard_scale_kernel(const void* __restrict__ x,
                                                             const float* __restrict__ c,
                                                             float* __restrict__ xt,
                                                             int64_t total, int64_t K, int hb,
                                                             float norm) {
  __shared__ float lds[1024];
  const int t = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * 1024;

  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t gi = base + 4 * t + i;
    v[i] = (gi < total) ? load_x<kBF16>(x, gi) * c[gi % K] : 0.0f;
  }
  if (hb > 1) { butterfly(v[0], v[1]); butterfly(v[2], v[3]); }   // stride 1
  if (hb > 2) { butterfly(v[0], v[2]); butterfly(v[1], v[3]); }   // stride 2
  for (int s = 1; s < 64 && 4 * s < hb; s <<= 1) {                 // strides 4..128
    const bool upper = (t & s) != 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float o = __shfl_xor(v[i], s, 64);
      v[i] = upper ? (o - v[i]) : (v[i] + o);
    }
  }
  if (hb > 256) {                                                  // strides 256, 512
#pragma unroll
    for (int i = 0; i < 4; ++i) lds[4 * t + i] = v[i];
    __syncthreads();
    float w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = lds[t + 256 * j];
    butterfly(w[0], w[1]);
    butterfly(w[2], w[3]);
    if (hb > 512) { butterfly(w[0], w[2]); butterfly(w[1], w[3]); }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t gi = base + t + 256 * j;
      if (gi < total) xt[gi] = w[j] * norm;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t gi = base + 4 * t + i;
      if (gi < total) xt[gi] = v[i] * norm;
    }
  }
}

}  // namespace

hipError_t launch_hadamard_scale(const void* x, bool x_bf16, int64_t B, int64_t K, int hb,
                                 const float* c, float* xt, hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error of an earlier runtime call
  const int64_t total = B * K;
  const int64_t blocks = (total + 1023) / 1024;
  // 1/sqrt(hb) for hb = 2^k: exact when k is even, correctly rounded otherwise.
  int k = 0;
  while ((1 << k) < hb) ++k;
  const float norm = (k % 2 == 0) ? ldexpf(1.0f, -k / 2) : (float)(1.0 / sqrt((double)hb));
  if (x_bf16)
    hipLaunchKernelGGL(hadamard_scale_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       x, c, xt, total, K, hb, norm);
  else
    hipLaunchKernelGGL(hadamard_scale_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       x, c, xt, total, K, hb, norm);
  return hipGetLastError();
}

}  // namespace lq
