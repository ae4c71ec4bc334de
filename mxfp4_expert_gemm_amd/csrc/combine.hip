// Weighted combine of the k expert outputs of each token in the latent space:
// z[t][l] = bf16(sum_j w[t][j] * y[t*k + j][l]), fp32 accumulation in slot order
// (kimi-k3-mlx digest: router weights are probabilities over the kept experts;
// Stable LatentMoE combines before the single up-projection).
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ y, const float* __restrict__ w,
                                                      int64_t T, int32_t k, int32_t L,
                                                      uint16_t* __restrict__ z) {
  const int64_t t = blockIdx.y;
  const int l = 4 * (blockIdx.x * blockDim.x + threadIdx.x);
  if (t >= T || l >= L) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const float wj = w[t * k + j];
    const float4 v = *reinterpret_cast<const float4*>(y + (t * k + j) * L + l);
    acc.x = fmaf(wj, v.x, acc.x);
    acc.y = fmaf(wj, v.y, acc.y);
    acc.z = fmaf(wj, v.z, acc.z);
    acc.w = fmaf(wj, v.w, acc.w);
  }
  uint2 o;
  o.x = (uint32_t)f32_to_bf16(acc.x) | ((uint32_t)f32_to_bf16(acc.y) << 16);
  o.y = (uint32_t)f32_to_bf16(acc.z) | ((uint32_t)f32_to_bf16(acc.w) << 16);
  *reinterpret_cast<uint2*>(z + t * L + l) = o;
}

hipError_t launch_combine(const float* y, const float* w, int64_t T, int32_t k, int32_t L, uint16_t* z,
                          hipStream_t st) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)ceil_div(L / 4, 256), (unsigned)T);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, st, y, w, T, k, L, z);
  return hipGetLastError();
}

}  // namespace moe
