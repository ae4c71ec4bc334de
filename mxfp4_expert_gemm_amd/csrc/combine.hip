// Weighted combine of the k expert outputs of each token in the latent space:
// z[t][l] = bf16(sum_j w[t][j] * y[t*k + j][l]), accumulated in fp64 in slot order
// (the fp32 products are exact in fp64), rounded once
// (kimi-k3-mlx digest: router weights are probabilities over the kept experts;
// Stable LatentMoE combines before the single up-projection).
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ y, const float* __restrict__ w,
                                                      int64_t T, int32_t k, int32_t L,
                                                      uint16_t* __restrict__ z) {
  const int l = 4 * (blockIdx.x * blockDim.x + threadIdx.x);
  if (l >= L) return;
  // tokens blockIdx.y, blockIdx.y + gridDim.y, ... (the grid's second dimension is capped)
  for (int64_t t = blockIdx.y; t < T; t += gridDim.y) {
    double ax = 0.0, ay = 0.0, az = 0.0, aw = 0.0;
    for (int j = 0; j < k; ++j) {
      const double wj = (double)w[t * k + j];
      const float4 v = *reinterpret_cast<const float4*>(y + (t * k + j) * L + l);
      ax += wj * (double)v.x;
      ay += wj * (double)v.y;
      az += wj * (double)v.z;
      aw += wj * (double)v.w;
    }
    uint2 o;
    o.x = (uint32_t)f64_to_bf16(ax) | ((uint32_t)f64_to_bf16(ay) << 16);
    o.y = (uint32_t)f64_to_bf16(az) | ((uint32_t)f64_to_bf16(aw) << 16);
    *reinterpret_cast<uint2*>(z + t * L + l) = o;
  }
}

hipError_t launch_combine(const float* y, const float* w, int64_t T, int32_t k, int32_t L, uint16_t* z,
                          hipStream_t st) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)ceil_div(L / 4, 256), (unsigned)(T < 65535 ? T : 65535));
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, st, y, w, T, k, L, z);
  return hipGetLastError();
}

}  // namespace moe
