// Weighted combine of the k expert outputs of each token in the latent space:
// z[t][l] = bf16(sum_j w[t][j] * y[t*k + j][l]), accumulated in fp64 in slot order
// (the fp32 products are exact in fp64), rounded once
// (kimi-k3-mlx digest: router weights are probabilities over the kept experts;
// Stable LatentMoE combines before the single up-projection).
#include "common.h"
#include "kernels.h"

namespace moe {

// One thread per 4 consecutive latent values of a token, over the flattened [T][L/4]
// index space, so every lane has work whatever L is; y is read once, with nontemporal
// loads (prefill32k: 7.5 GB at 5.5 TB/s, against 5.25 for a grid of 256-thread blocks
// over L / 4 and the tokens, whose last block per token had half its lanes idle).
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ y, const float* __restrict__ w,
                                                      int64_t T, int32_t k, int32_t L,
                                                      uint16_t* __restrict__ z) {
  const int64_t L4 = L / 4, n = T * L4;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < n; q += (int64_t)gridDim.x * 256) {
    const int64_t t = q / L4;
    const int l = 4 * (int)(q - t * L4);
    double ax = 0.0, ay = 0.0, az = 0.0, aw = 0.0;
    for (int j = 0; j < k; ++j) {
      const double wj = (double)w[t * k + j];
      const uint4 v = load_nt16(y + (t * k + j) * L + l);
      ax += wj * (double)__uint_as_float(v.x);
      ay += wj * (double)__uint_as_float(v.y);
      az += wj * (double)__uint_as_float(v.z);
      aw += wj * (double)__uint_as_float(v.w);
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
  if (L % 4) return hipErrorInvalidValue;
  int64_t blocks = ceil_div(T * (L / 4), 256);
  if (blocks > (1 << 20)) blocks = 1 << 20;  // the rest by the grid-stride loop
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, st, y, w, T, k, L, z);
  return hipGetLastError();
}

}  // namespace moe
