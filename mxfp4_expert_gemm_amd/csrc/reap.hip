// REAP saliency of the routed experts (kimi-k3-mlx digest, REAP section): the score of
// expert j is the mean over calibration tokens x of g_j(x) ||e_j(x)||_2, the router
// weight the token gave the expert times the size of the expert's output.  Here e_j is
// the expert's output in the latent space (y, the rows moe_expert_ffn produces) and the
// kernel accumulates the sum; the caller divides by the number of tokens.
//
// One block per expert walks its rows in the grouped order (tokens ascending), so the
// fp64 sums are deterministic: per row, each thread adds the squares of its strided
// elements in fp64, the block adds the 256 partials in a fixed tree, and thread 0 adds
// w ||y|| to the expert's running sum.  Pruning itself needs no kernel: an expert
// removed from the layer is a router bias of -inf (the routing treats it as exactly
// -inf, and the weights are renormalised over the experts that remain).
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ void __launch_bounds__(256) reap_saliency_kernel(const float* __restrict__ y, const float* __restrict__ w,
                                                            const int32_t* __restrict__ perm,
                                                            const int32_t* __restrict__ offsets, int32_t L,
                                                            double* __restrict__ saliency) {
  __shared__ double part[256];
  const int e = blockIdx.x, tid = threadIdx.x;
  const int r0 = offsets[e], r1 = offsets[e + 1];
  double acc = 0.0;  // thread 0's running sum
  for (int r = r0; r < r1; ++r) {
    const int slot = perm[r];
    const float* row = y + (int64_t)slot * L;
    double sq = 0.0;
    for (int l = tid; l < L; l += 256) {
      const double v = (double)row[l];
      sq += v * v;
    }
    part[tid] = sq;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
      if (tid < h) part[tid] += part[tid + h];
      __syncthreads();
    }
    if (tid == 0) acc += (double)w[slot] * sqrt(part[0]);
    __syncthreads();
  }
  if (tid == 0 && r1 > r0) saliency[e] += acc;
}

hipError_t launch_reap_saliency(const float* y, const float* w, const int32_t* perm, const int32_t* offsets,
                                int32_t E, int32_t L, double* saliency, hipStream_t st) {
  hipLaunchKernelGGL(reap_saliency_kernel, dim3((unsigned)E), dim3(256), 0, st, y, w, perm, offsets, L, saliency);
  return hipGetLastError();
}

}  // namespace moe
