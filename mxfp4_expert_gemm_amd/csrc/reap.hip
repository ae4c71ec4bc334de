// REAP saliency of the routed experts (kimi-k3-mlx digest, REAP section): the score of
// expert j is the mean over calibration tokens x of g_j(x) ||e_j(x)||_2, the router
// weight the token gave the expert times the size of the expert's output.  Here e_j is
// the expert's output in the latent space (y, the rows moe_expert_ffn produces) and the
// kernel accumulates the sum; the caller divides by the number of tokens.
//
// One block per expert walks its rows in the grouped order (tokens ascending), so the
// fp64 sums are deterministic: per row, each thread adds the squares of its strided
// elements in fp64, the block adds the 256 partials in a fixed tree, and thread 0 adds
// w ||y|| to the expert's running sum.
//
// Inside the layer the sums come from the down kernels themselves: each writes, per
// routed row, the sum of y^2 over its block of latent rows (a fixed order inside the
// block), and reap_partials_kernel adds a row's partials in block order, so the result
// is deterministic and y need not be read again.
//
// Pruning is a router bias of -inf on the removed experts (the routing treats it as
// exactly -inf, and the weights are renormalised over the experts that remain);
// reap_keep_bias_kernel writes that bias for the experts of highest saliency.
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

// One block per expert: thread i takes the expert's rows i, i + 256, ... (grouped order),
// and the block adds the 256 sums in a fixed tree.
__global__ void __launch_bounds__(256) reap_partials_kernel(const double* __restrict__ sal, int32_t nch,
                                                            const float* __restrict__ w,
                                                            const int32_t* __restrict__ perm,
                                                            const int32_t* __restrict__ offsets,
                                                            double* __restrict__ saliency) {
  __shared__ double part[256];
  const int e = blockIdx.x, tid = threadIdx.x;
  const int r0 = offsets[e], r1 = offsets[e + 1];
  if (r1 <= r0) return;  // the same for the whole block
  double acc = 0.0;
  for (int r = r0 + tid; r < r1; r += 256) {
    const int slot = perm[r];
    const double* ps = sal + (int64_t)slot * nch;
    double sq = 0.0;
    for (int c = 0; c < nch; ++c) sq += ps[c];
    acc += (double)w[slot] * sqrt(sq);
  }
  part[tid] = acc;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (tid < h) part[tid] += part[tid + h];
    __syncthreads();
  }
  if (tid == 0) saliency[e] += part[0];
}

// One thread per expert (E <= 1024): its rank is the number of experts ordered before
// it (higher saliency, or equal and a lower index; NaN after every number).
__global__ void __launch_bounds__(1024) reap_keep_bias_kernel(const double* __restrict__ s, int32_t E, int32_t n_keep,
                                                              float* __restrict__ bias) {
  __shared__ double sv[1024];
  const int e = threadIdx.x;
  if (e < E) sv[e] = s[e];
  __syncthreads();
  if (e >= E) return;
  const double me = sv[e];
  const bool me_nan = me != me;
  int rank = 0;
  for (int j = 0; j < E; ++j) {
    const double o = sv[j];
    const bool o_nan = o != o;
    const bool before = o_nan ? (me_nan && j < e) : (me_nan || o > me || (o == me && j < e));
    rank += before ? 1 : 0;
  }
  bias[e] = rank < n_keep ? 0.f : -__builtin_huge_valf();
}

hipError_t launch_reap_partials(const double* sal, int32_t nch, const float* w, const int32_t* perm,
                                const int32_t* offsets, int32_t E, double* saliency, hipStream_t st) {
  if (E == 0) return hipSuccess;
  hipLaunchKernelGGL(reap_partials_kernel, dim3((unsigned)E), dim3(256), 0, st, sal, nch, w, perm, offsets, saliency);
  return hipGetLastError();
}

hipError_t launch_reap_keep_bias(const double* saliency, int32_t E, int32_t n_keep, float* bias, hipStream_t st) {
  if (E < 1 || E > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(reap_keep_bias_kernel, dim3(1), dim3(1024), 0, st, saliency, E, n_keep, bias);
  return hipGetLastError();
}

hipError_t launch_reap_saliency(const float* y, const float* w, const int32_t* perm, const int32_t* offsets,
                                int32_t E, int32_t L, double* saliency, hipStream_t st) {
  hipLaunchKernelGGL(reap_saliency_kernel, dim3((unsigned)E), dim3(256), 0, st, y, w, perm, offsets, L, saliency);
  return hipGetLastError();
}

}  // namespace moe
