// Experts held outside HBM: the layer's expert records stay in host memory (pinned,
// readable by the device over the host link) and only the experts a batch routes to
// are copied into HBM slots before the expert kernels run.
//
// The in-c post (its section on how the memory requirement shrinks, and the one on
// streaming the trunk) keeps only the routed experts of each layer resident and reads
// the others when a token needs them; with 16 of 896 experts active per layer and
// token, a decode step needs 16 records of 17,547,264 bytes per layer.  Here the copy
// is a kernel that takes the active-expert list the grouping wrote on the device, so
// no host round trip sits between routing and the expert kernels, and the grouping is
// renumbered to slot indices so the unchanged expert kernels read the slots.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int64_t GATHER_CHUNK = 256 * 1024;  // bytes of one record copied by one block
constexpr int GATHER_UNROLL = 8;              // 16-byte loads in flight per thread

// Block (c, j): bytes [c GATHER_CHUNK, (c+1) GATHER_CHUNK) of the record of active expert
// j (tiles[j].x) into slot j.  Slots past the active count are left alone.
__global__ void __launch_bounds__(256) gather_experts_kernel(const uint8_t* __restrict__ src, int64_t eb,
                                                             const int4* __restrict__ tiles,
                                                             const int32_t* __restrict__ n_active,
                                                             uint8_t* __restrict__ dst) {
  const int j = blockIdx.y;
  if (j >= *n_active) return;
  const int64_t e = tiles[j].x;
  const int64_t u0 = (int64_t)blockIdx.x * (GATHER_CHUNK / 16);
  const int64_t u1 = u0 + GATHER_CHUNK / 16 < eb / 16 ? u0 + GATHER_CHUNK / 16 : eb / 16;
  const uint4* s = reinterpret_cast<const uint4*>(src + e * eb);
  uint4* d = reinterpret_cast<uint4*>(dst + (int64_t)j * eb);
  for (int64_t u = u0 + threadIdx.x; u < u1; u += 256 * GATHER_UNROLL) {
    uint4 v[GATHER_UNROLL];
#pragma unroll
    for (int i = 0; i < GATHER_UNROLL; ++i)
      if (u + 256 * i < u1) v[i] = s[u + 256 * i];
#pragma unroll
    for (int i = 0; i < GATHER_UNROLL; ++i)
      if (u + 256 * i < u1) d[u + 256 * i] = v[i];
  }
}

hipError_t launch_gather_experts(const uint8_t* src, int64_t expert_bytes, const int4* tiles, const int32_t* n_active,
                                 int32_t max_slots, uint8_t* dst, hipStream_t st) {
  if (max_slots <= 0) return hipSuccess;
  if (expert_bytes % 16 || max_slots > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)ceil_div(expert_bytes, GATHER_CHUNK), (unsigned)max_slots);
  hipLaunchKernelGGL(gather_experts_kernel, grid, dim3(256), 0, st, src, expert_bytes, tiles, n_active, dst);
  return hipGetLastError();
}

// The grouping renumbered to slots: active expert j (ascending ids) becomes expert j.
// tiles_s[j] = {j, offset, rows, first row}; counts_s / offsets_s over max_slots
// experts (slots past the active count hold no rows); idx_s[r] = slot of idx[r].
constexpr int REMAP_THREADS = 1024;
constexpr int REMAP_MAX_SLOTS = 1024;

__global__ void __launch_bounds__(REMAP_THREADS) remap_slots_kernel(const int4* __restrict__ tiles,
                                                                    const int32_t* __restrict__ n_active,
                                                                    int32_t max_slots,
                                                                    const int32_t* __restrict__ counts,
                                                                    const int32_t* __restrict__ offsets,
                                                                    const int32_t* __restrict__ idx, int64_t rows,
                                                                    int4* __restrict__ tiles_s,
                                                                    int32_t* __restrict__ counts_s,
                                                                    int32_t* __restrict__ offsets_s,
                                                                    int32_t* __restrict__ idx_s) {
  __shared__ int ids[REMAP_MAX_SLOTS];
  const int na = *n_active;
  for (int j = threadIdx.x; j < max_slots; j += blockDim.x) {
    const int4 t = tiles[j];
    if (j < na) {
      ids[j] = t.x;
      tiles_s[j] = make_int4(j, t.y, t.z, t.w);
      counts_s[j] = counts[t.x];
      offsets_s[j] = offsets[t.x];
    } else {
      tiles_s[j] = t;
      counts_s[j] = 0;
      offsets_s[j] = (int32_t)rows;
    }
  }
  if (threadIdx.x == 0) offsets_s[max_slots] = (int32_t)rows;
  __syncthreads();
  for (int64_t r = threadIdx.x; r < rows; r += blockDim.x) {
    const int e = idx[r];
    int lo = 0, hi = na;  // ids[0..na) ascending; e is among them
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (ids[mid] <= e) lo = mid;
      else hi = mid;
    }
    idx_s[r] = lo;
  }
}

hipError_t launch_remap_to_slots(const int4* tiles, const int32_t* n_active, int32_t max_slots, const int32_t* counts,
                                 const int32_t* offsets, const int32_t* idx, int64_t rows, int4* tiles_s,
                                 int32_t* counts_s, int32_t* offsets_s, int32_t* idx_s, hipStream_t st) {
  if (max_slots > REMAP_MAX_SLOTS || rows > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(remap_slots_kernel, dim3(1), dim3(REMAP_THREADS), 0, st, tiles, n_active, max_slots, counts,
                     offsets, idx, rows, tiles_s, counts_s, offsets_s, idx_s);
  return hipGetLastError();
}

}  // namespace moe
