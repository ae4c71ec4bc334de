// Grouping of routed (token, slot) rows by expert: counts, offsets, a stable
// permutation sorted by (expert, token) and the list of active experts.
//
// Rows are cut into chunks of PERM_CHUNK.  Per chunk an LDS histogram counts the
// rows of each expert (integer atomics, so the counts do not depend on order); one
// block then forms, for every expert, the running count over chunks and the
// exclusive prefix over experts; finally each chunk sorts its (expert, row) keys
// with a bitonic network in LDS and writes each row at its expert's chunk base plus
// its rank within the chunk.  Every step is deterministic.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int PERM_THREADS = 1024;
constexpr uint32_t PAD_KEY = 0xFFFFFFFFu;

// workspace: chunk counts [nchunks][E], then the tile slot of each expert [E]
static size_t cc_bytes(int64_t rows, int32_t E) {
  return align_up((size_t)ceil_div(rows, PERM_CHUNK) * (size_t)E * sizeof(int32_t), 256);
}
size_t permute_ws_bytes(int64_t rows, int32_t E) {
  return cc_bytes(rows, E) + align_up((size_t)E * sizeof(int32_t), 256);
}

// exclusive scan of n ints in LDS, in place; returns the total.  All threads call it.
__device__ int block_exclusive_scan(int* data, int n, int* partial /* PERM_THREADS ints */) {
  const int tid = threadIdx.x;
  const int per = (n + PERM_THREADS - 1) / PERM_THREADS;
  const int b = tid * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (b + i < n) local += data[b + i];
  partial[tid] = local;
  __syncthreads();
  for (int off = 1; off < PERM_THREADS; off <<= 1) {
    int v = tid >= off ? partial[tid - off] : 0;
    __syncthreads();
    partial[tid] += v;
    __syncthreads();
  }
  int run = tid ? partial[tid - 1] : 0;
  int total = partial[PERM_THREADS - 1];
  for (int i = 0; i < per; ++i)
    if (b + i < n) {
      int v = data[b + i];
      data[b + i] = run;
      run += v;
    }
  __syncthreads();
  return total;
}

__global__ void __launch_bounds__(PERM_THREADS) perm_count_kernel(const int32_t* __restrict__ idx,
                                                                  int64_t rows, int32_t E,
                                                                  int32_t* __restrict__ cc) {
  extern __shared__ int hist[];
  for (int e = threadIdx.x; e < E; e += PERM_THREADS) hist[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * PERM_CHUNK;
  for (int i = threadIdx.x; i < PERM_CHUNK; i += PERM_THREADS) {
    int64_t r = base + i;
    if (r < rows) {
      int e = idx[r];
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += PERM_THREADS) cc[(int64_t)blockIdx.x * E + e] = hist[e];
}

// one block: chunk counts -> each chunk's first row within its expert's group (in place),
// counts, offsets, active list.  A thread runs down one expert's column of chunk counts,
// PS_BATCH loads issued before the first is used.
constexpr int PS_BATCH = 16;
__global__ void __launch_bounds__(PERM_THREADS) perm_scan_kernel(int32_t* __restrict__ cc, int nchunks,
                                                                 int32_t E, int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ offsets,
                                                                 int4* __restrict__ tiles,
                                                                 int32_t* __restrict__ n_active, int max_tiles,
                                                                 int32_t* __restrict__ slot_of) {
  extern __shared__ int sh[];
  int* tot = sh;               // E
  int* act = sh + E;           // E
  int* partial = sh + 2 * E;   // PERM_THREADS
  for (int e = threadIdx.x; e < E; e += PERM_THREADS) {
    int run = 0;
    for (int c0 = 0; c0 < nchunks; c0 += PS_BATCH) {
      int v[PS_BATCH];
#pragma unroll
      for (int u = 0; u < PS_BATCH; ++u) v[u] = c0 + u < nchunks ? cc[(int64_t)(c0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < PS_BATCH; ++u)
        if (c0 + u < nchunks) {
          cc[(int64_t)(c0 + u) * E + e] = run;
          run += v[u];
        }
    }
    tot[e] = run;
    counts[e] = run;
    act[e] = run > 0;
  }
  __syncthreads();
  int total = block_exclusive_scan(tot, E, partial);
  int nact = block_exclusive_scan(act, E, partial);
  for (int e = threadIdx.x; e < E; e += PERM_THREADS) {
    offsets[e] = tot[e];
    if (counts[e] > 0) tiles[act[e]] = make_int4(e, tot[e], counts[e], -1);  // first row: scatter
    slot_of[e] = act[e];
  }
  for (int sl = nact + threadIdx.x; sl < max_tiles; sl += PERM_THREADS) tiles[sl] = make_int4(-1, 0, 0, -1);
  if (threadIdx.x == 0) {
    offsets[E] = total;
    *n_active = nact;
  }
}

__device__ void bitonic_sort_keys(uint32_t* keys) {
  for (int size = 2; size <= PERM_CHUNK; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < PERM_CHUNK; i += PERM_THREADS) {
        int j = i ^ stride;
        if (j > i) {
          bool up = (i & size) == 0;
          uint32_t a = keys[i], b = keys[j];
          if ((a > b) == up) {
            keys[i] = b;
            keys[j] = a;
          }
        }
      }
      __syncthreads();
    }
}

__global__ void __launch_bounds__(PERM_THREADS) perm_scatter_kernel(const int32_t* __restrict__ idx,
                                                                    int64_t rows, int32_t E,
                                                                    const int32_t* __restrict__ cbase,
                                                                    const int32_t* __restrict__ offsets,
                                                                    const int32_t* __restrict__ slot_of,
                                                                    int32_t* __restrict__ perm,
                                                                    int4* __restrict__ tiles) {
  extern __shared__ int sh[];
  uint32_t* keys = reinterpret_cast<uint32_t*>(sh);  // PERM_CHUNK
  int* sstart = sh + PERM_CHUNK;                     // E
  const int64_t base = (int64_t)blockIdx.x * PERM_CHUNK;
  for (int i = threadIdx.x; i < PERM_CHUNK; i += PERM_THREADS) {
    int64_t r = base + i;
    int e = r < rows ? idx[r] : -1;
    keys[i] = (e >= 0 && e < E) ? ((uint32_t)e << 11) | (uint32_t)i : PAD_KEY;
  }
  __syncthreads();
  bitonic_sort_keys(keys);
  for (int p = threadIdx.x; p < PERM_CHUNK; p += PERM_THREADS) {
    uint32_t key = keys[p];
    if (key != PAD_KEY) {
      uint32_t e = key >> 11;
      if (p == 0 || (keys[p - 1] >> 11) != e) sstart[e] = p;
    }
  }
  __syncthreads();
  for (int p = threadIdx.x; p < PERM_CHUNK; p += PERM_THREADS) {
    uint32_t key = keys[p];
    if (key != PAD_KEY) {
      uint32_t e = key >> 11, i = key & (PERM_CHUNK - 1);
      const int pos = offsets[e] + cbase[(int64_t)blockIdx.x * E + e] + (p - sstart[e]);
      perm[pos] = (int32_t)(base + i);
      if (pos == offsets[e]) tiles[slot_of[e]].w = (int32_t)(base + i);
    }
  }
}

// rows <= PERM_CHUNK: everything in one block
__global__ void __launch_bounds__(PERM_THREADS) perm_small_kernel(const int32_t* __restrict__ idx,
                                                                  int64_t rows, int32_t E,
                                                                  int32_t* __restrict__ counts,
                                                                  int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ perm,
                                                                  int4* __restrict__ tiles,
                                                                  int32_t* __restrict__ n_active,
                                                                  int max_tiles) {
  extern __shared__ int sh[];
  uint32_t* keys = reinterpret_cast<uint32_t*>(sh);  // PERM_CHUNK
  int* hist = sh + PERM_CHUNK;                       // E
  int* act = hist + E;                               // E
  int* sstart = act + E;                             // E
  int* cnt = sstart + E;                             // E
  int* partial = cnt + E;                            // PERM_THREADS
  for (int e = threadIdx.x; e < E; e += PERM_THREADS) hist[e] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < PERM_CHUNK; i += PERM_THREADS) {
    int e = i < rows ? idx[i] : -1;
    bool ok = e >= 0 && e < E;
    keys[i] = ok ? ((uint32_t)e << 11) | (uint32_t)i : PAD_KEY;
    if (ok) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += PERM_THREADS) {
    counts[e] = hist[e];
    cnt[e] = hist[e];
    act[e] = hist[e] > 0;
  }
  __syncthreads();
  int total = block_exclusive_scan(hist, E, partial);
  int nact = block_exclusive_scan(act, E, partial);
  for (int e = threadIdx.x; e < E; e += PERM_THREADS) offsets[e] = hist[e];
  for (int sl = nact + threadIdx.x; sl < max_tiles; sl += PERM_THREADS) tiles[sl] = make_int4(-1, 0, 0, -1);
  if (threadIdx.x == 0) {
    offsets[E] = total;
    *n_active = nact;
  }
  bitonic_sort_keys(keys);
  for (int p = threadIdx.x; p < PERM_CHUNK; p += PERM_THREADS) {
    uint32_t key = keys[p];
    if (key != PAD_KEY) {
      uint32_t e = key >> 11;
      if (p == 0 || (keys[p - 1] >> 11) != e) sstart[e] = p;
    }
  }
  __syncthreads();
  for (int p = threadIdx.x; p < PERM_CHUNK; p += PERM_THREADS) {
    uint32_t key = keys[p];
    if (key != PAD_KEY) {
      uint32_t e = key >> 11, i = key & (PERM_CHUNK - 1);
      perm[hist[e] + (p - sstart[e])] = (int32_t)i;
      if (p == sstart[e]) tiles[act[e]] = make_int4((int)e, hist[e], cnt[e], (int32_t)i);
    }
  }
}

hipError_t launch_permute(const int32_t* idx, int64_t rows, int32_t E, const PermOut& o, void* ws,
                          hipStream_t st) {
  if (rows <= PERM_CHUNK) {
    size_t lds = (PERM_CHUNK + 4 * (size_t)E + PERM_THREADS) * sizeof(int);
    hipLaunchKernelGGL(perm_small_kernel, dim3(1), dim3(PERM_THREADS), lds, st, idx, rows, E, o.counts, o.offsets,
                       o.perm, o.tiles, o.n_active, o.max_tiles);
    return hipGetLastError();
  }
  int nchunks = (int)ceil_div(rows, PERM_CHUNK);
  int32_t* cc = reinterpret_cast<int32_t*>(ws);
  int32_t* slot_of = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + cc_bytes(rows, E));
  hipLaunchKernelGGL(perm_count_kernel, dim3(nchunks), dim3(PERM_THREADS), (size_t)E * sizeof(int), st, idx,
                     rows, E, cc);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(PERM_THREADS), (2 * (size_t)E + PERM_THREADS) * sizeof(int),
                     st, cc, nchunks, E, o.counts, o.offsets, o.tiles, o.n_active, o.max_tiles, slot_of);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(nchunks), dim3(PERM_THREADS),
                     (PERM_CHUNK + (size_t)E) * sizeof(int), st, idx, rows, E, cc, o.offsets, slot_of, o.perm,
                     o.tiles);
  return hipGetLastError();
}

}  // namespace moe
