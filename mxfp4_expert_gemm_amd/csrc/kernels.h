// Internal launchers shared between the kernel files and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

namespace moe {

// ---- dequant.hip
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t cols,
                          float* out, hipStream_t st);

// ---- dense_gemv.hip
// One output "segment" of a dense bf16 GEMV over rows of W[rows][K].
struct DenseSeg {
  const uint16_t* W;
  int32_t rows;
  int32_t router;    // 0: out = bf16 [T][rows]; 1: out = fp32 [T][rows] (fp64-folded), wnorm, xnorm
  void* out;
  float* wnorm;      // router only: [rows] Euclidean row norms of W (fp32 sum of squares, rounded sqrt)
  float* xnorm;      // router only: [T] Euclidean norms of the tokens
  const float* add = nullptr;  // bf16 outputs only, nullable: fp32 [T][add_rows][rows] added before the rounding
  int32_t add_rows = 0;
};
// Relative accumulation error bound of router logits from launch_dense_gemv, per
// unit of |x_t| |w_e| (see the kernel for its derivation).
constexpr double GEMV_ROUTER_GAMMA = 16.0 / 8388608.0;  // 16 * 2^-23
hipError_t launch_dense_gemv(const uint16_t* x, int64_t T, int32_t K, const DenseSeg* segs, int nseg,
                             hipStream_t st);

// ---- dense_mfma.hip: the same projections on the matrix cores for token batches
constexpr double DENSE_MFMA_ROUTER_GAMMA = 66.0 / 8388608.0;  // 66 * 2^-23
bool dense_uses_mfma(int64_t T, int32_t K);
// relative error bound of the router logits of launch_dense for T tokens of width K
double dense_router_gamma(int64_t T, int32_t K);
hipError_t launch_dense_mfma(const uint16_t* x, int64_t T, int32_t K, const DenseSeg& s, hipStream_t st);
// the GEMV for few tokens, the matrix-core GEMM otherwise
hipError_t launch_dense(const uint16_t* x, int64_t T, int32_t K, const DenseSeg* segs, int nseg, hipStream_t st);

// ---- route.hip
struct RouteArgs {
  const float* logits_fast;  // [T][E] unbiased fast logits (nullptr in topk mode)
  const float* xnorm;       // [T]
  const float* wnorm;       // [E]
  double gamma;              // relative error bound of logits_fast per |x||w|
  const float* exact_logits; // topk mode: [T][E] caller logits taken as exact (already biased)
  const float* bias;         // nullable
  int64_t bias_stride;
  const uint16_t* x;         // [T][d] for exact recompute
  const uint16_t* router_w;  // [E][d]
  int32_t d;
  int64_t T;
  int32_t E, k, renormalize, flags;
  int32_t* idx;              // [T][k]
  float* w;                  // [T][k]
  float* logits_out;         // nullable [T][E] biased logits
  int32_t* stats;            // [4] counters: tokens needing recompute, logits recomputed, Kulisch uses
  const uint16_t* h;         // nullable [T][L] latent rows to quantise for the experts
  int32_t L;
  int32_t mxfp8;             // 1: quantise h as MXFP8 (one term), 0: two exact e4m3 terms
  QRows hq;
};
hipError_t launch_route(const RouteArgs& a, hipStream_t st);

// Grouping of routed rows by expert.  tiles[0, n_active) = {expert, offset, count, first
// row} of the active experts, ascending; tiles[n_active, max_tiles) = {-1, 0, 0, -1}.
struct PermOut {
  int32_t* counts;    // [E]
  int32_t* offsets;   // [E+1]
  int32_t* perm;      // [T*k]
  int4* tiles;        // [max_tiles]
  int32_t* n_active;  // [1]
  int32_t max_tiles;  // min(E, T*k)
};
// routing, quantisation of h and the grouping in one block, for T <= ROUTE_FUSED_TOKENS
constexpr int ROUTE_FUSED_TOKENS = 8;
hipError_t launch_route_permute_small(const RouteArgs& a, const PermOut& p, hipStream_t st);
// grouping of the rows of routed tokens (distinct valid experts per token),
// T <= 64 and T*k <= ROUTE_SMALL_ROWS
constexpr int ROUTE_SMALL_ROWS = 1024;
constexpr int ROUTE_PLACE_TOKENS = 64;
hipError_t launch_place_rows(const int32_t* idx, int64_t T, int32_t k, int32_t E, const PermOut& p,
                             hipStream_t st);

// ---- permute.hip
constexpr int PERM_CHUNK = 2048;
size_t permute_ws_bytes(int64_t rows, int32_t E);
hipError_t launch_permute(const int32_t* idx, int64_t rows, int32_t E, const PermOut& out, void* ws,
                          hipStream_t st);

// ---- expert_mfma.hip
// Packed expert layout (moe_pack_experts): bytes of one 16-row group of a matrix with K
// columns, and of one expert.
__host__ __device__ constexpr int64_t packed_group_bytes(int K) {
  return (int64_t)(K / 128) * 1024 + (int64_t)((K / 128 + 3) / 4) * 256;
}
__host__ __device__ constexpr int64_t packed_expert_bytes(int L, int F) {
  return 2 * (int64_t)(F / 16) * packed_group_bytes(L) + (int64_t)(L / 16) * packed_group_bytes(F);
}
hipError_t launch_pack_experts(const uint8_t* src, uint8_t* dst, int E, int L, int F, hipStream_t st);

// Start and end events stamped by a kernel's own dispatch (hipExtLaunchKernelGGL): they
// bracket that kernel alone, with no launch gap; both null for a plain launch.
struct KernelEvents {
  hipEvent_t begin = nullptr, end = nullptr;
};
template <typename... Args, typename F = void (*)(Args...)>
inline hipError_t dispatch(const KernelEvents& ev, F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t st,
                           Args... args) {
  if (ev.begin || ev.end)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, st, ev.begin, ev.end, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
  return hipGetLastError();
}

struct MxArgs {
  const uint8_t* blob;
  int32_t packed;            // 1: blob in the packed layout, 0: checkpoint records
  int32_t L, F, k;
  int64_t T;
  const int4* tiles;         // [max_active] {expert, offset in perm, rows, first row}; expert -1: none
  int32_t max_active;        // grid bound: min(E, T*k)
  const int32_t* perm;       // [T*k] slots t*k+j grouped by expert
  QRows hq;                  // [T][L] latent rows h, two-term e4m3
  QRows aq;                  // [T*k][F] GLU outputs by slot, two-term e4m3 (MXFP8 mode: lo term zero)
  int32_t mxfp8;             // activation format of aq (and of hq): MXFP8, else two exact e4m3 terms
  uint16_t* a_bf16;          // nullable [T*k][F] GLU outputs by slot, bf16
  float* y;                  // [T*k][L] down outputs by slot
  unsigned long long* clock; // nullable: MOE_CLOCK_SLOTS {start, end} pairs of the kernel's blocks (clock_begin/end)
  double* sal;               // nullable [T*k][sal_chunks]: per slot, the sum of y^2 over each block of latent rows
  int32_t sal_chunks;        // latent-row blocks of the down kernel that runs (down_*_sal_chunks)
};
hipError_t launch_gateup_mx(const MxArgs& p, hipStream_t st, const KernelEvents& ev = KernelEvents());
hipError_t launch_down_mx(const MxArgs& p, hipStream_t st, const KernelEvents& ev = KernelEvents());
bool down_combine_fits(int64_t T, int32_t k);
// latent-row blocks per routed row of each down kernel: the REAP partials it writes
int32_t down_mx_sal_chunks(int32_t L);
int32_t down_combine_sal_chunks(int32_t L);
hipError_t launch_down_combine_mx(const MxArgs& p, const int32_t* idx, const float* w, uint16_t* z,
                                  hipStream_t st, const KernelEvents& ev = KernelEvents());
hipError_t launch_quantize_rows(const uint16_t* src, int64_t rows, int K, const QRows& q, bool mxfp8, hipStream_t st);

// ---- expert_gemm.hip: grouped GEMMs for experts with many routed rows
// tiles of up to 64 routed rows per active expert, built from counts/offsets, followed by
// their count (GEMM_TILES_TAIL_BYTES): gemm_tiles_bytes in all
constexpr int GEMM_TILES_TAIL_BYTES = 16;
int64_t gemm_max_tiles(int64_t rows, int32_t E);
size_t gemm_tiles_bytes(int64_t rows, int32_t E);
hipError_t launch_gemm_tiles(const int32_t* counts, const int32_t* offsets, int32_t E, int4* gtiles,
                             int64_t max_gtiles, hipStream_t st);
hipError_t launch_gateup_gemm(const MxArgs& p, const int4* gtiles, int64_t max_gtiles, hipStream_t st,
                              const KernelEvents& ev = KernelEvents());
hipError_t launch_down_gemm(const MxArgs& p, const int4* gtiles, int64_t max_gtiles, hipStream_t st,
                            const KernelEvents& ev = KernelEvents());
int32_t down_gemm_sal_chunks(int32_t L);

// ---- stream.hip: expert records fetched from host memory into HBM slots
// copies the record of active expert j (tiles[j].x, j < *n_active) from src (device-
// readable host memory, expert_bytes per record) into slot j of dst
hipError_t launch_gather_experts(const uint8_t* src, int64_t expert_bytes, const int4* tiles, const int32_t* n_active,
                                 int32_t max_slots, uint8_t* dst, hipStream_t st);
// the grouping renumbered to slots (active expert j -> expert j): tiles_s [max_slots],
// counts_s [max_slots], offsets_s [max_slots + 1], idx_s [rows]
hipError_t launch_remap_to_slots(const int4* tiles, const int32_t* n_active, int32_t max_slots, const int32_t* counts,
                                 const int32_t* offsets, const int32_t* idx, int64_t rows, int4* tiles_s,
                                 int32_t* counts_s, int32_t* offsets_s, int32_t* idx_s, hipStream_t st);

// ---- reap.hip: saliency[e] += sum over e's rows (perm order) of w[slot] ||y[slot]||_2
hipError_t launch_reap_saliency(const float* y, const float* w, const int32_t* perm, const int32_t* offsets,
                                int32_t E, int32_t L, double* saliency, hipStream_t st);
// the same sums from the down kernels' partials: ||y[slot]||^2 = sum over c of sal[slot][c]
hipError_t launch_reap_partials(const double* sal, int32_t nch, const float* w, const int32_t* perm,
                                const int32_t* offsets, int32_t E, double* saliency, hipStream_t st);
// bias[e] = 0 for the n_keep experts of highest saliency (ties to the lower index, NaN
// lowest), -inf for the others
hipError_t launch_reap_keep_bias(const double* saliency, int32_t E, int32_t n_keep, float* bias, hipStream_t st);

// ---- combine.hip
hipError_t launch_combine(const float* y, const float* w, int64_t T, int32_t k, int32_t L, uint16_t* z,
                          hipStream_t st);

}  // namespace moe
