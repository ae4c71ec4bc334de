// Internal launchers shared between the kernel files and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
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
  int32_t router;    // 0: out = bf16 [T][rows]; 1: out = fp32 [T][rows] (fp64-folded), wnorm2, xnorm2
  void* out;
  float* wnorm2;     // router only: [rows] squared row norms of W
  float* xnorm2;     // router only: [T] squared norms of the tokens
};
// Relative accumulation error bound of router logits from launch_dense_gemv, per
// unit of |x_t| |w_e| (see the kernel for its derivation).
constexpr double GEMV_ROUTER_GAMMA = 16.0 / 8388608.0;  // 16 * 2^-23
hipError_t launch_dense_gemv(const uint16_t* x, int64_t T, int32_t K, const DenseSeg* segs, int nseg,
                             hipStream_t st);

// ---- route.hip
struct RouteArgs {
  const float* logits_fast;  // [T][E] unbiased fast logits (nullptr in topk mode)
  const float* xnorm2;       // [T]
  const float* wnorm2;       // [E]
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
};
hipError_t launch_route(const RouteArgs& a, hipStream_t st);

// ---- permute.hip
constexpr int PERM_CHUNK = 2048;
size_t permute_ws_bytes(int64_t rows, int32_t E);
hipError_t launch_permute(const int32_t* idx, int64_t rows, int32_t E, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* active, int32_t* n_active, void* ws, hipStream_t st);

// ---- expert_gemv.hip
struct ExpertArgs {
  const uint16_t* h;         // [T][L] bf16
  const uint8_t* blob;
  int32_t L, F, k;
  int64_t T;
  const int32_t* counts;     // [E]
  const int32_t* offsets;    // [E+1]
  const int32_t* perm;       // [T*k]
  const int32_t* active;     // [E] active experts, ascending
  const int32_t* n_active;   // [1]
  int32_t max_active;        // grid bound: min(E, T*k)
  uint16_t* a;               // [T*k][F] bf16, permuted row order
  float* y;                  // [T*k][L] fp32, slot order (row t*k+j)
};
hipError_t launch_expert_gateup(const ExpertArgs& a, hipStream_t st);
hipError_t launch_expert_down(const ExpertArgs& a, hipStream_t st);
hipError_t launch_unpermute_rows(const uint16_t* a_perm, const int32_t* perm, int64_t rows, int32_t F,
                                 uint16_t* a_slot, hipStream_t st);

// ---- combine.hip
hipError_t launch_combine(const float* y, const float* w, int64_t T, int32_t k, int32_t L, uint16_t* z,
                          hipStream_t st);

}  // namespace moe
