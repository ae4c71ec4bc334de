// Dense bf16 GEMV for few tokens: router logits and the latent projections.
//
// out[t][r] = sum_i x[t][i] * W[r][i] over rows of W[rows][K] (kimi-k3-mlx digest,
// architecture table: the router scores 896 experts from the 7168-wide token;
// Stable LatentMoE projects 7168 -> 3584 and back with bf16 matrices).
//
// Memory-bound: every weight byte is read once per token group, so sums are kept in
// fp64 (fp32 partials of 8 exact products folded into fp64) at no cost in time; the
// bf16 outputs are then the correctly rounded sums but for fp64-level ties.  One wave owns one
// row; lane l reads 16 bytes (8 bf16) at column 8*(64c + l) for chunk c, so each
// load instruction covers 1 KiB of the row contiguously, and reads the matching token
// values from the block's copy of the token rows in LDS.  Products of bf16 pairs are
// exact in fp32 (v_dot2_f32_bf16).
//
// Router rows fold each 8-element chunk partial into an fp64 accumulator.  Error
// bound: a chunk partial is 4 dot2 steps from zero, at most 8 fp32 roundings of
// partial sums bounded by the chunk's sum of |products| (2^-23 each, covering
// round-toward-zero too); the fp64 folds and the 6-step wave tree add at most
// (NCH + 6) * 2^-53 relative to the sum of |products|.  With S = sum |x_i w_i|
// <= |x| |w|, the error of the fp64 logit is below 8.0001 * 2^-23 * |x||w|;
// GEMV_ROUTER_GAMMA = 16 * 2^-23 leaves a factor of two for the fp32 norm sums.
// A token or router row holding a subnormal bf16 value (which the dot instructions
// might flush) gets the norm +inf: its logits are all recomputed exactly.
#include "common.h"
#include "kernels.h"

namespace moe {

struct DenseParams {
  const uint16_t* x;
  int64_t T;
  int32_t K;
  int32_t nseg;
  DenseSeg seg[2];
};

// The token rows are staged once per block in LDS (their loads issued first, then the
// weight row's, so the wait for them leaves the weight loads in flight): the registers
// then hold only the weight row, and more waves fit a SIMD, so the router + latent-down
// grid (4480 rows at one token) and the latent-up grid (7168 rows) run in one round.
template <int NCH, int G>
__global__ void __launch_bounds__(256) dense_gemv_kernel(DenseParams p) {
  constexpr int XN = G * NCH * 64;            // 16-byte pieces of the block's token rows
  constexpr int XPT = (XN + 255) / 256;       // per thread
  __shared__ uint4 xs[XN];
  const int lane = lane_id();
  const int wave = threadIdx.x / WAVE;
  int64_t row = (int64_t)blockIdx.x * 4 + wave;
  // the segment is chosen with scalar selects so every field stays in kernel-argument
  // registers (an indexed p.seg[si] would be read from memory after the loads)
  const bool second = row >= p.seg[0].rows;
  if (second) row -= p.seg[0].rows;
  const DenseSeg s = second ? p.seg[1] : p.seg[0];
  // a wave past the last row works on the segment's last row and writes nothing (no
  // wave leaves before the block's barrier)
  const bool valid = !second || (p.nseg >= 2 && row < p.seg[1].rows);
  if (!valid) row = s.rows - 1;
  const int32_t K = p.K;
  const int64_t t0 = (int64_t)blockIdx.y * G;

  uint4 xv[XPT];
#pragma unroll
  for (int u = 0; u < XPT; ++u) {
    const int i = threadIdx.x + 256 * u < XN ? threadIdx.x + 256 * u : XN - 1;
    const int g = i / (NCH * 64), rem = i - g * (NCH * 64);
    const int col = 8 * rem;  // piece rem = 64 c + lane of token g
    const int64_t t = t0 + g < p.T ? t0 + g : p.T - 1;
    xv[u] = *reinterpret_cast<const uint4*>(p.x + t * K + (col < K ? col : 0));
    if (col >= K || t0 + g >= p.T) xv[u] = make_uint4(0, 0, 0, 0);
  }
  uint4 wr[NCH];
  const uint16_t* wrow = s.W + row * K;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int col = 8 * (64 * c + lane);
    wr[c] = load_nt16(wrow + (col < K ? col : 0));
    if (col >= K) wr[c] = make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < XPT; ++u)
    if (threadIdx.x + 256 * u < XN) xs[threadIdx.x + 256 * u] = xv[u];
  lds_barrier();  // the weight loads stay in flight
  auto xr = [&](int g, int c) -> uint4 { return xs[g * (NCH * 64) + 64 * c + lane]; };

  if (!s.router) {
    // latent projections: fp32 chunk partials folded into fp64, rounded once to bf16
    double acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.0;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint4 xc = xr(g, c);
        float pc = dot2(xc.x, wr[c].x, 0.f);
        pc = dot2(xc.y, wr[c].y, pc);
        pc = dot2(xc.z, wr[c].z, pc);
        pc = dot2(xc.w, wr[c].w, pc);
        acc[g] += (double)pc;
      }
    uint16_t* out = reinterpret_cast<uint16_t*>(s.out);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      double v = wave_sum_dpp(acc[g]);
      if (valid && lane == 0 && t0 + g < p.T) {
        for (int a = 0; a < s.add_rows; ++a) v += (double)s.add[((t0 + g) * s.add_rows + a) * s.rows + row];
        out[(t0 + g) * s.rows + row] = f64_to_bf16(v);
      }
    }
    return;
  }

  // router row: fp32 chunk partials folded into fp64
  double acc[G];
  float wn = 0.f;
  uint32_t wsub = 0;
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = 0.0;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    wn = dot2(wr[c].x, wr[c].x, wn);
    wn = dot2(wr[c].y, wr[c].y, wn);
    wn = dot2(wr[c].z, wr[c].z, wn);
    wn = dot2(wr[c].w, wr[c].w, wn);
    wsub |= bf16x2_subnormal(wr[c].x) | bf16x2_subnormal(wr[c].y) | bf16x2_subnormal(wr[c].z) |
            bf16x2_subnormal(wr[c].w);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint4 xc = xr(g, c);
      float pc = dot2(xc.x, wr[c].x, 0.f);
      pc = dot2(xc.y, wr[c].y, pc);
      pc = dot2(xc.z, wr[c].z, pc);
      pc = dot2(xc.w, wr[c].w, pc);
      acc[g] += (double)pc;
    }
  }
  float* out = reinterpret_cast<float*>(s.out);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    double v = wave_sum_dpp(acc[g]);
    if (valid && lane == 0 && t0 + g < p.T) out[(t0 + g) * s.rows + row] = (float)v;
  }
  wn = wave_sum_dpp(wn);
  const bool wany = __any(wsub != 0u);
  if (valid && lane == 0 && blockIdx.y == 0) s.wnorm[row] = wany ? __builtin_inff() : sqrtf(wn);
  if (valid && row == 0) {  // one wave per token group writes the token norms
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float xn = 0.f;
      uint32_t xsub = 0;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint4 xc = xr(g, c);
        xn = dot2(xc.x, xc.x, xn);
        xn = dot2(xc.y, xc.y, xn);
        xn = dot2(xc.z, xc.z, xn);
        xn = dot2(xc.w, xc.w, xn);
        xsub |= bf16x2_subnormal(xc.x) | bf16x2_subnormal(xc.y) | bf16x2_subnormal(xc.z) |
                bf16x2_subnormal(xc.w);
      }
      xn = wave_sum_dpp(xn);
      const bool xany = __any(xsub != 0u);
      if (lane == 0 && t0 + g < p.T) s.xnorm[t0 + g] = xany ? __builtin_inff() : sqrtf(xn);
    }
  }
}

template <int NCH, int G>
static hipError_t launch_nch_g(const DenseParams& p, hipStream_t st) {
  int64_t rows = p.seg[0].rows + (p.nseg > 1 ? p.seg[1].rows : 0);
  if (ceil_div(p.T, G) > 65535 || ceil_div(rows, 4) > 0x7FFFFFFF) return hipErrorInvalidValue;
  dim3 grid((unsigned)ceil_div(rows, 4), (unsigned)ceil_div(p.T, G));
  hipLaunchKernelGGL((dense_gemv_kernel<NCH, G>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

template <int NCH>
static hipError_t launch_nch(const DenseParams& p, hipStream_t st) {
  // keep the token registers (G * NCH * 4 VGPRs) near 64
  if (NCH <= 4 && p.T >= 4) return launch_nch_g<NCH, 4>(p, st);
  if (NCH <= 8 && p.T >= 2) return launch_nch_g<NCH, 2>(p, st);
  return launch_nch_g<NCH, 1>(p, st);
}

hipError_t launch_dense_gemv(const uint16_t* x, int64_t T, int32_t K, const DenseSeg* segs, int nseg,
                             hipStream_t st) {
  DenseParams p;
  p.x = x;
  p.T = T;
  p.K = K;
  p.nseg = nseg;
  p.seg[0] = segs[0];
  p.seg[1] = nseg > 1 ? segs[1] : segs[0];
  if (T == 0) return hipSuccess;
  int nch = (int)ceil_div(K, 512);
  switch (nch) {
    case 1: return launch_nch<1>(p, st);
    case 2: return launch_nch<2>(p, st);
    case 3: case 4: return launch_nch<4>(p, st);
    case 5: case 6: case 7: return launch_nch<7>(p, st);
    case 8: return launch_nch<8>(p, st);
    case 9: case 10: case 11: case 12: case 13: case 14: return launch_nch<14>(p, st);
    case 15: case 16: return launch_nch<16>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
