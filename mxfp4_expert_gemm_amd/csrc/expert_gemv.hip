// Routed experts for few tokens per expert: memory-bound MXFP4 GEMV.
//
// Expert e is a GLU FFN in the latent space (kimi-k3-mlx digest, architecture table
// and the LatentMoE and SiTU-GLU bullets; kimi-k3-in-c post, MXFP4 section: three
// 3584 x 3072 matrices, 4-bit codes with one 8-bit exponent per 32 weights):
//   g = W_g h, u = W_u h (fp32), a = bf16(silu(g) * u) in fp32, y = W_dn a (fp32).
//
// One block per (active expert, group of rows).  One wave owns one output row at a
// time; lane l reads the code dword at byte 4*(64c + l) of the row for chunk c, so
// each load instruction reads 256 contiguous bytes and the eight weights of a dword
// always share one scale (32 weights = 4 dwords).  The row's scale bytes come in
// one dword load per lane and are handed out with a lane shuffle.  Weights are
// expanded in registers with v_cvt_scalef32_pk_bf16_fp4 (E2M1 times 2^(s-127) is
// exact in bf16 inside the range of the e8m0 exponents) and multiplied with the
// bf16 activations by v_dot2_f32_bf16 into fp32 accumulators; the activations for
// the row's columns stay in registers for all rows the wave visits.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int EXP_WAVES = 4;
constexpr int EXP_RPW = 4;  // rows per wave per block
constexpr int EXP_ROWS = EXP_WAVES * EXP_RPW;

template <int NCH>
struct RowCodes {
  uint32_t q[NCH];
  uint32_t s;  // this lane's dword of the row's scale bytes
};

template <int NCH>
__device__ __forceinline__ void load_row(RowCodes<NCH>& r, const uint8_t* codes, const uint8_t* scales,
                                         int cols, int lane) {
  const uint32_t* c32 = reinterpret_cast<const uint32_t*>(codes);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    int m = 64 * c + lane;
    r.q[c] = (8 * m < cols) ? __builtin_nontemporal_load(c32 + m) : 0u;
  }
  r.s = (4 * lane < cols / 32) ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(scales) + lane)
                               : 0u;
}

// acc[i] += sum over this lane's columns of act[i] * W for the row in r
template <int NCH, int NT>
__device__ __forceinline__ void row_dot(const RowCodes<NCH>& r, const uint4 (&act)[NT][NCH], float (&acc)[NT],
                                        int lane) {
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    int b = (64 * c + lane) >> 2;  // 32-weight block of this dword
    uint32_t sd = __shfl(r.s, b >> 2);
    float sc = e8m0_to_f32((sd >> (8 * (b & 3))) & 0xFFu);
    uint32_t w01 = fp4x2_to_bf16x2<0>(r.q[c], sc);
    uint32_t w23 = fp4x2_to_bf16x2<1>(r.q[c], sc);
    uint32_t w45 = fp4x2_to_bf16x2<2>(r.q[c], sc);
    uint32_t w67 = fp4x2_to_bf16x2<3>(r.q[c], sc);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      acc[i] = dot2(act[i][c].x, w01, acc[i]);
      acc[i] = dot2(act[i][c].y, w23, acc[i]);
      acc[i] = dot2(act[i][c].z, w45, acc[i]);
      acc[i] = dot2(act[i][c].w, w67, acc[i]);
    }
  }
}

// SiLU in fp32 without overflow: for g < 0 use g e^g / (1 + e^g), so a large |g|
// underflows gracefully instead of dividing by an infinite exp(-g).
__device__ __forceinline__ float silu_f32(float g) {
  if (g >= 0.f) return g / (1.0f + expf(-g));
  float e = expf(g);
  return g * e / (1.0f + e);
}

template <int NCH, int NT>
__global__ void __launch_bounds__(256) gateup_glu_kernel(ExpertArgs p) {
  const int nfb = (int)ceil_div(p.F, EXP_ROWS);
  const int slot = blockIdx.x / nfb;
  if (slot >= *p.n_active) return;
  const int f0 = (blockIdx.x - slot * nfb) * EXP_ROWS;
  const int e = p.active[slot];
  const int lane = lane_id(), wave = threadIdx.x / WAVE;
  const int L = p.L, F = p.F;
  const int64_t mat = (int64_t)F * L / 2 + (int64_t)F * L / 32;
  const uint8_t* rec = p.blob + (int64_t)e * 3 * mat;
  const uint8_t* gcodes = rec;
  const uint8_t* gscales = rec + (int64_t)F * L / 2;
  const uint8_t* ucodes = rec + mat;
  const uint8_t* uscales = ucodes + (int64_t)F * L / 2;
  const int r0 = p.offsets[e], ne = p.counts[e];

  for (int p0 = 0; p0 < ne; p0 += NT) {
    uint4 act[NT][NCH];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const bool tok_ok = p0 + i < ne;
      const int64_t t = tok_ok ? p.perm[r0 + p0 + i] / p.k : 0;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        int m = 64 * c + lane;
        act[i][c] = (tok_ok && 8 * m < L) ? *reinterpret_cast<const uint4*>(p.h + t * L + 8 * m)
                                          : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll 1
    for (int rr = 0; rr < EXP_RPW; ++rr) {
      const int f = f0 + wave * EXP_RPW + rr;
      if (f >= F) break;
      RowCodes<NCH> gr, ur;
      load_row(gr, gcodes + (int64_t)f * (L / 2), gscales + (int64_t)f * (L / 32), L, lane);
      load_row(ur, ucodes + (int64_t)f * (L / 2), uscales + (int64_t)f * (L / 32), L, lane);
      float ag[NT], au[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i) ag[i] = au[i] = 0.f;
      row_dot<NCH, NT>(gr, act, ag, lane);
      row_dot<NCH, NT>(ur, act, au, lane);
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        float g = wave_sum(ag[i]);
        float u = wave_sum(au[i]);
        if (lane == i && p0 + i < ne) p.a[(int64_t)(r0 + p0 + i) * F + f] = f32_to_bf16(silu_f32(g) * u);
      }
    }
  }
}

template <int NCH, int NT>
__global__ void __launch_bounds__(256) down_kernel(ExpertArgs p) {
  const int nlb = (int)ceil_div(p.L, EXP_ROWS);
  const int slot = blockIdx.x / nlb;
  if (slot >= *p.n_active) return;
  const int l0 = (blockIdx.x - slot * nlb) * EXP_ROWS;
  const int e = p.active[slot];
  const int lane = lane_id(), wave = threadIdx.x / WAVE;
  const int L = p.L, F = p.F;
  const int64_t mat = (int64_t)F * L / 2 + (int64_t)F * L / 32;
  const uint8_t* dcodes = p.blob + (int64_t)e * 3 * mat + 2 * mat;
  const uint8_t* dscales = dcodes + (int64_t)L * F / 2;
  const int r0 = p.offsets[e], ne = p.counts[e];

  for (int p0 = 0; p0 < ne; p0 += NT) {
    uint4 act[NT][NCH];
    int64_t dst[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const bool tok_ok = p0 + i < ne;
      const int64_t r = r0 + p0 + (tok_ok ? i : 0);
      dst[i] = tok_ok ? p.perm[r] : -1;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        int m = 64 * c + lane;
        act[i][c] = (tok_ok && 8 * m < F) ? *reinterpret_cast<const uint4*>(p.a + r * F + 8 * m)
                                          : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll 1
    for (int rr = 0; rr < EXP_RPW; ++rr) {
      const int l = l0 + wave * EXP_RPW + rr;
      if (l >= L) break;
      RowCodes<NCH> dr;
      load_row(dr, dcodes + (int64_t)l * (F / 2), dscales + (int64_t)l * (F / 32), F, lane);
      float ay[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i) ay[i] = 0.f;
      row_dot<NCH, NT>(dr, act, ay, lane);
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        float v = wave_sum(ay[i]);
        if (lane == i && dst[i] >= 0) p.y[dst[i] * L + l] = v;
      }
    }
  }
}

template <int NCH, int NT>
static hipError_t launch_k(bool gate, const ExpertArgs& p, dim3 grid, hipStream_t st) {
  if (gate)
    hipLaunchKernelGGL((gateup_glu_kernel<NCH, NT>), grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((down_kernel<NCH, NT>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

template <int NCH>
static hipError_t launch_nt(bool gate, const ExpertArgs& p, int rows_total, hipStream_t st) {
  dim3 grid((unsigned)(p.max_active * ceil_div(rows_total, EXP_ROWS)));
  // tokens handled per pass over the weights: the mean rows per possible slot
  const double per = (double)p.T * p.k / (double)p.max_active;
  if (per <= 1.0) return launch_k<NCH, 1>(gate, p, grid, st);
  if (per <= 2.0) return launch_k<NCH, 2>(gate, p, grid, st);
  return launch_k<NCH, 4>(gate, p, grid, st);
}

static hipError_t dispatch(bool gate, const ExpertArgs& p, int cols, int rows_total, hipStream_t st) {
  switch ((int)ceil_div(cols, 512)) {
    case 1: return launch_nt<1>(gate, p, rows_total, st);
    case 2: return launch_nt<2>(gate, p, rows_total, st);
    case 3: case 4: return launch_nt<4>(gate, p, rows_total, st);
    case 5: case 6: return launch_nt<6>(gate, p, rows_total, st);
    case 7: return launch_nt<7>(gate, p, rows_total, st);
    case 8: return launch_nt<8>(gate, p, rows_total, st);
    case 9: case 10: case 11: case 12: return launch_nt<12>(gate, p, rows_total, st);
    case 13: case 14: case 15: case 16: return launch_nt<16>(gate, p, rows_total, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_expert_gateup(const ExpertArgs& p, hipStream_t st) {
  if (p.T == 0 || p.max_active == 0) return hipSuccess;
  return dispatch(true, p, p.L, p.F, st);
}

hipError_t launch_expert_down(const ExpertArgs& p, hipStream_t st) {
  if (p.T == 0 || p.max_active == 0) return hipSuccess;
  return dispatch(false, p, p.F, p.L, st);
}

// a_slot[perm[r]] = a_perm[r], rows of F bf16
__global__ void unpermute_rows_kernel(const uint16_t* __restrict__ a_perm, const int32_t* __restrict__ perm,
                                      int64_t rows, int32_t F, uint16_t* __restrict__ a_slot) {
  const int64_t r = blockIdx.x;
  if (r >= rows) return;
  const int64_t d = perm[r];
  for (int c = threadIdx.x; c < F / 8; c += blockDim.x)
    *reinterpret_cast<uint4*>(a_slot + d * F + 8 * c) = *reinterpret_cast<const uint4*>(a_perm + r * F + 8 * c);
}

hipError_t launch_unpermute_rows(const uint16_t* a_perm, const int32_t* perm, int64_t rows, int32_t F,
                                 uint16_t* a_slot, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(unpermute_rows_kernel, dim3((unsigned)rows), dim3(128), 0, st, a_perm, perm, rows, F, a_slot);
  return hipGetLastError();
}

}  // namespace moe
