// Dense bf16 GEMMs on the matrix cores for token batches: the router logits and the
// latent projections, out[t][n] = sum_i x[t][i] W[n][i] (kimi-k3-mlx digest,
// architecture table: the router scores 896 experts from the 7168-wide token; Stable
// LatentMoE projects 7168 -> 3584 and back with bf16 matrices).
//
// Above a few dozen tokens the GEMV (one weight read per 4 tokens) turns into a
// re-read of the weights per token group; here a block owns a tile of BM tokens x BN
// output rows and every weight byte is read once per BM tokens.  Both operands are
// K-contiguous, the natural operand order of v_mfma_f32_16x16x32_bf16: lane l supplies
// row l%16 of its tile and eight consecutive K values of block l/16 (the K order inside
// an instruction is the same for both operands, so it does not change the sum), and
// result register j of lane l is D[4(l/16)+j][l%16].
//
// Block: 4 waves in 2 x 2, wave tile (16 WM) tokens x (16 WN) rows.  The K loop moves in
// tiles of 64: both operand tiles are loaded by the whole block into registers PF tiles
// ahead (every address clamped into the matrix, so the loads are unconditional and
// retire in issue order), written to one of two LDS buffers, and read back in MFMA
// order; one barrier per K tile hands the buffers over.  An LDS row holds the tile's 128
// bytes with 16-byte chunk c stored at chunk c ^ (row & 7): the MFMA-order reads of 16
// consecutive rows and the row-order writes are then free of bank conflicts on gfx950
// (padding rows to 144 bytes is not: it costs 4 conflict cycles per 16-byte read).
//
// The grid is rasterised in groups of 8 token tiles (the blocks resident at one time
// share a few operand panels) and remapped so that each XCD (blocks b with the same
// b mod 8) runs a contiguous range of that order.
//
// Router logits: the fp32 accumulator of each K tile (two MFMAs from zero) is folded
// into an fp64 sum, and the fp64 sum is rounded once to fp32.  Error bound, modelling
// an MFMA as at most 32 fp32 additions of exact bf16 products to the accumulator, each
// within 2^-23 of the running sum (round-toward-zero included): a K tile errs by at most
// 64 (1 + 2^-18) 2^-23 S_tile with S_tile its sum of |products|; the fp64 folds add
// (K/64) 2^-53 S.  With S <= |x| |w| this stays below 64.001 2^-23 |x||w|;
// DENSE_MFMA_ROUTER_GAMMA = 66 2^-23 leaves room for the fp32 norms (a few 2^-23
// relative).  Products or partial sums below 2^-126 that the matrix cores may flush
// are covered by the absolute padding of the routing certificate (2^-125 per product);
// subnormal bf16 inputs, which could be flushed before the multiply, make the row norm
// +inf (see row_norms_kernel) so every logit of that token or expert is recomputed.
#include "common.h"
#include "kernels.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int DM_BK = 64;     // K per tile
constexpr int DM_RS = 128;    // LDS row stride in bytes (no padding: chunks are swizzled)
constexpr int DM_GROUP = 8;   // token tiles per raster group

struct DenseMfmaArgs {
  const uint16_t* x;  // [T][K]
  const uint16_t* W;  // [N][K]
  void* out;          // bf16 [T][N], or fp32 [T][N] for the router
  int64_t T;
  int32_t K, N;
  int32_t ntm, ntn;   // token tiles, row tiles
  int32_t nblocks;    // ntm * ntn (the grid is rounded up to a multiple of 8)
  const float* add;   // nullable: fp32 [T][add_rows][N] added before the bf16 rounding
  int32_t add_rows;
};

template <int WM, int WN, int PF, bool ROUTER>
__global__ void __launch_bounds__(256, 2) dense_mfma_kernel(DenseMfmaArgs p) {
  constexpr int BM = 32 * WM, BN = 32 * WN;
  constexpr int AP = BM * 8 / 256, BP = BN * 8 / 256;  // 16-byte pieces per thread and K tile
  constexpr int NP = AP + BP;
  constexpr int A_BYTES = BM * DM_RS, STAGE = (BM + BN) * DM_RS;
  extern __shared__ __align__(16) uint8_t lds[];

  const int nbp = gridDim.x;
  const int lb = (blockIdx.x & 7) * (nbp >> 3) + (blockIdx.x >> 3);
  if (lb >= p.nblocks) return;
  const int span = DM_GROUP * p.ntn;
  const int grp = lb / span, first = grp * DM_GROUP;
  const int gs = p.ntm - first < DM_GROUP ? p.ntm - first : DM_GROUP;
  const int within = lb - grp * span;
  const int tm = first + within % gs, tn = within / gs;
  const int64_t t0 = (int64_t)tm * BM;
  const int n0 = tn * BN;
  const int K = p.K, nkt = K / DM_BK;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / WAVE;
  const int wm = wave >> 1, wn = wave & 1, nl = lane & 15, g = lane >> 4;

  // the thread's pieces: piece u is row (tid + 256 u) / 8 of the A tile (u < AP) or of
  // the B tile, 16 bytes at K offset 8 ((tid + 256 u) % 8); rows past the matrix are
  // clamped to its last row (their results are not stored)
  const uint16_t* src[NP];
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const int j = tid + 256 * (u < AP ? u : u - AP);
    const int row = j >> 3, part = j & 7;
    if (u < AP) {
      const int64_t t = t0 + row < p.T ? t0 + row : p.T - 1;
      src[u] = p.x + t * K + 8 * part;
    } else {
      const int n = n0 + row < p.N ? n0 + row : p.N - 1;
      src[u] = p.W + (int64_t)n * K + 8 * part;
    }
  }
  auto dst_off = [&](int u) {
    const int j = tid + 256 * (u < AP ? u : u - AP);
    const int row = j >> 3;
    return (u < AP ? 0 : A_BYTES) + row * DM_RS + 16 * ((j & 7) ^ (row & 7));
  };
  u32x4_t ring[PF][NP];
  auto gload = [&](u32x4_t (&r)[NP], int kt) {
#pragma unroll
    for (int u = 0; u < NP; ++u) r[u] = *reinterpret_cast<const u32x4_t*>(src[u] + (int64_t)kt * DM_BK);
  };
  auto lstore = [&](const u32x4_t (&r)[NP], int buf) {
    uint8_t* s = lds + buf * STAGE;
#pragma unroll
    for (int u = 0; u < NP; ++u) *reinterpret_cast<u32x4_t*>(s + dst_off(u)) = r[u];
  };

  f32x4_t acc[WM][WN];
  double accd[ROUTER ? WM : 1][ROUTER ? WN : 1][4];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int jn = 0; jn < WN; ++jn) acc[i][jn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (ROUTER) {
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int jn = 0; jn < WN; ++jn)
#pragma unroll
        for (int r = 0; r < 4; ++r) accd[i][jn][r] = 0.0;
  }

  // prologue: tiles 0 .. PF-1 in flight, tile 0 into buffer 0, tile PF into its slot.
  // Every load is issued with its tile clamped into the matrix (the loop runs over whole
  // groups of PF tiles and skips only the math past the end), so the loads in flight are
  // the same on every path and the compiler's waits for them are exact.
  unroll_n<PF>([&](auto uc) {
    constexpr int U = decltype(uc)::value;
    gload(ring[U], U < nkt ? U : nkt - 1);
  });
  lstore(ring[0], 0);
  gload(ring[0], PF < nkt ? PF : nkt - 1);
  lds_barrier();

  const int arow = 16 * WM * wm + nl, brow = 16 * WN * wn + nl;
  for (int kt0 = 0; kt0 < nkt; kt0 += PF) {
    unroll_n<PF>([&](auto uc) {
      constexpr int U = decltype(uc)::value;
      const int kt = kt0 + U;
      if (kt < nkt) {
        const uint8_t* s = lds + (kt & 1) * STAGE;
#pragma unroll
        for (int ks = 0; ks < DM_BK / 32; ++ks) {
          bf16x8_t a[WM], b[WN];
#pragma unroll
          for (int i = 0; i < WM; ++i)  // rows arow + 16 i share arow & 7 = nl & 7
            a[i] = *reinterpret_cast<const bf16x8_t*>(s + (arow + 16 * i) * DM_RS + 16 * ((4 * ks + g) ^ (nl & 7)));
#pragma unroll
          for (int jn = 0; jn < WN; ++jn)
            b[jn] = *reinterpret_cast<const bf16x8_t*>(s + A_BYTES + (brow + 16 * jn) * DM_RS +
                                                       16 * ((4 * ks + g) ^ (nl & 7)));
#pragma unroll
          for (int i = 0; i < WM; ++i)
#pragma unroll
            for (int jn = 0; jn < WN; ++jn)
              acc[i][jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[jn], acc[i][jn], 0, 0, 0);
        }
      }
      // tile kt+1 into buffer (kt+1)&1, last read in tile kt-1, which every wave has
      // finished; its slot takes tile kt+1+PF
      constexpr int S = (U + 1) % PF;
      lstore(ring[S], (kt + 1) & 1);
      gload(ring[S], kt + 1 + PF < nkt ? kt + 1 + PF : nkt - 1);
      lds_barrier();
      if constexpr (ROUTER) {
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
          for (int jn = 0; jn < WN; ++jn) {
#pragma unroll
            for (int r = 0; r < 4; ++r) accd[i][jn][r] += (double)acc[i][jn][r];
            acc[i][jn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
      }
    });
  }

#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int jn = 0; jn < WN; ++jn) {
      const int n = n0 + 16 * WN * wn + 16 * jn + nl;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = t0 + 16 * WM * wm + 16 * i + 4 * g + r;
        if (t < p.T && n < p.N) {
          if constexpr (ROUTER)
            static_cast<float*>(p.out)[t * p.N + n] = (float)accd[i][jn][r];
          else if (p.add_rows == 0)
            static_cast<uint16_t*>(p.out)[t * p.N + n] = f32_to_bf16(acc[i][jn][r]);
          else {
            double v = (double)acc[i][jn][r];
            for (int a = 0; a < p.add_rows; ++a) v += (double)p.add[(t * p.add_rows + a) * p.N + n];
            static_cast<uint16_t*>(p.out)[t * p.N + n] = f64_to_bf16(v);
          }
        }
      }
    }
}

// The same GEMM with both operand tiles loaded straight into LDS (lds_dma16: lane i of a
// wave writes its 16 bytes at the instruction's base + 16 i, so the chunk swizzle is
// applied on the source side): no staging registers and no LDS store instructions.  Two
// stages: K tile kt + 1 loads while tile kt is computed.  A K tile is (BM + BN) / 8
// blocks of 8 rows x 128 bytes, block j = 4 u + wave going to the wave's u-th load.  The
// K-tile arithmetic (and the router's fp64 folds) is the one of dense_mfma_kernel, so the
// results are the same.  (Wave tiles of 128 x 64 in 256 x 128 blocks, which the free
// registers allow at one block per CU, measured 2.69 ms against 1.67 ms at prefill32k.)
template <int WM, int WN, bool ROUTER, int MINB>
__global__ void __launch_bounds__(256, MINB) dense_mfma_dma_kernel(DenseMfmaArgs p) {
  constexpr int BM = 32 * WM, BN = 32 * WN;
  constexpr int NU = (BM + BN) / 32;  // 1 KB loads per wave and K tile
  constexpr int A_BYTES = BM * DM_RS, STAGE = (BM + BN) * DM_RS;
  extern __shared__ __align__(16) uint8_t lds[];

  const int nbp = gridDim.x;
  const int lb = (blockIdx.x & 7) * (nbp >> 3) + (blockIdx.x >> 3);
  if (lb >= p.nblocks) return;
  const int span = DM_GROUP * p.ntn;
  const int grp = lb / span, first = grp * DM_GROUP;
  const int gs = p.ntm - first < DM_GROUP ? p.ntm - first : DM_GROUP;
  const int within = lb - grp * span;
  const int tm = first + within % gs, tn = within / gs;
  const int64_t t0 = (int64_t)tm * BM;
  const int n0 = tn * BN;
  const int K = p.K, nkt = K / DM_BK;
  const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / WAVE));
  const int wm = wave >> 1, wn = wave & 1, nl = lane & 15, g = lane >> 4;

  // the lane's rows: row 8 j + lane / 8 of the A tile then the B tile (clamped into the
  // matrix, their results are not stored), chunk (lane mod 8) ^ (row mod 8)
  const uint16_t* src[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int r = 8 * (4 * u + wave) + (lane >> 3);
    const int c = (lane & 7) ^ ((lane >> 3) & 7);
    if (r < BM) {
      const int64_t t = t0 + r < p.T ? t0 + r : p.T - 1;
      src[u] = p.x + t * K + 8 * c;
    } else {
      const int n = n0 + (r - BM) < p.N ? n0 + (r - BM) : p.N - 1;
      src[u] = p.W + (int64_t)n * K + 8 * c;
    }
  }
  auto load_tile = [&](int kt, int buf) {
#pragma unroll
    for (int u = 0; u < NU; ++u) lds_dma16(src[u] + (int64_t)kt * DM_BK, lds + buf * STAGE + (4 * u + wave) * 1024);
  };
  auto wait_barrier = []() { asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  f32x4_t acc[WM][WN];
  double accd[ROUTER ? WM : 1][ROUTER ? WN : 1][4];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int jn = 0; jn < WN; ++jn) acc[i][jn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (ROUTER) {
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int jn = 0; jn < WN; ++jn)
#pragma unroll
        for (int r = 0; r < 4; ++r) accd[i][jn][r] = 0.0;
  }

  load_tile(0, 0);
  wait_barrier();
  const int arow = 16 * WM * wm + nl, brow = 16 * WN * wn + nl;
  for (int kt = 0; kt < nkt; ++kt) {
    // the other stage was last read in tile kt - 1, which every wave has finished
    if (kt + 1 < nkt) load_tile(kt + 1, (kt + 1) & 1);
    const uint8_t* s = lds + (kt & 1) * STAGE;
#pragma unroll
    for (int ks = 0; ks < DM_BK / 32; ++ks) {
      bf16x8_t a[WM], b[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i)  // rows arow + 16 i share arow & 7 = nl & 7
        a[i] = *reinterpret_cast<const bf16x8_t*>(s + (arow + 16 * i) * DM_RS + 16 * ((4 * ks + g) ^ (nl & 7)));
#pragma unroll
      for (int jn = 0; jn < WN; ++jn)
        b[jn] = *reinterpret_cast<const bf16x8_t*>(s + A_BYTES + (brow + 16 * jn) * DM_RS +
                                                   16 * ((4 * ks + g) ^ (nl & 7)));
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int jn = 0; jn < WN; ++jn)
          acc[i][jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[jn], acc[i][jn], 0, 0, 0);
    }
    if constexpr (ROUTER) {
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int jn = 0; jn < WN; ++jn) {
#pragma unroll
          for (int r = 0; r < 4; ++r) accd[i][jn][r] += (double)acc[i][jn][r];
          acc[i][jn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
    wait_barrier();  // tile kt + 1 is in LDS; every wave is past tile kt
  }

#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int jn = 0; jn < WN; ++jn) {
      const int n = n0 + 16 * WN * wn + 16 * jn + nl;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = t0 + 16 * WM * wm + 16 * i + 4 * g + r;
        if (t < p.T && n < p.N) {
          if constexpr (ROUTER)
            static_cast<float*>(p.out)[t * p.N + n] = (float)accd[i][jn][r];
          else if (p.add_rows == 0)
            static_cast<uint16_t*>(p.out)[t * p.N + n] = f32_to_bf16(acc[i][jn][r]);
          else {
            double v = (double)acc[i][jn][r];
            for (int a = 0; a < p.add_rows; ++a) v += (double)p.add[(t * p.add_rows + a) * p.N + n];
            static_cast<uint16_t*>(p.out)[t * p.N + n] = f64_to_bf16(v);
          }
        }
      }
    }
}

// Euclidean norms of bf16 rows, as the GEMV router computes them: each lane sums the
// squares of its 8-element chunks (exact products, fp32 sums, chunks in column order),
// the wave adds the lanes, the root is rounded once.  A row with a subnormal bf16 value
// gets +inf.  One launch covers the router's rows (a, na of them) and the tokens (b, nb);
// a lane's chunks are loaded RN_CH at a time, all before the first is used (K <= 8192: one
// memory round trip per row).
constexpr int RN_CH = 16;
__global__ void __launch_bounds__(256) row_norms_kernel(const uint16_t* __restrict__ a, int64_t na,
                                                        const uint16_t* __restrict__ b, int64_t nb, int32_t K,
                                                        float* __restrict__ outa, float* __restrict__ outb) {
  const int lane = lane_id();
  int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / WAVE;
  if (row >= na + nb) return;
  const bool second = row >= na;
  if (second) row -= na;
  const uint16_t* r = (second ? b : a) + row * K;
  float s = 0.f;
  uint32_t sub = 0;
  for (int c0 = 0; 8 * WAVE * c0 < K; c0 += RN_CH) {
    uint4 v[RN_CH];
#pragma unroll
    for (int c = 0; c < RN_CH; ++c) {
      const int col = 8 * (lane + WAVE * (c0 + c));
      v[c] = col < K ? load_nt16(r + col) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int c = 0; c < RN_CH; ++c) {
      const uint32_t d[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s = dot2(d[i], d[i], s);
        sub |= bf16x2_subnormal(d[i]);
      }
    }
  }
  s = wave_sum_dpp(s);
  const bool any_sub = __any(sub != 0u);
  if (lane == 0) (second ? outb : outa)[row] = any_sub ? __builtin_inff() : sqrtf(s);
}

// ------------------------------------------------------------------------- host

// tokens from which the matrix-core path replaces the GEMV
constexpr int64_t DENSE_MFMA_MIN_T = 32;

bool dense_uses_mfma(int64_t T, int32_t K) { return T >= DENSE_MFMA_MIN_T && K % DM_BK == 0; }

double dense_router_gamma(int64_t T, int32_t K) {
  return dense_uses_mfma(T, K) ? DENSE_MFMA_ROUTER_GAMMA : GEMV_ROUTER_GAMMA;
}

template <int WM, int WN, int PF, bool ROUTER>
static hipError_t launch_dm(const DenseMfmaArgs& a0, hipStream_t st) {
  constexpr int BM = 32 * WM, BN = 32 * WN;
  constexpr int LDS = 2 * (BM + BN) * DM_RS;
  DenseMfmaArgs a = a0;
  a.ntm = (int32_t)ceil_div(a.T, BM);
  a.ntn = (int32_t)ceil_div(a.N, BN);
  const int64_t nb = (int64_t)a.ntm * a.ntn;
  if (ceil_div(a.T, BM) > 0x7FFFFFFF || nb > 0x7FFFFFF0) return hipErrorInvalidValue;
  a.nblocks = (int32_t)nb;
  const unsigned grid = (unsigned)((nb + 7) / 8 * 8);
  if constexpr (LDS > 65536) {
    static const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&dense_mfma_kernel<WM, WN, PF, ROUTER>),
        hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((dense_mfma_kernel<WM, WN, PF, ROUTER>), dim3(grid), dim3(256), LDS, st, a);
  return hipGetLastError();
}

template <int WM, int WN, bool ROUTER, int MINB>
static hipError_t launch_dm_dma(const DenseMfmaArgs& a0, hipStream_t st) {
  constexpr int BM = 32 * WM, BN = 32 * WN;
  constexpr int LDS = 2 * (BM + BN) * DM_RS;
  DenseMfmaArgs a = a0;
  a.ntm = (int32_t)ceil_div(a.T, BM);
  a.ntn = (int32_t)ceil_div(a.N, BN);
  const int64_t nb = (int64_t)a.ntm * a.ntn;
  if (ceil_div(a.T, BM) > 0x7FFFFFFF || nb > 0x7FFFFFF0) return hipErrorInvalidValue;
  a.nblocks = (int32_t)nb;
  const unsigned grid = (unsigned)((nb + 7) / 8 * 8);
  if constexpr (LDS > 65536) {
    static const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&dense_mfma_dma_kernel<WM, WN, ROUTER, MINB>),
        hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((dense_mfma_dma_kernel<WM, WN, ROUTER, MINB>), dim3(grid), dim3(256), LDS, st, a);
  return hipGetLastError();
}

// The LDS-direct kernel loads one K tile ahead, the register-staged one PF tiles: the
// first is faster once the grid holds at least three blocks per CU slot pair (768
// blocks), where the other resident block covers the load latency (prefill32k: latent
// projections 1.90 -> 1.67 ms, router 0.68 -> 0.65 ms; prefill4k latent 0.31 -> 0.28 ms),
// the second for smaller grids (prefill4k's router, 448 blocks: 0.12 against 0.14 ms).
static bool dm_dma_pays(int64_t T, int32_t N, int BM, int BN) { return ceil_div(T, BM) * ceil_div(N, BN) >= 768; }

// Tile of a batch below 256 tokens: the largest of 64 x 64, 64 x 32 and 32 x 32 (tokens x
// rows) that still gives the grid about one block per CU, since a few dozen blocks (the
// router at 64 tokens has 14 tiles of 64 x 64) leave most of the chip idle.  Every shape
// runs the same K-tile arithmetic, so the results do not depend on the choice.
static int small_tile(int64_t T, int32_t N) {
  if (ceil_div(T, 64) * ceil_div(N, 64) >= 224) return 0;
  if (ceil_div(T, 64) * ceil_div(N, 32) >= 200) return 1;
  return 2;
}

hipError_t launch_dense_mfma(const uint16_t* x, int64_t T, int32_t K, const DenseSeg& s, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (!dense_uses_mfma(T, K) || s.rows <= 0) return hipErrorInvalidValue;
  DenseMfmaArgs a;
  a.x = x;
  a.W = s.W;
  a.out = s.out;
  a.T = T;
  a.K = K;
  a.N = s.rows;
  a.add = s.add;
  a.add_rows = s.add ? s.add_rows : 0;
  if (s.router) {
    hipLaunchKernelGGL(row_norms_kernel, dim3((unsigned)ceil_div(s.rows + T, 4)), dim3(256), 0, st, s.W,
                       (int64_t)s.rows, x, T, K, s.wnorm, s.xnorm);
    if (T >= 256)
      return dm_dma_pays(T, s.rows, 128, 64) ? launch_dm_dma<4, 2, true, 2>(a, st) : launch_dm<4, 2, 2, true>(a, st);
    switch (small_tile(T, s.rows)) {
      case 0: return launch_dm<2, 2, 4, true>(a, st);
      case 1: return launch_dm<2, 1, 4, true>(a, st);
      default: return launch_dm<1, 1, 4, true>(a, st);
    }
  }
  if (T >= 256)
    return dm_dma_pays(T, s.rows, 128, 128) ? launch_dm_dma<4, 4, false, 2>(a, st) : launch_dm<4, 4, 2, false>(a, st);
  switch (small_tile(T, s.rows)) {
    case 0: return launch_dm<2, 2, 4, false>(a, st);
    case 1: return launch_dm<2, 1, 4, false>(a, st);
    default: return launch_dm<1, 1, 4, false>(a, st);
  }
}

hipError_t launch_dense(const uint16_t* x, int64_t T, int32_t K, const DenseSeg* segs, int nseg, hipStream_t st) {
  if (!dense_uses_mfma(T, K)) return launch_dense_gemv(x, T, K, segs, nseg, st);
  for (int i = 0; i < nseg; ++i) {
    const hipError_t e = launch_dense_mfma(x, T, K, segs[i], st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace moe
