// Routed experts for large batches: grouped GEMMs on the block-scaled matrix cores.
//
// When an expert holds many routed rows (prefill: about 73 per expert at 4096 tokens,
// thousands on a popular expert), streaming its weights once per 4 rows as the decode
// kernels do would read them dozens of times.  Here a block owns a tile of GT_TOK = 64
// routed rows of one expert (the group's rows in perm order) times 64 weight rows, so
// each weight byte is read once per 64 rows and every MFMA tile is full.
//
// Block: 4 waves; wave w streams weight rows 16w..16w+15 of the block's 64 (gate and up
// for gate/up, down for down) straight from HBM with GT_PF steps in flight, and runs
// four 16x16x128 MFMA tiles (the 64 rows of the token tile) per matrix and per K step.
// The activation tile (two-term e4m3, see quantize_quad8) moves through LDS two K steps
// at a time, double-buffered: the loads of chunk c+1 are in registers while chunk c is
// computed, and one barrier per chunk hands the buffers over.
//
// The grid is ordered so that each XCD (blocks b with the same b mod 8) works through a
// contiguous range of tiles: the tiles of one expert, and the 48 (or 56) weight-row
// blocks of one token tile, meet in the same L2.
//
// Numerics are those of the decode kernels: identical operands per K step and the same
// fp32 accumulation order, so gate/up and down give bit-identical results to them.
#include "mfma_stream.h"

namespace moe {

constexpr int GT_TOK = 64;    // routed rows per tile
constexpr int GT_ROWS = 64;   // weight rows per block (4 waves x 16)
constexpr int GT_PF_GATEUP = 2;  // K steps of weights in flight per wave and matrix (gate/up: two matrices)
constexpr int GT_PF_DOWN = 4;
constexpr int GT_CHUNK = 2;   // K steps per LDS activation chunk
constexpr int GT_RS = 128;    // LDS row of a step's 128 code bytes, 16-byte chunk c at c ^ (row & 7)
// one K step of the tile in LDS: hi codes [64][GT_RS], lo codes [64][GT_RS], hi scales
// [64][4], lo scales [64][4].  The chunk swizzle keeps the MFMA-order reads of 16
// consecutive rows and the row-order writes free of bank conflicts on gfx950.
constexpr int GT_STEP_BYTES = 2 * GT_TOK * GT_RS + 2 * GT_TOK * 4;
constexpr int GT_BUF_BYTES = GT_CHUNK * GT_STEP_BYTES;
static_assert(16 % GT_PF_GATEUP == 0 && 16 % GT_PF_DOWN == 0 && 16 % GT_CHUNK == 0,
              "ring and chunks repeat every 16 steps");

// This thread's share of one chunk: 8 16-byte code pieces and one scale dword.
struct GtRegs {
  u32x4_t v[8];
  uint32_t s;
};

// Loads chunk c (steps GT_CHUNK c ..) of the tile's rows: item j = tid + 256 u is
// (step, term, row, 16-byte piece), so a wave moves 8 whole rows of one term.  Every
// load is issued: rows past the tile read the row srow holds for them (a valid token)
// and steps past the end re-read the last step, so the loads in flight are the same on
// every path (see prime_stream); what they bring for such rows and steps is never used.
__device__ __forceinline__ void gt_load(GtRegs& r, const QRows& q, const int64_t* srow, int K, int nks, int c) {
  const int tid = threadIdx.x;
  unroll_n<8>([&](auto uc) {
    constexpr int u = decltype(uc)::value;
    const int j = tid + 256 * u;  // 2048 = GT_CHUNK x 2 terms x 64 rows x 8 pieces
    const int s = j >> 10, term = (j >> 9) & 1, m = (j >> 3) & 63, part = j & 7;
    const int ks = GT_CHUNK * c + s < nks ? GT_CHUNK * c + s : nks - 1;
    r.v[u] = *reinterpret_cast<const u32x4_t*>((term ? q.lo : q.hi) + srow[m] * K + 128 * ks + 16 * part);
  });
  {
    const int s = tid >> 7, m = (tid >> 1) & 63, term = tid & 1;  // 256 = GT_CHUNK x 64 rows x 2 terms
    const int ks = GT_CHUNK * c + s < nks ? GT_CHUNK * c + s : nks - 1;
    r.s = *reinterpret_cast<const uint32_t*>((term ? q.slo : q.shi) + srow[m] * (K / 32) + 4 * ks);
  }
}

__device__ __forceinline__ void gt_store(const GtRegs& r, uint8_t* buf) {
  const int tid = threadIdx.x;
  unroll_n<8>([&](auto uc) {
    constexpr int u = decltype(uc)::value;
    const int j = tid + 256 * u;
    const int s = j >> 10, term = (j >> 9) & 1, m = (j >> 3) & 63, part = j & 7;
    *reinterpret_cast<u32x4_t*>(buf + s * GT_STEP_BYTES + term * GT_TOK * GT_RS + m * GT_RS + 16 * (part ^ (m & 7))) =
        r.v[u];
  });
  {
    const int s = tid >> 7, m = (tid >> 1) & 63, term = tid & 1;
    *reinterpret_cast<uint32_t*>(buf + s * GT_STEP_BYTES + 2 * GT_TOK * GT_RS + term * GT_TOK * 4 + m * 4) = r.s;
  }
}

// activation operand of step s of a chunk for tile row m (chunks g and 4 + g of the row)
__device__ __forceinline__ void gt_read(AStep& a, const uint8_t* buf, int s, int m, int g) {
  const uint8_t* st = buf + s * GT_STEP_BYTES;
  const int c0 = 16 * (g ^ (m & 7)), c1 = 16 * ((4 + g) ^ (m & 7));
  const uint4 h0 = *reinterpret_cast<const uint4*>(st + m * GT_RS + c0);
  const uint4 h1 = *reinterpret_cast<const uint4*>(st + m * GT_RS + c1);
  const uint4 l0 = *reinterpret_cast<const uint4*>(st + GT_TOK * GT_RS + m * GT_RS + c0);
  const uint4 l1 = *reinterpret_cast<const uint4*>(st + GT_TOK * GT_RS + m * GT_RS + c1);
  a.hi[0] = (int)h0.x; a.hi[1] = (int)h0.y; a.hi[2] = (int)h0.z; a.hi[3] = (int)h0.w;
  a.hi[4] = (int)h1.x; a.hi[5] = (int)h1.y; a.hi[6] = (int)h1.z; a.hi[7] = (int)h1.w;
  a.lo[0] = (int)l0.x; a.lo[1] = (int)l0.y; a.lo[2] = (int)l0.z; a.lo[3] = (int)l0.w;
  a.lo[4] = (int)l1.x; a.lo[5] = (int)l1.y; a.lo[6] = (int)l1.z; a.lo[7] = (int)l1.w;
  a.shi = st[2 * GT_TOK * GT_RS + m * 4 + g];
  a.slo = st[2 * GT_TOK * GT_RS + GT_TOK * 4 + m * 4 + g];
}

// logical block of physical block b: XCD x = b mod 8 runs logical blocks
// x * nb/8 .. (x+1) * nb/8 - 1 (nb a multiple of 8)
__device__ __forceinline__ int gt_logical_block(int b, int nb) { return (b & 7) * (nb >> 3) + (b >> 3); }

// The K loop of one tile: acc[q][tt] += A(token sub-tile tt) x W_q^T over all K steps.
// The loop runs over whole 16-step blocks; steps past the end issue their (clamped)
// loads, stores and barriers like the others and skip only the math, so every path
// issues the same loads and the waits for them are exact.
template <class W, int NMAT, int GT_PF>
__device__ __forceinline__ void gt_mainloop(const W (&w)[NMAT], const QRows& q, const int64_t* srow, int n, int K,
                                            uint8_t* lds, f32x4 (&acc)[NMAT][4]) {
  const int lane = lane_id(), g = lane >> 4, nl = lane & 15;
  const int nks = K / 128, nc = (nks + 15) / 16;
  const int ntt = (n + 15) / 16;  // token sub-tiles holding rows
  // chunk 0 into buffer 0, chunk 1 into registers, the first weight steps in flight
  GtRegs rg;
  gt_load(rg, q, srow, K, nks, 0);
  SBlock sb[NMAT], sbn[NMAT];
  uint4 ring[NMAT][GT_PF];
  prime_stream<W, NMAT, GT_PF>(w, sb, ring, nks);
  gt_store(rg, lds);
  gt_load(rg, q, srow, K, nks, 1);
  lds_barrier();
  for (int cb = 0; cb < nc; ++cb) {
#pragma unroll
    for (int mq = 0; mq < NMAT; ++mq) w[mq].sblock(sbn[mq], cb + 1 < nc ? cb + 1 : cb);
    unroll16([&](auto jc) {
      constexpr int J = decltype(jc)::value;
      const int ks = 16 * cb + J;
      const int ch = ks / GT_CHUNK;
      const uint8_t* buf = lds + (ch & 1) * GT_BUF_BYTES;
      uint4 cw[NMAT];
#pragma unroll
      for (int mq = 0; mq < NMAT; ++mq) {
        cw[mq] = ring[mq][J % GT_PF];
        ring[mq][J % GT_PF] = w[mq].load(ks + GT_PF < nks ? ks + GT_PF : nks - 1);
      }
      if (ks < nks) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          if (tt >= ntt) continue;  // token sub-tile past the tile's rows
          AStep a;
          gt_read(a, buf, J % GT_CHUNK, 16 * tt + nl, g);
#pragma unroll
          for (int mq = 0; mq < NMAT; ++mq) {
            const uint32_t sw = w[mq].template scale<J>(sb[mq]);
            const i32x8 b = as_b(cw[mq]);
            acc[mq][tt] = mx_mfma<W::opsel(J)>(a.hi, b, acc[mq][tt], a.shi, sw);
            acc[mq][tt] = mx_mfma<W::opsel(J)>(a.lo, b, acc[mq][tt], a.slo, sw);
          }
        }
      }
      if constexpr (J % GT_CHUNK == GT_CHUNK - 1) {
        // end of chunk ch: the registers hold chunk ch+1; every wave is past chunk ch-1,
        // so its buffer is free
        gt_store(rg, lds + ((ch + 1) & 1) * GT_BUF_BYTES);
        gt_load(rg, q, srow, K, nks, ch + 2);
        lds_barrier();
      }
    });
#pragma unroll
    for (int mq = 0; mq < NMAT; ++mq) sb[mq] = sbn[mq];
  }
}

// Gate/up with the GLU: a = bf16(silu(g) u) for the tile, re-quantised to two e4m3 terms
// into aq (routed-row order), optionally also as bf16.
template <class W>
__global__ void __launch_bounds__(256, 2) gateup_gemm_kernel(MxArgs p, const int4* __restrict__ gtiles, int ntiles,
                                                              int nb) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int64_t srow[GT_TOK];
  __shared__ int sslot[GT_TOK];
  const int F = p.F, L = p.L, nrt = F / GT_ROWS;
  const int lb = gt_logical_block(blockIdx.x, nb);
  if (lb / nrt >= ntiles) return;  // the grid is rounded up to a multiple of 8
  const int4 tile = gtiles[lb / nrt];
  if (tile.x < 0) return;
  const int rt = lb - (lb / nrt) * nrt;
  const int e = tile.x, r0 = tile.y, n = tile.z;
  const int lane = lane_id(), wave = threadIdx.x / WAVE, g = lane >> 4, nl = lane & 15;
  for (int m = threadIdx.x; m < GT_TOK; m += blockDim.x) {
    const int sl = m < n ? p.perm[r0 + m] : 0;
    sslot[m] = sl;
    srow[m] = sl / p.k;
  }
  __syncthreads();
  const W w[2] = {W::make(p.blob, e, L, F, MAT_GATE, rt * 4 + wave, lane),
                  W::make(p.blob, e, L, F, MAT_UP, rt * 4 + wave, lane)};
  f32x4 acc[2][4];
#pragma unroll
  for (int mq = 0; mq < 2; ++mq)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[mq][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  gt_mainloop<W, 2, GT_PF_GATEUP>(w, p.hq, srow, n, L, lds, acc);
  // GLU into an LDS tile (the activation buffers are free now), then the requantisation
  float* at = reinterpret_cast<float*>(lds);  // [64 tokens][65]
  const int f = rt * GT_ROWS + 16 * wave + nl;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = 16 * tt + 4 * g + j;
      if (m < n) {
        const uint16_t ab = glu_bf16(acc[0][tt][j], acc[1][tt][j]);
        at[m * 65 + 16 * wave + nl] = bf16f(ab);
        if (p.a_bf16) p.a_bf16[(int64_t)sslot[m] * F + f] = ab;
      }
    }
  __syncthreads();
  for (int it = threadIdx.x; it < GT_TOK * 8; it += blockDim.x) {
    // a quad of lanes per (token, scale block): 64 tokens x 2 blocks x 4 lanes
    const int m = it >> 3, blk = (it >> 2) & 1, sub = it & 3;
    if (m < n) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = at[m * 65 + 32 * blk + 8 * sub + i];
      uint32_t hi[2], lo[2], shi, slo;
      quantize_quad8_fmt(v, hi, lo, shi, slo, p.mxfp8 != 0);
      const int64_t off = (int64_t)sslot[m] * F + rt * GT_ROWS + 32 * blk + 8 * sub;
      *reinterpret_cast<uint2*>(p.aq.hi + off) = make_uint2(hi[0], hi[1]);
      *reinterpret_cast<uint2*>(p.aq.lo + off) = make_uint2(lo[0], lo[1]);
      if (sub == 0) {
        const int64_t soff = (int64_t)sslot[m] * (F / 32) + (rt * GT_ROWS) / 32 + blk;
        p.aq.shi[soff] = (uint8_t)shi;
        p.aq.slo[soff] = (uint8_t)slo;
      }
    }
  }
}

// Down: y[slot][l] fp32 for the tile's routed rows.
template <class W>
__global__ void __launch_bounds__(256, 2) down_gemm_kernel(MxArgs p, const int4* __restrict__ gtiles, int ntiles,
                                                            int nb) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int64_t srow[GT_TOK];
  const int F = p.F, L = p.L, nrt = L / GT_ROWS;
  const int lb = gt_logical_block(blockIdx.x, nb);
  if (lb / nrt >= ntiles) return;  // the grid is rounded up to a multiple of 8
  const int4 tile = gtiles[lb / nrt];
  if (tile.x < 0) return;
  const int rt = lb - (lb / nrt) * nrt;
  const int e = tile.x, r0 = tile.y, n = tile.z;
  const int lane = lane_id(), wave = threadIdx.x / WAVE, g = lane >> 4, nl = lane & 15;
  for (int m = threadIdx.x; m < GT_TOK; m += blockDim.x) srow[m] = m < n ? p.perm[r0 + m] : 0;
  __syncthreads();
  const W w[1] = {W::make(p.blob, e, L, F, MAT_DOWN, rt * 4 + wave, lane)};
  f32x4 acc[1][4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) acc[0][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  gt_mainloop<W, 1, GT_PF_DOWN>(w, p.aq, srow, n, F, lds, acc);
  const int l = rt * GT_ROWS + 16 * wave + nl;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = 16 * tt + 4 * g + j;
      if (m < n) p.y[srow[m] * L + l] = acc[0][tt][j];
    }
}

// Tiles of GT_TOK routed rows per active expert, in expert order: gtiles[0, ntiles) =
// {expert, first row in perm, rows, 0}; gtiles[ntiles, max_gtiles) = {-1, 0, 0, 0}.
__global__ void __launch_bounds__(1024) gemm_tiles_kernel(const int32_t* __restrict__ counts,
                                                          const int32_t* __restrict__ offsets, int E,
                                                          int4* __restrict__ gtiles, int max_gtiles) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / WAVE;
  const int per = (E + 1023) / 1024;  // consecutive experts per thread
  int loc = 0;
  for (int q = 0; q < per; ++q) {
    const int e = tid * per + q;
    if (e < E) loc += (counts[e] + GT_TOK - 1) / GT_TOK;
  }
  int wtot = 0;
  const int wex = wave_excl_scan(loc, wtot);
  if (lane == 0) wsum[wave] = wtot;
  __syncthreads();
  int run = wex, total = 0;
  for (int w = 0; w < 16; ++w) {
    run += w < wave ? wsum[w] : 0;
    total += wsum[w];
  }
  for (int q = 0; q < per; ++q) {
    const int e = tid * per + q;
    if (e < E) {
      const int c = counts[e], o = offsets[e];
      for (int i = 0; i < c; i += GT_TOK) gtiles[run++] = make_int4(e, o + i, c - i < GT_TOK ? c - i : GT_TOK, 0);
    }
  }
  for (int j = total + tid; j < max_gtiles; j += 1024) gtiles[j] = make_int4(-1, 0, 0, 0);
}

int64_t gemm_max_tiles(int64_t rows, int32_t E) { return ceil_div(rows, GT_TOK) + (rows < E ? rows : E); }

hipError_t launch_gemm_tiles(const int32_t* counts, const int32_t* offsets, int32_t E, int4* gtiles,
                             int64_t max_gtiles, hipStream_t st) {
  if (E > 16 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_tiles_kernel, dim3(1), dim3(1024), 0, st, counts, offsets, E, gtiles, (int)max_gtiles);
  return hipGetLastError();
}

template <class W>
static hipError_t gemm_lds_limit(const void* fn) {
  (void)sizeof(W);
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 2 * GT_BUF_BYTES);
}

hipError_t launch_gateup_gemm(const MxArgs& p, const int4* gtiles, int64_t max_gtiles, hipStream_t st) {
  if (p.T == 0) return hipSuccess;
  if (p.F % GT_ROWS || p.L % 128) return hipErrorInvalidValue;
  const int64_t nb = (max_gtiles * (p.F / GT_ROWS) + 7) / 8 * 8;
  if (nb > 0x7FFFFFFF) return hipErrorInvalidValue;
  const size_t lds = 2 * GT_BUF_BYTES;
  if (p.packed) {
    static const hipError_t e = gemm_lds_limit<PackedW>(reinterpret_cast<const void*>(&gateup_gemm_kernel<PackedW>));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gateup_gemm_kernel<PackedW>, dim3((unsigned)nb), dim3(256), lds, st, p, gtiles, (int)max_gtiles, (int)nb);
  } else {
    static const hipError_t e = gemm_lds_limit<RecordW>(reinterpret_cast<const void*>(&gateup_gemm_kernel<RecordW>));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gateup_gemm_kernel<RecordW>, dim3((unsigned)nb), dim3(256), lds, st, p, gtiles, (int)max_gtiles, (int)nb);
  }
  return hipGetLastError();
}

hipError_t launch_down_gemm(const MxArgs& p, const int4* gtiles, int64_t max_gtiles, hipStream_t st) {
  if (p.T == 0) return hipSuccess;
  if (p.L % GT_ROWS || p.F % 128) return hipErrorInvalidValue;
  const int64_t nb = (max_gtiles * (p.L / GT_ROWS) + 7) / 8 * 8;
  if (nb > 0x7FFFFFFF) return hipErrorInvalidValue;
  const size_t lds = 2 * GT_BUF_BYTES;
  if (p.packed) {
    static const hipError_t e = gemm_lds_limit<PackedW>(reinterpret_cast<const void*>(&down_gemm_kernel<PackedW>));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(down_gemm_kernel<PackedW>, dim3((unsigned)nb), dim3(256), lds, st, p, gtiles, (int)max_gtiles, (int)nb);
  } else {
    static const hipError_t e = gemm_lds_limit<RecordW>(reinterpret_cast<const void*>(&down_gemm_kernel<RecordW>));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(down_gemm_kernel<RecordW>, dim3((unsigned)nb), dim3(256), lds, st, p, gtiles, (int)max_gtiles, (int)nb);
  }
  return hipGetLastError();
}

}  // namespace moe
