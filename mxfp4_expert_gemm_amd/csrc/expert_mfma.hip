// Routed experts on the CDNA4 block-scaled matrix cores.
//
// Expert e is a GLU FFN in the latent space (kimi-k3-mlx digest, architecture table
// and the LatentMoE and SiTU-GLU bullets; kimi-k3-in-c post, MXFP4 section: three
// 3584 x 3072 matrices of 4-bit codes with one 8-bit exponent per 32 weights):
//   g = W_g h, u = W_u h (fp32), a = bf16(silu(g) * u) in fp32, y = W_dn a (fp32).
//
// Every product runs on v_mfma_scale_f32_16x16x128_f8f6f4 with the weights in their
// checkpoint encoding as the FP4 operand: in that instruction a lane holds 32
// consecutive K values (16 bytes) of one of 16 columns and supplies the e8m0 scale of
// exactly those 32 values, which is one code block and one scale byte of a weight row.
// So no instruction is spent expanding weights.  The activations are the FP8 operand,
// split exactly into two e4m3 terms (hi, lo) with their own e8m0 scales (see
// quantize_quad8), so two MFMAs per K step give the bf16 x MXFP4 product.
//
// Two weight layouts feed the same arithmetic (the MFMA operands are identical, so the
// results are bit-identical):
//  * RecordW streams the checkpoint record as it is: a lane loads its row's 16-byte
//    block, so one wave load touches 16 rows x 64 bytes.  Scale bytes are fetched 16 K
//    steps at a time (one 16-byte load per lane, SBlock) and handed to the lane that
//    needs them with a cross-lane permute.
//  * PackedW streams the layout written by moe_pack_experts, where the 1024 bytes one
//    K step of 16 rows needs are contiguous in lane order and the scales of 4 steps
//    are one dword per lane (the matrix core's scale byte select picks the step), so
//    every wave load is a contiguous 1 KB or 256 B run.
//
// Accuracy: one such instruction sums its 128 scaled products with an error of about
// 2^-22 of their absolute sum (measured), which is the level of an fp32 dot product;
// the fp32 accumulator chains the K steps.
//
// A 16x16 MFMA tile covers 16 weight rows x 16 tokens of one expert.  Decode has one
// or two tokens per expert, so most of the tile is idle arithmetic, which costs
// nothing here: the kernels stream weights at HBM speed while the matrix cores stay
// mostly idle.  Weight loads run a fixed number of steps ahead of their MFMAs; the
// activations come from LDS, staged after the first weight loads are issued, because
// vmcnt retires loads in order and a late global load would drain the weight ring.
//
// The matrix-core wrapper, the weight streams and the staged activation operand are in
// mfma_stream.h.
#include "mfma_stream.h"

namespace moe {

// ------------------------------------------------------------ staged activations

// Activations of up to MX_TOK rows staged in LDS: codes [MX_TOK][K] hi, then lo, then
// the e8m0 bytes [MX_TOK][K/32] hi, then lo.
constexpr int MX_TOK = 4;
constexpr size_t MX_LDS_MAX = 60 * 1024;  // dynamic LDS the gate/up and down kernels may take
__host__ __device__ constexpr size_t mx_lds_bytes(int K) { return (size_t)MX_TOK * (2 * K + 2 * (K / 32)); }

// Copy rows src_rows[0..ntok) of q into LDS rows 0..ntok-1 of d; threads tid of
// nthreads (default: the whole block) take part.  The caller syncs.
__device__ __forceinline__ void stage_rows(const ALds& d, const QRows& q, const int64_t* src_rows, int ntok, int K,
                                           int tid = threadIdx.x, int nthreads = blockDim.x) {
  const int per = K / 16;  // 16-byte chunks per row and term
  for (int c = tid; c < 2 * ntok * per; c += nthreads) {
    const int term = c / (ntok * per), rem = c - term * ntok * per;
    const int i = rem / per, off = 16 * (rem - i * per);
    const uint8_t* src = (term ? q.lo : q.hi) + src_rows[i] * K + off;
    uint8_t* dst = (term ? d.lo : d.hi) + i * K + off;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }
  const int nsb = K / 32;
  for (int c = tid; c < 2 * ntok * nsb; c += nthreads) {
    const int term = c / (ntok * nsb), rem = c - term * ntok * nsb;
    const int i = rem / nsb, b = rem - i * nsb;
    (term ? d.slo : d.shi)[i * nsb + b] = (term ? q.slo : q.shi)[src_rows[i] * nsb + b];
  }
}

// Staging in two phases, so that weight loads can be issued between them: the loads of
// this thread's chunks into registers, later their stores to LDS.  Fits when the rows
// take at most NREG 16-byte chunks and 2 scale dwords per thread.
template <int NREG>
struct StageRegs {
  u32x4_t v[NREG];  // native vectors: HIP's uint4 wrapper can keep the array in memory
  uint32_t s[2];
};
template <int NREG>
__device__ __forceinline__ bool stage_fits(int ntok, int K, int nthreads) {
  return 2 * ntok * (K / 16) <= NREG * nthreads && 2 * ntok * (K / 128) <= 2 * nthreads;
}
// thread `tid` of `nthreads`; chunks c = tid + u nthreads (u a compile-time index, so
// the registers never go to memory)
template <int NREG>
__device__ __forceinline__ void stage_load(StageRegs<NREG>& r, const QRows& q, const int64_t* src_rows, int ntok,
                                           int K, int tid, int nthreads) {
  const int per = K / 16, nsd = K / 128;
  unroll_n<NREG>([&](auto uc) {
    constexpr int u = decltype(uc)::value;
    const int c = tid + u * nthreads;
    if (c < 2 * ntok * per) {
      const int term = c / (ntok * per), rem = c - term * ntok * per;
      const int i = rem / per, off = 16 * (rem - i * per);
      r.v[u] = *reinterpret_cast<const u32x4_t*>((term ? q.lo : q.hi) + src_rows[i] * K + off);
    }
  });
  unroll_n<2>([&](auto uc) {
    constexpr int u = decltype(uc)::value;
    const int c = tid + u * nthreads;
    if (c < 2 * ntok * nsd) {
      const int term = c / (ntok * nsd), rem = c - term * ntok * nsd;
      const int i = rem / nsd, b = rem - i * nsd;
      r.s[u] = *reinterpret_cast<const uint32_t*>((term ? q.slo : q.shi) + src_rows[i] * (K / 32) + 4 * b);
    }
  });
}
template <int NREG>
__device__ __forceinline__ void stage_store(const StageRegs<NREG>& r, const ALds& d, int ntok, int K, int tid,
                                            int nthreads) {
  const int per = K / 16, nsd = K / 128;
  unroll_n<NREG>([&](auto uc) {
    constexpr int u = decltype(uc)::value;
    const int c = tid + u * nthreads;
    if (c < 2 * ntok * per) {
      const int term = c / (ntok * per), rem = c - term * ntok * per;
      const int i = rem / per, off = 16 * (rem - i * per);
      *reinterpret_cast<u32x4_t*>((term ? d.lo : d.hi) + i * K + off) = r.v[u];
    }
  });
  unroll_n<2>([&](auto uc) {
    constexpr int u = decltype(uc)::value;
    const int c = tid + u * nthreads;
    if (c < 2 * ntok * nsd) {
      const int term = c / (ntok * nsd), rem = c - term * ntok * nsd;
      const int i = rem / nsd, b = rem - i * nsd;
      *reinterpret_cast<uint32_t*>((term ? d.slo : d.shi) + i * (K / 32) + 4 * b) = r.s[u];
    }
  });
}
// One row (a wave's own) in the same two phases: lane l takes 16-byte chunks
// l + 64u of the hi and of the lo codes and scale dword l.  Fits when K <= 1024 NH.
template <int NH>
struct RowRegs {
  u32x4_t h[NH], l[NH];
  uint32_t s;
};
template <int NH>
__device__ __forceinline__ bool row_fits(int K) {
  return K / 16 <= WAVE * NH && K / 64 <= WAVE;
}
template <int NH>
__device__ __forceinline__ void row_load(RowRegs<NH>& r, const QRows& q, int K, int lane) {
  unroll_n<NH>([&](auto uc) {
    constexpr int u = decltype(uc)::value;
    const int c = lane + WAVE * u;
    if (c < K / 16) {
      r.h[u] = *reinterpret_cast<const u32x4_t*>(q.hi + 16 * c);
      r.l[u] = *reinterpret_cast<const u32x4_t*>(q.lo + 16 * c);
    }
  });
  if (lane < K / 64)
    r.s = lane < K / 128 ? *reinterpret_cast<const uint32_t*>(q.shi + 4 * lane)
                         : *reinterpret_cast<const uint32_t*>(q.slo + 4 * (lane - K / 128));
}
template <int NH>
__device__ __forceinline__ void row_store(const RowRegs<NH>& r, const ALds& d, int K, int lane) {
  unroll_n<NH>([&](auto uc) {
    constexpr int u = decltype(uc)::value;
    const int c = lane + WAVE * u;
    if (c < K / 16) {
      *reinterpret_cast<u32x4_t*>(d.hi + 16 * c) = r.h[u];
      *reinterpret_cast<u32x4_t*>(d.lo + 16 * c) = r.l[u];
    }
  });
  if (lane < K / 64) {
    if (lane < K / 128) *reinterpret_cast<uint32_t*>(d.shi + 4 * lane) = r.s;
    else *reinterpret_cast<uint32_t*>(d.slo + 4 * (lane - K / 128)) = r.s;
  }
}

// the rows of a QRows view that starts at row r
__device__ __forceinline__ QRows qrows_from(const QRows& q, int64_t r, int K) {
  return QRows{q.hi + r * K, q.lo + r * K, q.shi + r * (K / 32), q.slo + r * (K / 32)};
}
__constant__ int64_t kRow0[1] = {0};

// One weight row group (16 rows) times the staged activation rows: acc += A W^T over
// all K steps with the weights PF steps in flight (prime_stream filled sb and ring).
// The NMAT weight streams share the activations (gate and up: 2).
template <class W, int NMAT, int PF>
__device__ __forceinline__ void stream_group(const W (&w)[NMAT], SBlock (&sb)[NMAT], uint4 (&ring)[NMAT][PF],
                                             const ALds& ad, int m, int ntok, int K, int g, f32x4 (&acc)[NMAT]) {
  const int nks = K / 128, nc = (nks + 15) / 16;
  SBlock sbn[NMAT];
  for (int c = 0; c < nc; ++c) {
    // the loads of every step are issued, clamped (see prime_stream); only the math of
    // steps past the end is skipped
#pragma unroll
    for (int q = 0; q < NMAT; ++q) w[q].sblock(sbn[q], c + 1 < nc ? c + 1 : c);
    unroll16([&](auto jc) {
      constexpr int J = decltype(jc)::value;
      const int ks = 16 * c + J;
      uint4 cw[NMAT];
#pragma unroll
      for (int q = 0; q < NMAT; ++q) {
        cw[q] = ring[q][J % PF];
        ring[q][J % PF] = w[q].load(ks + PF < nks ? ks + PF : nks - 1);
      }
      if (ks < nks) {
        AStep a;
        read_a(a, ad, m, ntok, K, ks, g);
#pragma unroll
        for (int q = 0; q < NMAT; ++q) {
          const uint32_t sw = w[q].template scale<J>(sb[q]);
          const i32x8 b = as_b(cw[q]);
          acc[q] = mx_mfma<W::opsel(J)>(a.hi, b, acc[q], a.shi, sw);
          acc[q] = mx_mfma<W::opsel(J)>(a.lo, b, acc[q], a.slo, sw);
        }
      }
    });
#pragma unroll
    for (int q = 0; q < NMAT; ++q) sb[q] = sbn[q];
  }
}

constexpr int MX_ROWS = 64;  // weight rows per block (4 waves x 16)
constexpr int MX_PF = 4;     // K steps of weights in flight per wave (gate/up: per matrix)
static_assert(8 * MX_TOK <= 256 && MX_ROWS == 64, "gate/up requantisation: a quad per token and scale block");
static_assert(16 % MX_PF == 0, "ring slots must repeat every 16 steps");

// ---------------------------------------------------------------- gate / up

// Block: one active expert x 64 rows of gate and up.  Writes a = bf16(silu(g) u) of
// its rows for every token of the expert, re-quantised to two e4m3 terms for the
// down projection (64 rows = two complete scale blocks per token).  Tokens go in
// passes of MX_TOK with their latent rows staged in LDS.
template <class W>
__device__ __forceinline__ void gateup_mx_kernel_body(MxArgs p) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ float atile[MX_TOK][MX_ROWS + 1];
  __shared__ int64_t srows[MX_TOK];
  __shared__ int sslot[MX_TOK];
  const int nrt = p.F / MX_ROWS;
  const int slot = blockIdx.x / nrt;
  const int4 tile = p.tiles[slot];
  const int e = tile.x, r0 = tile.y, ne = tile.z;
  if (e < 0) return;
  const int rt = blockIdx.x - slot * nrt;
  const int lane = lane_id(), wave = threadIdx.x / WAVE;
  const int n = lane & 15, g = lane >> 4;
  const int L = p.L, F = p.F, nks = L / 128;
  const int f = rt * MX_ROWS + 16 * wave + n;  // weight row of this lane
  const W w[2] = {W::make(p.blob, e, L, F, MAT_GATE, rt * 4 + wave, lane),
                  W::make(p.blob, e, L, F, MAT_UP, rt * 4 + wave, lane)};
  const ALds ad = alds(smem, L, MX_TOK);

  for (int p0 = 0; p0 < ne; p0 += MX_TOK) {
    const int ntok = ne - p0 < MX_TOK ? ne - p0 : MX_TOK;
    if (threadIdx.x < MX_TOK) {
      const int sl = threadIdx.x >= ntok ? -1 : ne == 1 ? tile.w : p.perm[r0 + p0 + threadIdx.x];
      sslot[threadIdx.x] = sl;
      srows[threadIdx.x] = sl >= 0 ? sl / p.k : 0;
    }
    __syncthreads();
    // loads in the order they are needed: the token rows, the first scales, the ring
    SBlock sb[2];
    uint4 ring[2][MX_PF];
    if (stage_fits<4>(ntok, L, blockDim.x)) {
      StageRegs<4> sr;
      stage_load(sr, p.hq, srows, ntok, L, threadIdx.x, blockDim.x);
      prime_stream<W, 2, MX_PF>(w, sb, ring, nks);
      stage_store(sr, ad, ntok, L, threadIdx.x, blockDim.x);
    } else {
      stage_rows(ad, p.hq, srows, ntok, L);
      prime_stream<W, 2, MX_PF>(w, sb, ring, nks);
    }
    lds_barrier();  // the primed weight loads stay in flight
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    stream_group<W, 2, MX_PF>(w, sb, ring, ad, n, ntok, L, g, acc);
    // lane holds g, u of tile rows 4g+j for weight row f; rows < ntok are tokens
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int mm = 4 * g + j;
      if (mm < ntok) {
        const uint16_t ab = glu_bf16(acc[0][j], acc[1][j]);
        atile[mm][16 * wave + n] = bf16f(ab);
        if (p.a_bf16) p.a_bf16[(int64_t)sslot[mm] * F + f] = ab;
      }
    }
    __syncthreads();
    if (threadIdx.x < 8 * MX_TOK) {
      // a quad of lanes per (token, scale block), 8 GLU outputs per lane
      const int mm = threadIdx.x >> 3, blk = (threadIdx.x >> 2) & 1, sub = threadIdx.x & 3;
      if (mm < ntok) {
        const int srow = sslot[mm];
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = atile[mm][32 * blk + 8 * sub + i];
        uint32_t hi[2], lo[2], shi, slo;
        quantize_quad8_fmt(v, hi, lo, shi, slo, p.mxfp8 != 0);
        const int64_t off = (int64_t)srow * F + rt * MX_ROWS + 32 * blk + 8 * sub;
        *reinterpret_cast<uint2*>(p.aq.hi + off) = make_uint2(hi[0], hi[1]);
        *reinterpret_cast<uint2*>(p.aq.lo + off) = make_uint2(lo[0], lo[1]);
        if (sub == 0) {
          const int64_t soff = (int64_t)srow * (F / 32) + (rt * MX_ROWS) / 32 + blk;
          p.aq.shi[soff] = (uint8_t)shi;
          p.aq.slo[soff] = (uint8_t)slo;
        }
      }
    }
    __syncthreads();
  }
}

template <class W>
__global__ void __launch_bounds__(256, 2) gateup_mx_kernel(MxArgs p) {
  clock_begin(p.clock);
  gateup_mx_kernel_body<W>(p);
  clock_end(p.clock);
}

// -------------------------------------------------------------------- down

// Block: one active expert x 64 rows of down; y[slot][l] for every token of the expert.
template <class W>
__device__ __forceinline__ void down_mx_kernel_body(MxArgs p) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int64_t srows[MX_TOK];
  __shared__ float ytile[MX_TOK][MX_ROWS];  // REAP partials: the pass's y rows
  const int nrt = p.L / MX_ROWS;
  const int slot = blockIdx.x / nrt;
  const int4 tile = p.tiles[slot];
  const int e = tile.x, r0 = tile.y, ne = tile.z;
  if (e < 0) return;
  const int rt = blockIdx.x - slot * nrt;
  const int lane = lane_id(), wave = threadIdx.x / WAVE;
  const int n = lane & 15, g = lane >> 4;
  const int L = p.L, F = p.F, nks = F / 128;
  const int l = rt * MX_ROWS + 16 * wave + n;
  const W w[1] = {W::make(p.blob, e, L, F, MAT_DOWN, rt * 4 + wave, lane)};
  const ALds ad = alds(smem, F, MX_TOK);

  for (int p0 = 0; p0 < ne; p0 += MX_TOK) {
    const int ntok = ne - p0 < MX_TOK ? ne - p0 : MX_TOK;
    if (threadIdx.x < MX_TOK)
      srows[threadIdx.x] = threadIdx.x >= ntok ? 0 : ne == 1 ? tile.w : p.perm[r0 + p0 + threadIdx.x];
    __syncthreads();
    SBlock sb[1];
    uint4 ring[1][MX_PF];
    if (stage_fits<4>(ntok, F, blockDim.x)) {
      StageRegs<4> sr;
      stage_load(sr, p.aq, srows, ntok, F, threadIdx.x, blockDim.x);
      prime_stream<W, 1, MX_PF>(w, sb, ring, nks);
      stage_store(sr, ad, ntok, F, threadIdx.x, blockDim.x);
    } else {
      stage_rows(ad, p.aq, srows, ntok, F);
      prime_stream<W, 1, MX_PF>(w, sb, ring, nks);
    }
    lds_barrier();  // the primed weight loads stay in flight
    f32x4 acc[1] = {{0.f, 0.f, 0.f, 0.f}};
    stream_group<W, 1, MX_PF>(w, sb, ring, ad, n, ntok, F, g, acc);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int mm = 4 * g + j;
      if (mm < ntok) p.y[srows[mm] * L + l] = acc[0][j];
    }
    if (p.sal) {
      // sum of y^2 over the block's 64 latent rows, per routed row, in row order
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * g + j < ntok) ytile[4 * g + j][16 * wave + n] = acc[0][j];
      __syncthreads();
      if (threadIdx.x < ntok) {
        double q = 0.0;
        for (int i = 0; i < MX_ROWS; ++i) {
          const double v = (double)ytile[threadIdx.x][i];
          q += v * v;
        }
        p.sal[srows[threadIdx.x] * p.sal_chunks + rt] = q;
      }
    }
    __syncthreads();
  }
}

template <class W>
__global__ void __launch_bounds__(256) down_mx_kernel(MxArgs p) {
  clock_begin(p.clock);
  down_mx_kernel_body<W>(p);
  clock_end(p.clock);
}

// Small batches (T*k <= 64): the down projection of every routed row and the weighted
// combine in one kernel.  Block b owns latent rows 16b..16b+15 for all T*k rows t*k+j,
// one wave per routed row (DCM_WAVES waves); y stays in LDS and the block sums it per
// token in slot order in fp64, z[t][l] = bf16(sum_j w[t][j] y[t*k+j][l]), exactly as the
// combine kernel.  Each wave stages its routed row in its own LDS region, so no block
// barrier sits between a wave's first loads and its first step, and the registers hold
// a deep weight ring.  Only tile row 0 carries the routed row; the result's row 0 is used.
constexpr int DCM_SLOTS = 64;
constexpr int DCM_WAVES = 16;
constexpr int DCM_PF = 4;
static_assert(16 % DCM_PF == 0, "ring slots must repeat every 16 steps");
// LDS of one staged row (hi and lo codes, hi and lo scales), padded to 16 bytes
__host__ __device__ constexpr size_t dcm_row_bytes(int F) { return ((size_t)2 * F + F / 16 + 15) & ~(size_t)15; }
constexpr size_t DCM_LDS_MAX = 160 * 1024 - DCM_SLOTS * 16 * sizeof(float);

template <class W>
__device__ __forceinline__ void down_combine_mx_kernel_body(MxArgs p, const int32_t* __restrict__ idx,
                                                            const float* __restrict__ w, uint16_t* __restrict__ z) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ float ys[DCM_SLOTS][16];
  const int lane = lane_id(), wave = threadIdx.x / WAVE;
  const int n = lane & 15, g = lane >> 4;
  const int L = p.L, F = p.F, k = p.k, nks = F / 128;
  const int nslot = (int)p.T * k;
  uint8_t* row = smem + wave * dcm_row_bytes(F);
  const ALds ad{row, row + F, row + 2 * F, row + 2 * F + F / 32};
  for (int s = wave; s < nslot; s += DCM_WAVES) {
    const QRows arow = qrows_from(p.aq, s, F);
    W wr[1] = {W::make(p.blob, idx[s], L, F, MAT_DOWN, blockIdx.x, lane)};
    SBlock sb[1];
    uint4 ring[1][DCM_PF];
    if (row_fits<3>(F)) {
      RowRegs<3> rr;
      row_load(rr, arow, F, lane);
      prime_stream<W, 1, DCM_PF>(wr, sb, ring, nks);
      row_store(rr, ad, F, lane);
    } else {
      stage_rows(ad, arow, kRow0, 1, F, lane, WAVE);
      prime_stream<W, 1, DCM_PF>(wr, sb, ring, nks);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    f32x4 acc[1] = {{0.f, 0.f, 0.f, 0.f}};
    stream_group<W, 1, DCM_PF>(wr, sb, ring, ad, n, 1, F, g, acc);
    if (g == 0) ys[s][n] = acc[0][0];  // D[0][n]
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // the next row may overwrite this one
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  __syncthreads();
  if (p.sal) {
    // REAP partials: sum of y^2 over the block's 16 latent rows, per routed row
    for (int s = threadIdx.x; s < nslot; s += blockDim.x) {
      double q = 0.0;
      for (int nn = 0; nn < 16; ++nn) {
        const double v = (double)ys[s][nn];
        q += v * v;
      }
      p.sal[(int64_t)s * p.sal_chunks + blockIdx.x] = q;
    }
  }
  for (int q = threadIdx.x; q < (int)p.T * 16; q += blockDim.x) {
    const int t = q >> 4, nn = q & 15;
    double acc = 0.0;
    for (int j = 0; j < k; ++j) acc += (double)w[t * k + j] * (double)ys[t * k + j][nn];
    z[(int64_t)t * L + blockIdx.x * 16 + nn] = f64_to_bf16(acc);
  }
}

template <class W>
__global__ void __launch_bounds__(DCM_WAVES * WAVE) down_combine_mx_kernel(MxArgs p, const int32_t* __restrict__ idx,
                                                                         const float* __restrict__ w,
                                                                         uint16_t* __restrict__ z) {
  clock_begin(p.clock);
  down_combine_mx_kernel_body<W>(p, idx, w, z);
  clock_end(p.clock);
}

// ------------------------------------------------------------------ packing

// One thread per 16-byte code unit or per scale dword of the packed layout.
__global__ void __launch_bounds__(256) pack_experts_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                           int E, int L, int F) {
  const int64_t mrec = (int64_t)F * L / 2 + (int64_t)F * L / 32;
  const int64_t prec = packed_expert_bytes(L, F);
  const int64_t gu = (int64_t)(F / 16) * packed_group_bytes(L);
  // units per matrix: R/16 groups x (code tiles + scale tiles) x 64 lanes
  auto units = [](int K, int R) -> int64_t { return (int64_t)(R / 16) * ((K / 128) + (K / 128 + 3) / 4) * 64; };
  const int64_t u_gate = units(L, F), u_exp = 2 * u_gate + units(F, L);
  const int64_t total = (int64_t)E * u_exp;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = u / u_exp;
    int64_t r = u - e * u_exp;
    const int mat = r < u_gate ? MAT_GATE : r < 2 * u_gate ? MAT_UP : MAT_DOWN;
    r -= mat * u_gate;
    const int K = mat == MAT_DOWN ? F : L, R = mat == MAT_DOWN ? L : F;
    const int nks = K / 128, nsc = (nks + 3) / 4;
    const int64_t per_grp = (int64_t)(nks + nsc) * 64;
    const int grp = (int)(r / per_grp);
    const int within = (int)(r - grp * per_grp);
    const int tile = within / 64, lane = within % 64;
    const int row = 16 * grp + (lane & 15), kb = lane >> 4;
    const uint8_t* m = src + e * 3 * mrec + mat * mrec;
    uint8_t* pg = dst + e * prec + (mat == MAT_GATE ? 0 : mat == MAT_UP ? gu : 2 * gu) +
                  (int64_t)grp * packed_group_bytes(K);
    if (tile < nks) {
      *reinterpret_cast<uint4*>(pg + 1024 * tile + 16 * lane) =
          *reinterpret_cast<const uint4*>(m + (int64_t)row * (K / 2) + 64 * tile + 16 * kb);
    } else {
      const int c = tile - nks;
      const uint8_t* srow = m + (int64_t)R * (K / 2) + (int64_t)row * (K / 32);
      uint32_t v = 0;
      for (int j = 0; j < 4; ++j) {
        const int s = 4 * c + j;
        v |= (s < nks ? (uint32_t)srow[4 * s + kb] : 127u) << (8 * j);
      }
      *reinterpret_cast<uint32_t*>(pg + (int64_t)nks * 1024 + 256 * c + 4 * lane) = v;
    }
  }
}

hipError_t launch_pack_experts(const uint8_t* src, uint8_t* dst, int E, int L, int F, hipStream_t st) {
  if (E == 0) return hipSuccess;
  if (L % 128 || F % 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_experts_kernel, dim3(8192), dim3(256), 0, st, src, dst, E, L, F);
  return hipGetLastError();
}

// ------------------------------------------------------------------ launchers

hipError_t launch_gateup_mx(const MxArgs& p, hipStream_t st, const KernelEvents& ev) {
  if (p.T == 0 || p.max_active == 0) return hipSuccess;
  if (p.F % MX_ROWS || p.L % 128) return hipErrorInvalidValue;
  if (mx_lds_bytes(p.L) > MX_LDS_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(p.max_active * (p.F / MX_ROWS)));
  if (p.packed) return dispatch(ev, gateup_mx_kernel<PackedW>, grid, dim3(256), mx_lds_bytes(p.L), st, p);
  return dispatch(ev, gateup_mx_kernel<RecordW>, grid, dim3(256), mx_lds_bytes(p.L), st, p);
}

hipError_t launch_down_mx(const MxArgs& p, hipStream_t st, const KernelEvents& ev) {
  if (p.T == 0 || p.max_active == 0) return hipSuccess;
  if (p.L % MX_ROWS || p.F % 128) return hipErrorInvalidValue;
  if (mx_lds_bytes(p.F) > MX_LDS_MAX) return hipErrorInvalidValue;
  if (p.sal && p.sal_chunks != down_mx_sal_chunks(p.L)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(p.max_active * (p.L / MX_ROWS)));
  if (p.packed) return dispatch(ev, down_mx_kernel<PackedW>, grid, dim3(256), mx_lds_bytes(p.F), st, p);
  return dispatch(ev, down_mx_kernel<RecordW>, grid, dim3(256), mx_lds_bytes(p.F), st, p);
}

bool down_combine_fits(int64_t T, int32_t k) { return T * k <= DCM_SLOTS; }
int32_t down_mx_sal_chunks(int32_t L) { return L / MX_ROWS; }
int32_t down_combine_sal_chunks(int32_t L) { return L / 16; }

template <class W>
static hipError_t down_combine_lds_limit() {
  // the per-wave rows exceed the 64 KB default: raise this kernel's limit once
  static const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&down_combine_mx_kernel<W>),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)DCM_LDS_MAX);
  return e;
}

hipError_t launch_down_combine_mx(const MxArgs& p, const int32_t* idx, const float* w, uint16_t* z,
                                  hipStream_t st, const KernelEvents& ev) {
  if (p.T == 0) return hipSuccess;
  const int nslot = (int)(p.T * p.k);
  const int waves = nslot < DCM_WAVES ? nslot : DCM_WAVES;
  const size_t lds = (size_t)waves * dcm_row_bytes(p.F);
  if (!down_combine_fits(p.T, p.k) || p.L % 16 || p.F % 128 || lds > DCM_LDS_MAX) return hipErrorInvalidValue;
  if (p.sal && p.sal_chunks != down_combine_sal_chunks(p.L)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(p.L / 16)), block(DCM_WAVES * WAVE);
  if (p.packed) {
    const hipError_t e = down_combine_lds_limit<PackedW>();
    if (e != hipSuccess) return e;
    return dispatch(ev, down_combine_mx_kernel<PackedW>, grid, block, (uint32_t)lds, st, p, idx, w, z);
  }
  const hipError_t e = down_combine_lds_limit<RecordW>();
  if (e != hipSuccess) return e;
  return dispatch(ev, down_combine_mx_kernel<RecordW>, grid, block, (uint32_t)lds, st, p, idx, w, z);
}

// ------------------------------------------------- activation quantisation

__global__ void __launch_bounds__(256) quantize_rows_kernel(const uint16_t* __restrict__ src, int64_t rows, int K,
                                                            QRows q, int mxfp8) {
  quantize_quads(src, q, rows * K, (int64_t)blockIdx.x * blockDim.x + threadIdx.x, (int64_t)gridDim.x * blockDim.x,
                 mxfp8 != 0);
}

hipError_t launch_quantize_rows(const uint16_t* src, int64_t rows, int K, const QRows& q, bool mxfp8, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (K % 32) return hipErrorInvalidValue;
  int64_t blocks = ceil_div(rows * (K / 8), 256);
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, rows, K, q, (int)mxfp8);
  return hipGetLastError();
}

}  // namespace moe
