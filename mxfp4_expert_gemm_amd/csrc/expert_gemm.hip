// Routed experts for large batches: grouped GEMMs on the block-scaled matrix cores.
//
// When an expert holds many routed rows (prefill: about 73 per expert at 4096 tokens,
// thousands on a popular expert), streaming its weights once per 4 rows as the decode
// kernels do would read them dozens of times.  Here a block owns a tile of up to GT_TOK =
// 64 routed rows of one expert (the group's rows in perm order) and a block of weight
// rows, so each weight byte is read once per tile.
//
// The products run on v_mfma_scale_f32_32x32x64_f8f6f4: the FP8 operand is a 32-row token
// sub-tile of the activations (two exact e4m3 terms, see quantize_quad8), the FP4 operand
// 32 weight rows as stored, each with its e8m0 scales.  Operand layout, measured on gfx950
// with exact small-integer operands: lane l works on row/column l%32 and g = l/32; the
// FP8 operand holds K = 16g..16g+15 in registers 0-3 and 32+16g..32+16g+15 in registers
// 4-7; the FP4 operand holds K = 32g..32g+31 (low nibble first); lane r + 32b supplies the
// scale of row/column r for K block b; result register v of lane l is
// D[8(v/4) + 4g + v%4][l%32].  One such product does twice the work of the 16x16x128 form
// per operand byte read.
//
// Block: 4 waves.  A wave owns 32 weight rows of each of its two matrices (gate and up,
// or two 32-row groups of down) and the tile's 32-row token sub-tiles; a K step of 128 is
// two half-steps of 64.  Weight operands are loaded per wave straight from memory into
// registers, PF steps ahead; the activation tile moves through LDS in chunks of 128
// row-steps (two K steps of 64 rows, four of 32), double-buffered: chunk c+1 is loaded
// straight into the other buffer while chunk c is computed, and one barrier per chunk
// hands the buffers over.  Two blocks share a CU.
//
// Block b of the grid runs on XCD b mod 8, and XCD x takes one eighth of the active
// (tile, row block) items, a contiguous range in order: the tiles of one expert, and the
// row blocks of one token tile, meet in the same L2.  The ranges are set from the active
// tile count on the device, so the padding of the tile list past its last tile (the grid
// is sized for the most tiles a batch can have) leaves every XCD the same share of work.
#include "mfma_stream.h"

namespace moe {

constexpr int GT_TOK = 64;    // routed rows per tile
constexpr int GT_RS = 128;    // LDS row of a step's 128 code bytes, 16-byte chunk c at c ^ gt_swz(row)
// The activation tile moves through LDS in chunks of GT_CHUNK_ROWSTEPS rows x steps: a
// tile padded to R = 16, 32 or 64 rows stages 128 / R K steps per chunk, so a tile with
// few rows waits for its activations less often.  (64 row-steps per chunk measured the
// same; four blocks per CU would need the kernels in 128 VGPRs, and they take about 200.)
// One step of R rows in LDS: hi codes [R][GT_RS], lo codes [R][GT_RS], hi scales [R][4],
// lo scales [R][4].
constexpr int GT_CHUNK_ROWSTEPS = 128;
// The chunk swizzle.  gfx950 serves a wave's 16-byte LDS reads in four passes of 16
// lanes, lanes 0-7 with 24-31, 8-15 with 16-23 (and the same 32 higher); a pass is free
// of bank conflicts when its 16 lanes touch the 16 four-bank groups once each (measured
// with SQ_LDS_BANK_CONFLICT on single-wave kernels with chosen lane-to-address maps).
// Lane l of a matrix-core read takes row l mod 32: with chunk c of row m at c ^ (m/2 mod 8)
// each pass reads 16 distinct groups, and the row-order writes (8 lanes per row) are
// free for any swizzle, two rows of different parity sharing a pass.
__host__ __device__ constexpr int gt_swz(int m) { return (m >> 1) & 7; }
__host__ __device__ constexpr int gt_step_bytes(int R) { return 2 * R * GT_RS + 2 * R * 4; }
constexpr int GT_BUF_BYTES = (GT_CHUNK_ROWSTEPS / GT_TOK) * gt_step_bytes(GT_TOK);
static_assert((GT_CHUNK_ROWSTEPS / 16) * gt_step_bytes(16) == GT_BUF_BYTES &&
                  (GT_CHUNK_ROWSTEPS / 32) * gt_step_bytes(32) == GT_BUF_BYTES,
              "every chunk shape fills the same buffer");
// Each chunk goes from memory straight into LDS (global_load_lds_dwordx4 and _dword: lane
// i of a wave writes what it loads to LDS at the instruction's base + 16 i, or + 4 i, so
// the swizzle is applied on the source side), with no staging registers.  A chunk of a
// tile padded to R rows holds CH = 128 / R K steps; per step, TERMS code planes of R rows
// x 128 bytes and the scale dwords (TERMS = 2: the two exact e4m3 terms of bf16
// activations; TERMS = 1: the MXFP8 mode, whose second term is zero and is neither moved
// nor multiplied).  Its 16 TERMS code blocks of 1 KB (8 rows of one step and term) go four
// to a wave, block j = 4 u + wave for the wave's u-th load, so a lane's rows are
// 8 wave + lane / 8 plus 32 (u / (R / 32)) mod 2 at R = 64; its 128 TERMS scale bytes lie
// in one step.  The loads are counted by vmcnt like any other: the chunk's last reader
// waits for them before the barrier that hands the buffer over (gt_wait_barrier).
template <int TERMS, int R>
struct GtDma {
  static constexpr int CH = GT_CHUNK_ROWSTEPS / R;  // K steps per chunk
  static constexpr int RB = R / 8;                   // code blocks per step and term
  static constexpr int NA = RB / 4;                  // distinct rows of a lane's code loads
  static constexpr int NU = 4 * TERMS;               // code loads per wave and chunk
  static constexpr int WPS = R / 32;                 // waves sharing one step's scale bytes
  int64_t src[NA];   // srow[m] * K + 16 * ((lane mod 8) ^ gt_swz(m)), m = 32 a + 8 wave + lane / 8
  int64_t ssrc;      // srow[m_s] * (K / 32): the lane's scale dword (lanes < 32 TERMS)
  const uint8_t* sbase;  // its scale plane (hi or lo)
  int ss;            // step of the wave's scale bytes within the chunk
  int soff;          // their LDS offset within the step
};

template <int TERMS, int R>
__device__ __forceinline__ GtDma<TERMS, R> gt_dma_setup(const QRows& q, const int64_t* srow, int K, int wave,
                                                       int lane) {
  using D = GtDma<TERMS, R>;
  D t;
#pragma unroll
  for (int a = 0; a < D::NA; ++a) {
    const int m = 32 * a + 8 * wave + (lane >> 3);
    t.src[a] = srow[m] * K + 16 * ((lane & 7) ^ gt_swz(m));
  }
  // scale bytes of the wave: step wave / WPS, bytes 128 TERMS (wave mod WPS) + 4 lane of
  // that step's [hi R x 4][lo R x 4]
  t.ss = wave / D::WPS;
  t.soff = 2 * R * GT_RS + 128 * TERMS * (wave % D::WPS);
  const int o = 128 * TERMS * (wave % D::WPS) + 4 * (lane < 32 * TERMS ? lane : 0);
  const int term = o / (4 * R), ms = (o % (4 * R)) / 4;
  t.sbase = term ? q.slo : q.shi;
  t.ssrc = srow[ms] * (K / 32);
  return t;
}

// Issues the loads of chunk c (steps CH c .. CH c + CH - 1) into buf: NU code loads and
// one scale load per wave.  Steps past the end re-read the last step (never used).  buf
// and wave are wave-uniform.  The empty asm keeps the compiler from moving later memory
// operations above these loads, so the loads counted after them by gt_wait_barrier are
// the ones issued after them.
template <int TERMS, int R>
__device__ __forceinline__ void gt_dma(const GtDma<TERMS, R>& t, const QRows& q, int nks, int c, uint8_t* buf,
                                       int wave, int lane) {
  using D = GtDma<TERMS, R>;
  constexpr int SB = gt_step_bytes(R);
  unroll_n<D::NU>([&](auto uc) {
    constexpr int u = decltype(uc)::value;
    constexpr int s = u / (TERMS * D::RB / 4);
    constexpr int term = TERMS == 2 ? (u / (D::RB / 4)) & 1 : 0;
    constexpr int a = u % D::NA;
    const int ks0 = D::CH * c + s;
    const int ks = ks0 < nks ? ks0 : nks - 1;
    lds_dma16((term ? q.lo : q.hi) + t.src[a] + 128 * ks, buf + s * SB + term * R * GT_RS + (4 * a + wave) * 1024);
  });
  if (lane < 32 * TERMS) {
    const int ks0 = D::CH * c + t.ss;
    const int ks = ks0 < nks ? ks0 : nks - 1;
    lds_dma4(t.sbase + t.ssrc + 4 * ks, buf + t.ss * SB + t.soff);
  }
  asm volatile("" ::: "memory");
}

// Waits until at most N of this wave's memory loads are outstanding (N: the loads it
// issued after the chunk's gt_dma), then the block barrier that publishes the chunk.
template <int N>
__device__ __forceinline__ void gt_wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// The active tile count follows the tile list (gtiles[max_gtiles]), set by gemm_tiles_kernel.
__device__ __forceinline__ int gt_count(const int4* gtiles, int max_gtiles) {
  return *reinterpret_cast<const int*>(gtiles + max_gtiles);
}

// The item of block b: item lo + b / 8 of XCD x = b mod 8's range [x W / 8, (x + 1) W / 8)
// of the W = nitems active items, if the range holds that many.
__device__ __forceinline__ bool gt_block_item(int64_t nitems, int& lb) {
  const int x = blockIdx.x & 7;
  const int lo = (int)(nitems * x / 8), hi = (int)(nitems * (x + 1) / 8);
  lb = lo + (int)(blockIdx.x >> 3);
  return lb < hi;
}

// (tile, row block) of logical block lb.  Tiles go in groups of GT_GROUP consecutive
// tiles (the tiles of a popular expert are consecutive in the list), and within a group
// row block by row block: the group's blocks for one row block run together on one XCD,
// so a weight row block fetched for the first tile of an expert is served from that XCD's
// L2 to the others, while the group's activations (GT_GROUP x 64 rows, about 1.8 MB of
// two-term rows at K = 3584) stay in L2 across its row blocks.  Tiles past the last full
// group go tile by tile.  A bijection of [0, ntiles x nrt).
constexpr int GT_GROUP = 4;
__device__ __forceinline__ void gt_tile_of(int lb, int ntiles, int nrt, int& ti, int& rt) {
  const int full = ntiles / GT_GROUP * GT_GROUP * nrt;  // blocks in full groups
  if (lb < full) {
    const int g = lb / (GT_GROUP * nrt), w = lb - g * (GT_GROUP * nrt);
    rt = w / GT_GROUP;
    ti = g * GT_GROUP + (w - rt * GT_GROUP);
  } else {
    const int l2 = lb - full;
    ti = ntiles / GT_GROUP * GT_GROUP + l2 / nrt;
    rt = l2 - (l2 / nrt) * nrt;
  }
}

// ------------------------------------------------------------ operands

template <int N>
using f32xN = float __attribute__((ext_vector_type(N)));
typedef f32xN<16> f32x16;

template <int OPSEL_B>
__device__ __forceinline__ f32x16 mx_mfma32(const i32x8& a, const i32x8& b, f32x16 c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0 /*A: fp8 e4m3*/, 4 /*B: fp4 e2m1*/, 0, (int)sa,
                                                         OPSEL_B, (int)sb);
}

// One K step of one 32-row weight operand: the codes of the two half-steps.
struct W32Step {
  uint4 q[2];
};

// Packed layout: 32 weight rows are two 16-row groups; in group x, the 1024-byte code
// tile of step s holds row r%16, K block kb at bytes 16 (r%16 + 16 kb).  Lane l takes
// group (l%32)/16, row l%16, K block 2 hh + l/32 of the step: two 512-byte runs per load.
// Scale tile t (256 bytes) holds, at byte 4 (r%16 + 16 kb) + j, step 4 t + j: one dword
// per half-step serves four steps (the instruction's scale select picks the byte).
struct W32Packed {
  const uint8_t* c;
  const uint8_t* s;
  int nsc;
  struct Scales {
    uint32_t d[2];  // half-steps 0 and 1 of steps 4 G .. 4 G + 3
  };
  __device__ static W32Packed make(const uint8_t* blob, int e, int L, int F, int mat, int pair, int lane) {
    const int K = mat == MAT_DOWN ? F : L;
    const int64_t gu = (int64_t)(F / 16) * packed_group_bytes(L);
    const uint8_t* m =
        blob + (int64_t)e * packed_expert_bytes(L, F) + (mat == MAT_GATE ? 0 : mat == MAT_UP ? gu : 2 * gu);
    const uint8_t* grp = m + (int64_t)(2 * pair + ((lane & 31) >> 4)) * packed_group_bytes(K);
    const int pos = (lane & 15) + 16 * (lane >> 5);  // row in group + 16 x (K block within the half-step)
    W32Packed w;
    w.c = grp + 16 * pos;
    w.s = grp + (int64_t)(K / 128) * 1024 + 4 * pos;
    w.nsc = (K / 128 + 3) / 4;
    return w;
  }
  __device__ __forceinline__ W32Step step(int ks) const {
    W32Step r;
    const uint8_t* cs = c + 1024 * ks;
    r.q[0] = *reinterpret_cast<const uint4*>(cs);
    r.q[1] = *reinterpret_cast<const uint4*>(cs + 512);
    return r;
  }
  // the scales of steps 4 G .. 4 G + 3 (G < nsc)
  __device__ __forceinline__ Scales group(int G) const {
    const uint8_t* ss = s + 256 * G;
    return Scales{{*reinterpret_cast<const uint32_t*>(ss), *reinterpret_cast<const uint32_t*>(ss + 128)}};
  }
  template <int J>
  __device__ __forceinline__ static uint32_t scale(const Scales& sc, int hh) { return sc.d[hh]; }
  static constexpr int opsel(int j) { return j & 3; }
};

// Checkpoint record: row 32 pair + l%32, K block 4 s + 2 hh + l/32 of step s is bytes
// 64 s + 32 hh + 16 (l/32) of the row's codes; its scale is byte 4 s + 2 hh + l/32 of the
// row's scales, moved to the low byte (one dword per step).
struct W32Record {
  const uint8_t* c;
  const uint8_t* s;
  int sh;  // 8 x (l/32)
  struct Scales {
    uint32_t d[4];  // steps 4 G .. 4 G + 3: the four K-block scales of each
  };
  __device__ static W32Record make(const uint8_t* blob, int e, int L, int F, int mat, int pair, int lane) {
    const int64_t mbytes = (int64_t)F * L / 2 + (int64_t)F * L / 32;
    const int K = mat == MAT_DOWN ? F : L;
    const uint8_t* m = blob + (int64_t)e * 3 * mbytes + mat * mbytes;
    const int64_t row = 32 * pair + (lane & 31);
    W32Record w;
    w.c = m + row * (K / 2) + 16 * (lane >> 5);
    w.s = m + (int64_t)(mat == MAT_DOWN ? L : F) * (K / 2) + row * (K / 32);
    w.sh = 8 * (lane >> 5);
    return w;
  }
  __device__ __forceinline__ W32Step step(int ks) const {
    W32Step r;
    const uint8_t* cs = c + 64 * ks;
    r.q[0] = *reinterpret_cast<const uint4*>(cs);
    r.q[1] = *reinterpret_cast<const uint4*>(cs + 32);
    return r;
  }
  // the scales of steps 4 G .. 4 G + 3; a step past the last (K / 128 not a multiple of 4)
  // re-reads the last one and is never used
  __device__ __forceinline__ Scales group(int G, int nks) const {
    Scales r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ks = 4 * G + i < nks ? 4 * G + i : nks - 1;
      r.d[i] = *reinterpret_cast<const uint32_t*>(s + 4 * ks);
    }
    return r;
  }
  template <int J>
  __device__ __forceinline__ uint32_t scale(const Scales& sc, int hh) const { return sc.d[J & 3] >> (sh + 16 * hh); }
  static constexpr int opsel(int) { return 0; }
};

template <class W>
__device__ __forceinline__ typename W::Scales w32_group(const W& w, int G, int nks);
template <>
__device__ __forceinline__ W32Packed::Scales w32_group(const W32Packed& w, int G, int nks) {
  return w.group(G < w.nsc ? G : w.nsc - 1);
}
template <>
__device__ __forceinline__ W32Record::Scales w32_group(const W32Record& w, int G, int nks) {
  const int ng = (nks + 3) / 4;
  return w.group(G < ng ? G : ng - 1, nks);
}

__device__ __forceinline__ i32x8 as_b32(const uint4& q) {
  i32x8 b;
  b[0] = (int)q.x; b[1] = (int)q.y; b[2] = (int)q.z; b[3] = (int)q.w;
  b[4] = 0; b[5] = 0; b[6] = 0; b[7] = 0;
  return b;
}

// activation operand of half-step hh of chunk step s, tile row m, for lane group g
template <int TERMS, int R>
__device__ __forceinline__ void gt32_read(i32x8& hi, i32x8& lo, uint32_t& shi, uint32_t& slo, const uint8_t* buf,
                                          int s, int m, int g, int hh) {
  const uint8_t* st = buf + s * gt_step_bytes(R);
  const int c0 = 16 * ((4 * hh + g) ^ gt_swz(m)), c1 = 16 * ((4 * hh + 2 + g) ^ gt_swz(m));
  const uint4 h0 = *reinterpret_cast<const uint4*>(st + m * GT_RS + c0);
  const uint4 h1 = *reinterpret_cast<const uint4*>(st + m * GT_RS + c1);
  hi[0] = (int)h0.x; hi[1] = (int)h0.y; hi[2] = (int)h0.z; hi[3] = (int)h0.w;
  hi[4] = (int)h1.x; hi[5] = (int)h1.y; hi[6] = (int)h1.z; hi[7] = (int)h1.w;
  shi = st[2 * R * GT_RS + m * 4 + 2 * hh + g];
  if constexpr (TERMS == 2) {
    const uint4 l0 = *reinterpret_cast<const uint4*>(st + R * GT_RS + m * GT_RS + c0);
    const uint4 l1 = *reinterpret_cast<const uint4*>(st + R * GT_RS + m * GT_RS + c1);
    lo[0] = (int)l0.x; lo[1] = (int)l0.y; lo[2] = (int)l0.z; lo[3] = (int)l0.w;
    lo[4] = (int)l1.x; lo[5] = (int)l1.y; lo[6] = (int)l1.z; lo[7] = (int)l1.w;
    slo = st[2 * R * GT_RS + R * 4 + m * 4 + 2 * hh + g];
  }
}

// The K loop of one tile padded to R = 32 or 64 rows: acc[q][tt] += A(sub-tile tt) x W_q^T.
// Every load is issued with clamped indices and only the math is guarded, so the loads in
// flight are the same on every path and the compiler's waits for them are exact.
template <class W, int NMAT, int PF, int TERMS, int R>
__device__ __forceinline__ void gt32_mainloop(const W (&w)[NMAT], const QRows& q, const int64_t* srow, int n, int K,
                                              uint8_t* lds, f32x16 (&acc)[NMAT][R / 32]) {
  using D = GtDma<TERMS, R>;
  constexpr int CH = D::CH;
  static_assert(16 % PF == 0 && 16 % CH == 0, "ring and chunks repeat every 16 steps");
  const int lane = lane_id(), g = lane >> 5, nl = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / WAVE));
  const int nks = K / 128, nc = (nks + 15) / 16, nch = (nks + CH - 1) / CH;
  const int ntt = (n + 31) / 32;  // token sub-tiles holding rows
  const D dt = gt_dma_setup<TERMS, R>(q, srow, K, wave, lane);
  gt_dma<TERMS, R>(dt, q, nks, 0, lds, wave, lane);
  W32Step ring[NMAT][PF];
#pragma unroll
  for (int d = 0; d < PF; ++d)
#pragma unroll
    for (int mq = 0; mq < NMAT; ++mq) ring[mq][d] = w[mq].step(d < nks ? d : nks - 1);
  // scales in groups of 4 steps, the next group loaded at the start of the current one
  typename W::Scales sc[NMAT][2];
#pragma unroll
  for (int mq = 0; mq < NMAT; ++mq) sc[mq][0] = w32_group(w[mq], 0, nks);
  gt_wait_barrier<PF * NMAT * 2>();  // chunk 0: the weight ring's loads were issued after it
  for (int cb = 0; cb < nc; ++cb) {
    unroll16([&](auto jc) {
      constexpr int J = decltype(jc)::value;
      constexpr int SG = (J >> 2) & 1;  // parity of the step's scale group (4 groups per 16 steps)
      const int ks = 16 * cb + J;
      const int ch = ks / CH;
      const uint8_t* buf = lds + (ch & 1) * GT_BUF_BYTES;
      if constexpr ((J & 3) == 0) {
#pragma unroll
        for (int mq = 0; mq < NMAT; ++mq) sc[mq][SG ^ 1] = w32_group(w[mq], (ks >> 2) + 1, nks);
      }
      W32Step cw[NMAT];
#pragma unroll
      for (int mq = 0; mq < NMAT; ++mq) {
        cw[mq] = ring[mq][J % PF];
        ring[mq][J % PF] = w[mq].step(ks + PF < nks ? ks + PF : nks - 1);
      }
      if (ks < nks) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int tt = 0; tt < R / 32; ++tt) {
            if (tt >= ntt) continue;  // token sub-tile past the tile's rows
            i32x8 ahi, alo;
            uint32_t shi, slo;
            gt32_read<TERMS, R>(ahi, alo, shi, slo, buf, J % CH, 32 * tt + nl, g, hh);
#pragma unroll
            for (int mq = 0; mq < NMAT; ++mq) {
              const i32x8 b = as_b32(cw[mq].q[hh]);
              const uint32_t sw = w[mq].template scale<J>(sc[mq][SG], hh);
              acc[mq][tt] = mx_mfma32<W::opsel(J)>(ahi, b, acc[mq][tt], shi, sw);
              if constexpr (TERMS == 2) acc[mq][tt] = mx_mfma32<W::opsel(J)>(alo, b, acc[mq][tt], slo, sw);
            }
          }
          // Chunk ch + 1 goes into the buffer chunk ch - 1 left (every wave passed the
          // barrier after it), issued within the chunk's first step: the compiler's waits
          // for the weight loads issued before it also wait for these loads, and the
          // first such wait comes a step later.
          if constexpr (J % CH == 0)
            if (hh == 0 && ch + 1 < nch)
              gt_dma<TERMS, R>(dt, q, nks, ch + 1, lds + ((ch + 1) & 1) * GT_BUF_BYTES, wave, lane);
        }
      }
      if constexpr (J % CH == CH - 1) {
        // chunk ch + 1 is in LDS once the loads issued after it, the weight loads of the
        // chunk's later CH - 1 steps, are all that may be outstanding
        gt_wait_barrier<(CH - 1) * NMAT * 2>();
      }
    });
  }
}

// weight steps in flight per operand: deeper for 32-row tiles (half the accumulators)
template <int TERMS, int R>
constexpr int gt32_pf() { return R == 32 ? 4 : 2; }

template <class W> struct W32Of;
template <> struct W32Of<PackedW> { using type = W32Packed; };
template <> struct W32Of<RecordW> { using type = W32Record; };

constexpr int GT32_FROWS = 128;  // gate/up: F rows per block (4 waves x 32, gate and up)

// Gate/up of one tile padded to R rows: the K loop, then a = bf16(silu(g) u) into an LDS
// tile [64][GT32_FROWS + 1] (the activation buffers are free by then) and its two-term
// requantisation into aq.
template <class W, int TERMS, int R>
__device__ __forceinline__ void gateup32_tile(const MxArgs& p, int e, int rt, int n, const int64_t* srow,
                                              const int* sslot, uint8_t* lds) {
  using WS = typename W32Of<W>::type;
  const int F = p.F, L = p.L;
  const int lane = lane_id(), wave = threadIdx.x / WAVE, g = lane >> 5, nl = lane & 31;
  const int pair = rt * (GT32_FROWS / 32) + wave;
  const WS w[2] = {WS::make(p.blob, e, L, F, MAT_GATE, pair, lane), WS::make(p.blob, e, L, F, MAT_UP, pair, lane)};
  f32x16 acc[2][R / 32];
#pragma unroll
  for (int mq = 0; mq < 2; ++mq)
#pragma unroll
    for (int tt = 0; tt < R / 32; ++tt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mq][tt][v] = 0.f;
  gt32_mainloop<WS, 2, gt32_pf<TERMS, R>(), TERMS, R>(w, p.hq, srow, n, L, lds, acc);
  // the GLU of every accumulator row (rows past n are computed and never read), then the
  // tile into LDS [64 tokens][GT32_FROWS + 1] once the activation buffers are free
  float* at = reinterpret_cast<float*>(lds);
  constexpr int AS = GT32_FROWS + 1;
  static_assert(64 * AS * 4 + 2 * 64 * 4 <= 2 * GT_BUF_BYTES, "the GLU tile and its scale bytes fit the chunk buffers");
  uint8_t* sc = lds + 64 * AS * 4;           // scale bytes [term][64 tokens][4 blocks]
  const int fl = 32 * wave + nl, f = rt * GT32_FROWS + fl;
  uint16_t ab[R / 32][16];
#pragma unroll
  for (int tt = 0; tt < R / 32; ++tt)
#pragma unroll
    for (int v = 0; v < 16; ++v) ab[tt][v] = glu_bf16(acc[0][tt][v], acc[1][tt][v]);
  if (p.a_bf16) {
#pragma unroll
    for (int tt = 0; tt < R / 32; ++tt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = 32 * tt + 8 * (v >> 2) + 4 * g + (v & 3);
        if (m < n) p.a_bf16[(int64_t)sslot[m] * F + f] = ab[tt][v];
      }
  }
  lds_barrier();  // the activation buffers are free
  float* atl = at + (4 * g) * AS + fl;
#pragma unroll
  for (int tt = 0; tt < R / 32; ++tt)
#pragma unroll
    for (int v = 0; v < 16; ++v) atl[(32 * tt + 8 * (v >> 2) + (v & 3)) * AS] = bf16f(ab[tt][v]);
  lds_barrier();
  for (int it = threadIdx.x; it < R * (GT32_FROWS / 8); it += blockDim.x) {
    // a quad of lanes per (token, scale block): R tokens x 4 blocks x 4 lanes
    const int m = it >> 4, blk = (it >> 2) & 3, sub = it & 3;
    if (m < n) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = at[m * AS + 32 * blk + 8 * sub + i];
      uint32_t hi[2], lo[2], shi, slo;
      quantize_quad8_fmt(v, hi, lo, shi, slo, p.mxfp8 != 0);
      const int64_t off = (int64_t)sslot[m] * F + rt * GT32_FROWS + 32 * blk + 8 * sub;
      *reinterpret_cast<uint2*>(p.aq.hi + off) = make_uint2(hi[0], hi[1]);
      *reinterpret_cast<uint2*>(p.aq.lo + off) = make_uint2(lo[0], lo[1]);
      if (sub == 0) {
        sc[m * 4 + blk] = (uint8_t)shi;
        sc[256 + m * 4 + blk] = (uint8_t)slo;
      }
    }
  }
  lds_barrier();
  // the 4 scale bytes of a token and term in one store
  if (threadIdx.x < 2 * R) {
    const int m = threadIdx.x >> 1, term = threadIdx.x & 1;
    if (m < n) {
      const int64_t soff = (int64_t)sslot[m] * (F / 32) + (rt * GT32_FROWS) / 32;
      *reinterpret_cast<uint32_t*>((term ? p.aq.slo : p.aq.shi) + soff) =
          *reinterpret_cast<const uint32_t*>(sc + 256 * term + 4 * m);
    }
  }
}

template <class W, int TERMS>
__global__ void __launch_bounds__(256, 2) gateup_gemm32_kernel(MxArgs p, const int4* __restrict__ gtiles,
                                                                int max_gtiles) {
  clock_begin(p.clock);
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int64_t srow[GT_TOK];
  __shared__ int sslot[GT_TOK];
  const int nrt = p.F / GT32_FROWS, ntiles = gt_count(gtiles, max_gtiles);
  int lb;
  if (gt_block_item((int64_t)ntiles * nrt, lb)) {
    int ti, rt;
    gt_tile_of(lb, ntiles, nrt, ti, rt);
    const int4 tile = gtiles[ti];
    const int e = tile.x, r0 = tile.y, n = tile.z;
    for (int m = threadIdx.x; m < GT_TOK; m += blockDim.x) {
      const int sl = m < n ? p.perm[r0 + m] : 0;
      sslot[m] = sl;
      srow[m] = sl / p.k;
    }
    __syncthreads();
    if (n <= 32)
      gateup32_tile<W, TERMS, 32>(p, e, rt, n, srow, sslot, lds);
    else
      gateup32_tile<W, TERMS, 64>(p, e, rt, n, srow, sslot, lds);
  }
  clock_end(p.clock);
}

// Down of one tile: y[slot][l] fp32.  Each wave holds NG 32-row groups of the down matrix
// (groups 4 q + wave of the block's 4 NG), so a block covers 128 NG latent rows.
template <class W, int TERMS, int NG, int R>
__device__ __forceinline__ void down32_tile(const MxArgs& p, int e, int rt, int n, const int64_t* srow, uint8_t* lds) {
  using WS = typename W32Of<W>::type;
  const int F = p.F, L = p.L;
  const int lane = lane_id(), wave = threadIdx.x / WAVE, g = lane >> 5, nl = lane & 31;
  WS w[NG];
#pragma unroll
  for (int q = 0; q < NG; ++q) w[q] = WS::make(p.blob, e, L, F, MAT_DOWN, rt * 4 * NG + 4 * q + wave, lane);
  f32x16 acc[NG][R / 32];
#pragma unroll
  for (int q = 0; q < NG; ++q)
#pragma unroll
    for (int tt = 0; tt < R / 32; ++tt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[q][tt][v] = 0.f;
  gt32_mainloop<WS, NG, gt32_pf<TERMS, R>(), TERMS, R>(w, p.aq, srow, n, F, lds, acc);
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    const int l = (rt * 4 * NG + 4 * q + wave) * 32 + nl;
#pragma unroll
    for (int tt = 0; tt < R / 32; ++tt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = 32 * tt + 8 * (v >> 2) + 4 * g + (v & 3);
        if (m < n) p.y[srow[m] * L + l] = acc[q][tt][v];
      }
  }
  if (p.sal) {
    // REAP partials: the block's y tile goes to LDS (the activation chunks are free once
    // every wave is past the K loop); per routed row, four threads sum y^2 over a quarter
    // of the block's latent rows each, in row order, and add the quarters in a fixed order
    constexpr int YS = 128 * NG + 4;
    static_assert(64 * YS * 4 <= 2 * GT_BUF_BYTES, "the y tile fits the chunk buffers");
    float* yt = reinterpret_cast<float*>(lds);
    lds_barrier();
#pragma unroll
    for (int q = 0; q < NG; ++q)
#pragma unroll
      for (int tt = 0; tt < R / 32; ++tt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = 32 * tt + 8 * (v >> 2) + 4 * g + (v & 3);
          if (m < n) yt[m * YS + (4 * q + wave) * 32 + nl] = acc[q][tt][v];
        }
    lds_barrier();
    const int m = threadIdx.x >> 2, part = threadIdx.x & 3;
    double sq = 0.0;
    if (m < n)
      for (int i = part * 32 * NG; i < (part + 1) * 32 * NG; ++i) {
        const double v = (double)yt[m * YS + i];
        sq += v * v;
      }
    sq += __shfl_xor(sq, 1);  // (q0 + q1), (q2 + q3): the same sum on both lanes of a pair
    sq += __shfl_xor(sq, 2);  // then their sum
    if (part == 0 && m < n) p.sal[srow[m] * p.sal_chunks + rt] = sq;
  }
}

template <class W, int TERMS, int NG>
__global__ void __launch_bounds__(256, 2) down_gemm32_kernel(MxArgs p, const int4* __restrict__ gtiles,
                                                              int max_gtiles) {
  clock_begin(p.clock);
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int64_t srow[GT_TOK];
  const int nrt = p.L / (128 * NG), ntiles = gt_count(gtiles, max_gtiles);
  int lb;
  if (gt_block_item((int64_t)ntiles * nrt, lb)) {
    int ti, rt;
    gt_tile_of(lb, ntiles, nrt, ti, rt);
    const int4 tile = gtiles[ti];
    const int e = tile.x, r0 = tile.y, n = tile.z;
    for (int m = threadIdx.x; m < GT_TOK; m += blockDim.x) srow[m] = m < n ? p.perm[r0 + m] : 0;
    __syncthreads();
    if (n <= 32)
      down32_tile<W, TERMS, NG, 32>(p, e, rt, n, srow, lds);
    else
      down32_tile<W, TERMS, NG, 64>(p, e, rt, n, srow, lds);
  }
  clock_end(p.clock);
}

// Tiles of GT_TOK routed rows per active expert, in expert order: gtiles[0, ntiles) =
// {expert, first row in perm, rows, 0}; gtiles[ntiles, max_gtiles) = {-1, 0, 0, 0}; then
// the tile count.
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
  if (tid == 0) *reinterpret_cast<int*>(gtiles + max_gtiles) = total;
}

int64_t gemm_max_tiles(int64_t rows, int32_t E) { return ceil_div(rows, GT_TOK) + (rows < E ? rows : E); }
size_t gemm_tiles_bytes(int64_t rows, int32_t E) { return (size_t)gemm_max_tiles(rows, E) * 16 + GEMM_TILES_TAIL_BYTES; }

hipError_t launch_gemm_tiles(const int32_t* counts, const int32_t* offsets, int32_t E, int4* gtiles,
                             int64_t max_gtiles, hipStream_t st) {
  if (E > 16 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_tiles_kernel, dim3(1), dim3(1024), 0, st, counts, offsets, E, gtiles, (int)max_gtiles);
  return hipGetLastError();
}

template <class W, int TERMS>
static hipError_t gateup_gemm32_go(const MxArgs& p, const int4* gtiles, int64_t max_gtiles, unsigned grid,
                                   hipStream_t st, const KernelEvents& ev) {
  static const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gateup_gemm32_kernel<W, TERMS>),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, 2 * GT_BUF_BYTES);
  if (e != hipSuccess) return e;
  return dispatch(ev, gateup_gemm32_kernel<W, TERMS>, dim3(grid), dim3(256), 2 * GT_BUF_BYTES, st, p, gtiles,
                  (int)max_gtiles);
}

template <class W, int TERMS, int NG>
static hipError_t down_gemm32_go(const MxArgs& p, const int4* gtiles, int64_t max_gtiles, unsigned grid,
                                 hipStream_t st, const KernelEvents& ev) {
  static const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&down_gemm32_kernel<W, TERMS, NG>),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, 2 * GT_BUF_BYTES);
  if (e != hipSuccess) return e;
  return dispatch(ev, down_gemm32_kernel<W, TERMS, NG>, dim3(grid), dim3(256), 2 * GT_BUF_BYTES, st, p, gtiles,
                  (int)max_gtiles);
}

template <int NG>
static hipError_t down_gemm32_ng(const MxArgs& p, const int4* gtiles, int64_t max_gtiles, hipStream_t st,
                                 const KernelEvents& ev) {
  const int64_t grid64 = (max_gtiles * (p.L / (128 * NG)) + 7) / 8 * 8;  // the most items a batch can have
  if (grid64 > 0x7FFFFFFF) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)grid64;
  if (p.packed)
    return p.mxfp8 ? down_gemm32_go<PackedW, 1, NG>(p, gtiles, max_gtiles, grid, st, ev)
                   : down_gemm32_go<PackedW, 2, NG>(p, gtiles, max_gtiles, grid, st, ev);
  return p.mxfp8 ? down_gemm32_go<RecordW, 1, NG>(p, gtiles, max_gtiles, grid, st, ev)
                 : down_gemm32_go<RecordW, 2, NG>(p, gtiles, max_gtiles, grid, st, ev);
}

hipError_t launch_gateup_gemm(const MxArgs& p, const int4* gtiles, int64_t max_gtiles, hipStream_t st,
                              const KernelEvents& ev) {
  if (p.T == 0) return hipSuccess;
  if (p.F % GT32_FROWS || p.L % 128) return hipErrorInvalidValue;
  const int64_t grid64 = (max_gtiles * (p.F / GT32_FROWS) + 7) / 8 * 8;  // the most items a batch can have
  if (grid64 > 0x7FFFFFFF) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)grid64;
  if (p.packed)
    return p.mxfp8 ? gateup_gemm32_go<PackedW, 1>(p, gtiles, max_gtiles, grid, st, ev)
                   : gateup_gemm32_go<PackedW, 2>(p, gtiles, max_gtiles, grid, st, ev);
  return p.mxfp8 ? gateup_gemm32_go<RecordW, 1>(p, gtiles, max_gtiles, grid, st, ev)
                 : gateup_gemm32_go<RecordW, 2>(p, gtiles, max_gtiles, grid, st, ev);
}

int32_t down_gemm_sal_chunks(int32_t L) { return L / (L % 256 == 0 ? 256 : 128); }

hipError_t launch_down_gemm(const MxArgs& p, const int4* gtiles, int64_t max_gtiles, hipStream_t st,
                            const KernelEvents& ev) {
  if (p.T == 0) return hipSuccess;
  if (p.L % 128 || p.F % 128) return hipErrorInvalidValue;
  if (p.sal && p.sal_chunks != down_gemm_sal_chunks(p.L)) return hipErrorInvalidValue;
  return p.L % 256 == 0 ? down_gemm32_ng<2>(p, gtiles, max_gtiles, st, ev)
                        : down_gemm32_ng<1>(p, gtiles, max_gtiles, st, ev);
}

}  // namespace moe
