// Shared pieces of the expert kernels on the CDNA4 block-scaled matrix cores: the
// v_mfma_scale_f32_16x16x128_f8f6f4 wrapper, the two weight streams (checkpoint record
// and packed layout) and the staged activation operand.
//
// Operand layout of v_mfma_scale_f32_16x16x128_f8f6f4 (measured on gfx950): lane l
// works on row/column l%16 and K block g = l/16; an FP4 operand holds K = 32g..32g+31
// (low nibble first), an FP8 operand holds K = 16g..16g+15 in its first four
// registers and 64+16g..64+16g+15 in the last four; lane (r + 16 b) supplies the
// scale of row/column r, K block b for both operands, the byte of its scale register
// chosen by the instruction's scale select; the result register j of lane l is
// D[4(l/16)+j][l%16].
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int OPSEL_B>
__device__ __forceinline__ f32x4 mx_mfma(const i32x8& a, const i32x8& b, f32x4 c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0 /*A: fp8 e4m3*/, 4 /*B: fp4 e2m1*/, 0,
                                                          (int)sa, OPSEL_B, (int)sb);
}

__device__ __forceinline__ i32x8 as_b(const uint4& q) {
  i32x8 b;
  b[0] = (int)q.x; b[1] = (int)q.y; b[2] = (int)q.z; b[3] = (int)q.w;
  b[4] = 0; b[5] = 0; b[6] = 0; b[7] = 0;
  return b;
}

// --------------------------------------------------------------- weight streams

// Scale bytes of one 16-step block of K for the lane (see the two streams).
struct SBlock {
  uint32_t d[4];
};

enum { MAT_GATE = 0, MAT_UP = 1, MAT_DOWN = 2 };

// Checkpoint record: per expert gate [F][L], up [F][L], down [L][F], each its codes
// row-major then its e8m0 scales row-major.
struct RecordW {
  const uint8_t* c;  // codes of the lane's row + 16 g
  const uint8_t* s;  // scales of the lane's row
  int nsb, n, g;     // scale bytes per row; lane row and K block

  // matrix `mat` of expert e, rows 16 grp .. 16 grp + 15
  __device__ static RecordW make(const uint8_t* blob, int e, int L, int F, int mat, int grp, int lane) {
    const int64_t mbytes = (int64_t)F * L / 2 + (int64_t)F * L / 32;
    const int K = mat == MAT_DOWN ? F : L;
    const uint8_t* m = blob + (int64_t)e * 3 * mbytes + mat * mbytes;
    const int64_t row = 16 * grp + (lane & 15);
    RecordW w;
    w.n = lane & 15;
    w.g = lane >> 4;
    w.nsb = K / 32;
    w.c = m + row * (K / 2) + 16 * w.g;
    w.s = m + (int64_t)(mat == MAT_DOWN ? L : F) * (K / 2) + row * (K / 32);
    return w;
  }
  __device__ __forceinline__ uint4 load(int ks) const { return load_nt16(c + 64 * ks); }
  // lane (n, g) takes bytes 64 blk + 16 g .. +15 of row n: dword i holds the four block
  // scales of step 16 blk + 4 g + i.  All four loads are issued (a position past the row
  // reloads its last dword and is replaced by 127s), so every path issues the same loads.
  __device__ __forceinline__ void sblock(SBlock& b, int blk) const {
    const int off = 64 * blk + 16 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int o = off + 4 * i;
      const uint32_t v = *reinterpret_cast<const uint32_t*>(s + (o < nsb ? o : nsb - 4));
      b.d[i] = o < nsb ? v : 0x7F7F7F7Fu;
    }
  }
  // scale of step 16 blk + J, from the lane of the same row that holds it
  template <int J>
  __device__ __forceinline__ uint32_t scale(const SBlock& b) const {
    return (uint32_t)__shfl((int)b.d[J & 3], n + 16 * (J >> 2)) >> (8 * g);
  }
  static constexpr int opsel(int) { return 0; }
};

// Packed layout (moe_pack_experts): a matrix of R rows and K columns is R/16 row groups
// of packed_group_bytes(K): K/128 code tiles of 1024 bytes (tile s, bytes 16 l .. +15:
// row l%16 of the group, K values 128 s + 32 (l/16) .. +31), then ceil(K/512) scale
// tiles of 256 bytes (tile c, byte 4 l + j: the scale of those 32 values at step
// s = 4c + j; 127 past the last step).
struct PackedW {
  const uint8_t* c;  // code tile 0 + 16 lane
  const uint8_t* s;  // scale tile 0 + 4 lane
  int nsc;           // scale tiles

  __device__ static PackedW make(const uint8_t* blob, int e, int L, int F, int mat, int grp, int lane) {
    const int K = mat == MAT_DOWN ? F : L;
    const int64_t gu = (int64_t)(F / 16) * packed_group_bytes(L);
    const uint8_t* m =
        blob + (int64_t)e * packed_expert_bytes(L, F) + (mat == MAT_GATE ? 0 : mat == MAT_UP ? gu : 2 * gu);
    const uint8_t* grp0 = m + (int64_t)grp * packed_group_bytes(K);
    PackedW w;
    w.c = grp0 + 16 * lane;
    w.s = grp0 + (int64_t)(K / 128) * 1024 + 4 * lane;
    w.nsc = (K / 128 + 3) / 4;
    return w;
  }
  __device__ __forceinline__ uint4 load(int ks) const { return load_nt16(c + 1024 * ks); }
  // all four loads issued (a tile past the last reloads the last one), see RecordW
  __device__ __forceinline__ void sblock(SBlock& b, int blk) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * blk + i;
      const uint32_t v = *reinterpret_cast<const uint32_t*>(s + 256 * (t < nsc ? t : nsc - 1));
      b.d[i] = t < nsc ? v : 0x7F7F7F7Fu;
    }
  }
  template <int J>
  __device__ __forceinline__ uint32_t scale(const SBlock& b) const {
    return b.d[J >> 2];
  }
  static constexpr int opsel(int j) { return j & 3; }
};

// The first loads of a weight stream, in the order the first step needs them: the
// scales of steps 0..15, then PF steps of codes (an index past the last step reloads
// the last one).
//
// Every load of a stream is unconditional, with indices clamped into the matrix: the
// compiler counts loads in flight per path, and a load skipped on some path makes it
// wait for all of them (vmcnt(0)) where one step's data would do, which empties the
// prefetch ring at every step.
template <class W, int NMAT, int PF>
__device__ __forceinline__ void prime_stream(const W (&w)[NMAT], SBlock (&sb)[NMAT], uint4 (&ring)[NMAT][PF],
                                             int nks) {
#pragma unroll
  for (int q = 0; q < NMAT; ++q) w[q].sblock(sb[q], 0);
#pragma unroll
  for (int d = 0; d < PF; ++d)
#pragma unroll
    for (int q = 0; q < NMAT; ++q) ring[q][d] = w[q].load(d < nks ? d : nks - 1);
}

// ------------------------------------------------------------ staged activations

struct ALds {
  uint8_t* hi;
  uint8_t* lo;
  uint8_t* shi;
  uint8_t* slo;
};
__device__ __forceinline__ ALds alds(uint8_t* smem, int K, int rows) {
  return {smem, smem + rows * K, smem + 2 * rows * K, smem + 2 * rows * K + rows * (K / 32)};
}

// activation operand of one K step for tile row m (zero unless m < ntok)
struct AStep {
  i32x8 hi, lo;
  uint32_t shi, slo;
};
__device__ __forceinline__ void read_a(AStep& a, const ALds& d, int m, int ntok, int K, int ks, int g) {
  if (m < ntok) {
    const uint8_t* h = d.hi + m * K + 128 * ks + 16 * g;
    const uint8_t* l = d.lo + m * K + 128 * ks + 16 * g;
    const uint4 h0 = *reinterpret_cast<const uint4*>(h), h1 = *reinterpret_cast<const uint4*>(h + 64);
    const uint4 l0 = *reinterpret_cast<const uint4*>(l), l1 = *reinterpret_cast<const uint4*>(l + 64);
    a.hi[0] = (int)h0.x; a.hi[1] = (int)h0.y; a.hi[2] = (int)h0.z; a.hi[3] = (int)h0.w;
    a.hi[4] = (int)h1.x; a.hi[5] = (int)h1.y; a.hi[6] = (int)h1.z; a.hi[7] = (int)h1.w;
    a.lo[0] = (int)l0.x; a.lo[1] = (int)l0.y; a.lo[2] = (int)l0.z; a.lo[3] = (int)l0.w;
    a.lo[4] = (int)l1.x; a.lo[5] = (int)l1.y; a.lo[6] = (int)l1.z; a.lo[7] = (int)l1.w;
    a.shi = d.shi[m * (K / 32) + 4 * ks + g];
    a.slo = d.slo[m * (K / 32) + 4 * ks + g];
  } else {
    for (int i = 0; i < 8; ++i) a.hi[i] = a.lo[i] = 0;
    a.shi = a.slo = 127u;
  }
}

// a = bf16(silu(g) u) for the fp32 values g and u, evaluated in fp32: silu(g) =
// g / (1 + e^-g), as g e^g / (1 + e^g) for g < 0 so a large |g| cannot overflow.  The
// exponential is the hardware 2^x of -|g| log2(e) and the division a hardware reciprocal:
// each within a couple of fp32 ulps (the argument's rounding adds |g| 2^-24 relative), a
// few fp32 ulps in all, so the bf16 rounding of a differs from that of the exact value
// only for values within that distance of a bf16 rounding boundary (about 1 in 10^4).
// The hardware 2^x flushes results below 2^-126, so for |g| above 83 it is taken of the
// argument + 32 and the product g e^g scaled back by 2^-32 (an fp32 multiply, which keeps
// subnormal results).  NaN and infinities behave as in the exact formula: g = +inf gives
// +inf, g = -inf NaN.
__device__ __forceinline__ uint16_t glu_bf16(float g, float u) {
  const float x = -fabsf(g) * 1.44269504088896341f;  // log2 of e^-|g|
  const bool tiny = x < -120.f;
  const float e2 = __builtin_amdgcn_exp2f(tiny ? x + 32.f : x);  // e^-|g|, times 2^32 when tiny
  const float sc = tiny ? 0x1p-32f : 1.f;
  const float r = __builtin_amdgcn_rcpf(1.f + e2 * sc);
  const float s = (g >= 0.f ? g : (g * e2) * sc) * r;
  return f32_to_bf16(s * u);
}

}  // namespace moe
