// Shared device helpers for the gfx950 kernels of the MXFP4 Stable-LatentMoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "../../include/moe_layer.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

// ---------------------------------------------------------------- bf16 bits

__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.  Both results are
// formed and one is kept by a mask, so no branch is taken per value.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t nan = 0u - (uint32_t)(f != f);
  return (uint16_t)((((u | 0x00400000u) & nan) | ((u + 0x7FFFu + ((u >> 16) & 1u)) & ~nan)) >> 16);
}

// fp64 -> bf16 bits, round to nearest even in one step (no detour through fp32):
// the value is rounded to the 8-significant-bit grid of its binade (spacing 2^-133 in
// the subnormal range), overflow gives inf.
__device__ __forceinline__ uint16_t f64_to_bf16(double v) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t ex = (uint32_t)(u >> 52) & 0x7FFu;
  const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  if (ex == 0x7FFu) return (u & 0xFFFFFFFFFFFFFull) ? (uint16_t)0x7FC0 : (uint16_t)(sign | 0x7F80);
  if (ex == 0u) return sign;  // below 2^-1022: rounds to zero in bf16
  int q = (int)ex - 1023 - 7;
  if (q < -133) q = -133;
  const double step = __longlong_as_double((long long)(q + 1023) << 52);
  const double r = rint(v / step) * step;  // both operations exact; rint ties to even
  if (fabs(r) >= 0x1p128) return (uint16_t)(sign | 0x7F80);
  return (uint16_t)(__float_as_uint((float)r) >> 16);  // r has at most 8 significant bits
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }

// acc + a.lo*b.lo + a.hi*b.hi
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(b), acc, false);
}

// 1 if either bf16 half of d is subnormal (zero exponent field, nonzero fraction)
__device__ __forceinline__ uint32_t bf16x2_subnormal(uint32_t d) {
  return ((d & 0x7F80u) == 0u && (d & 0x7Fu) != 0u) | ((d & 0x7F800000u) == 0u && (d & 0x7F0000u) != 0u);
}
// e8m0 scale byte -> fp32 2^(s-127); s = 0 is the subnormal 2^-127, s = 255 NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  if (s == 0) return __uint_as_float(0x00400000u);
  if (s == 255) return __uint_as_float(0x7FC00000u);
  return __uint_as_float(s << 23);
}

// two E2M1 codes of byte `sel` of `codes` times `scale`, as packed bf16 (low nibble in the low half)
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t codes, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, SEL));
}

// 16-byte load that does not allocate in the caches (streamed weights)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------- wave reductions
//
// DPP reductions (GFX9 data-parallel primitives, no LDS round trip): two quad
// permutes and two row rotations give every lane its 16-lane row total, two row
// broadcasts fold rows 0..3 into lane 63, which readlane hands to the whole wave.
// The association order is fixed, so results are deterministic.

constexpr int DPP_QUAD_1032 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_2301 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_ROW_ROR4 = 0x124;
constexpr int DPP_ROW_ROR8 = 0x128;
constexpr int DPP_ROW_BCAST15 = 0x142;
constexpr int DPP_ROW_BCAST31 = 0x143;

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float v, float old) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_f64(double v, double old) {
  int2 a = __builtin_bit_cast(int2, v), o = __builtin_bit_cast(int2, old);
  int2 r;
  r.x = __builtin_amdgcn_update_dpp(o.x, a.x, CTRL, ROW_MASK, 0xF, false);
  r.y = __builtin_amdgcn_update_dpp(o.y, a.y, CTRL, ROW_MASK, 0xF, false);
  return __builtin_bit_cast(double, r);
}

__device__ __forceinline__ float readlane63(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ double readlane63(double v) {
  int2 a = __builtin_bit_cast(int2, v);
  a.x = __builtin_amdgcn_readlane(a.x, 63);
  a.y = __builtin_amdgcn_readlane(a.y, 63);
  return __builtin_bit_cast(double, a);
}

// sum over the 64 lanes, returned to every lane
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f32<DPP_QUAD_1032>(v, 0.f);
  v += dpp_f32<DPP_QUAD_2301>(v, 0.f);
  v += dpp_f32<DPP_ROW_ROR4>(v, 0.f);
  v += dpp_f32<DPP_ROW_ROR8>(v, 0.f);
  v += dpp_f32<DPP_ROW_BCAST15, 0xA>(v, 0.f);
  v += dpp_f32<DPP_ROW_BCAST31, 0xC>(v, 0.f);
  return readlane63(v);
}

__device__ __forceinline__ double wave_sum_dpp(double v) {
  v += dpp_f64<DPP_QUAD_1032>(v, 0.0);
  v += dpp_f64<DPP_QUAD_2301>(v, 0.0);
  v += dpp_f64<DPP_ROW_ROR4>(v, 0.0);
  v += dpp_f64<DPP_ROW_ROR8>(v, 0.0);
  v += dpp_f64<DPP_ROW_BCAST15, 0xA>(v, 0.0);
  v += dpp_f64<DPP_ROW_BCAST31, 0xC>(v, 0.0);
  return readlane63(v);
}

__device__ __forceinline__ float wave_max_dpp(float v) {
  const float lo = -__builtin_inff();
  v = fmaxf(v, dpp_f32<DPP_QUAD_1032>(v, lo));
  v = fmaxf(v, dpp_f32<DPP_QUAD_2301>(v, lo));
  v = fmaxf(v, dpp_f32<DPP_ROW_ROR4>(v, lo));
  v = fmaxf(v, dpp_f32<DPP_ROW_ROR8>(v, lo));
  v = fmaxf(v, dpp_f32<DPP_ROW_BCAST15, 0xA>(v, lo));
  v = fmaxf(v, dpp_f32<DPP_ROW_BCAST31, 0xC>(v, lo));
  return readlane63(v);
}

__device__ __forceinline__ float wave_min_dpp(float v) {
  const float hi = __builtin_inff();
  v = fminf(v, dpp_f32<DPP_QUAD_1032>(v, hi));
  v = fminf(v, dpp_f32<DPP_QUAD_2301>(v, hi));
  v = fminf(v, dpp_f32<DPP_ROW_ROR4>(v, hi));
  v = fminf(v, dpp_f32<DPP_ROW_ROR8>(v, hi));
  v = fminf(v, dpp_f32<DPP_ROW_BCAST15, 0xA>(v, hi));
  v = fminf(v, dpp_f32<DPP_ROW_BCAST31, 0xC>(v, hi));
  return readlane63(v);
}

// inclusive prefix sum over the 64 lanes: Hillis-Steele row shifts inside each row of
// 16, then the two row broadcasts carry the row totals forward
constexpr int DPP_ROW_SHR1 = 0x111;
constexpr int DPP_ROW_SHR2 = 0x112;
constexpr int DPP_ROW_SHR4 = 0x114;
constexpr int DPP_ROW_SHR8 = 0x118;
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);  // 0 where there is no source
}
__device__ __forceinline__ int wave_incl_scan_dpp(int v) {
  v += dpp_i32<DPP_ROW_SHR1>(v);
  v += dpp_i32<DPP_ROW_SHR2>(v);
  v += dpp_i32<DPP_ROW_SHR4>(v);
  v += dpp_i32<DPP_ROW_SHR8>(v);
  v += dpp_i32<DPP_ROW_BCAST15, 0xA>(v);
  v += dpp_i32<DPP_ROW_BCAST31, 0xC>(v);
  return v;
}
// exclusive prefix sum; total receives the wave's sum
__device__ __forceinline__ int wave_excl_scan(int v, int& total) {
  const int inc = wave_incl_scan_dpp(v);
  total = __builtin_amdgcn_readlane(inc, 63);
  return inc - v;
}

// shuffle-based reductions (any lane count pattern); kept for the exact-recompute path

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// compile-time unrolling: f(std::integral_constant<int, J>) for J = 0..15, or 0..N-1
template <class Fn, int... J>
__device__ __forceinline__ void unroll_impl(Fn&& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}
template <class Fn>
__device__ __forceinline__ void unroll16(Fn&& f) {
  unroll_impl(f, std::make_integer_sequence<int, 16>{});
}
template <int N, class Fn>
__device__ __forceinline__ void unroll_n(Fn&& f) {
  unroll_impl(f, std::make_integer_sequence<int, N>{});
}

// Workgroup barrier that hands over LDS only: it waits for this wave's LDS operations
// and not for its global loads in flight.  (__syncthreads also waits for every
// outstanding global load, which empties a prefetch pipeline at each barrier.)  The
// memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }

// One wave-wide load of 16 (or 4) bytes a lane from g into LDS at lds + 16 lane (4 lane);
// lds is wave-uniform.  Written as asm so that the compiler, which cannot tell which LDS
// bytes such a load writes, does not wait for every load in flight before each LDS read:
// the kernel waits for these loads itself (an s_waitcnt vmcnt before the barrier that
// hands the LDS over).  No register receives data,
// and m0, which the instruction takes its LDS base from, is restored (a write of m0 needs
// one wait state before an instruction that reads it).
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)p;
}
__device__ __forceinline__ void lds_dma16(const void* g, const uint8_t* lds) {
  uint32_t save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_nop 0\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(save)
               : "v"(g), "s"(lds_addr(lds))
               : "memory");
}
__device__ __forceinline__ void lds_dma4(const void* g, const uint8_t* lds) {
  uint32_t save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\ts_nop 0\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(save)
               : "v"(g), "s"(lds_addr(lds))
               : "memory");
}


// Optional stamps of a kernel's span on the device's constant-rate wall clock: block b
// lowers clk[2 (b % MOE_CLOCK_SLOTS)] to its start and raises the next word to its end
// (after a block barrier, so that is the end of its last wave).  The caller sets the
// slots to {UINT64_MAX, 0}; the kernel's span is the minimum start to the maximum end.
// Two global atomics without a return value per block, spread over the slots; nothing
// at all when clk is null.  Every thread of the block must call clock_end.
__device__ __forceinline__ void clock_begin(unsigned long long* clk) {
  if (clk && threadIdx.x == 0) atomicMin(clk + 2 * (blockIdx.x % MOE_CLOCK_SLOTS), (unsigned long long)wall_clock64());
}
__device__ __forceinline__ void clock_end(unsigned long long* clk) {
  if (clk) {
    __syncthreads();
    if (threadIdx.x == 0) atomicMax(clk + 2 * (blockIdx.x % MOE_CLOCK_SLOTS) + 1, (unsigned long long)wall_clock64());
  }
}

__host__ __device__ constexpr inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ constexpr inline size_t align_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

// ------------------------------------------------ two-term e4m3 activations
//
// The scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4) multiplies MXFP4 weights by
// 8-bit activations with one e8m0 scale per 32 values.  A bf16 value has 8
// significant bits and e4m3 has 4, so each 32-block of bf16 activations x is split
// into hi = e4m3(x / S_hi) and lo = e4m3((x - hi S_hi) / S_lo) with S_hi = 2^(E-7),
// E the exponent of the block maximum, and S_lo chosen the same way from the
// residuals.  The residual of an element within 2^13 of the block maximum has at
// most 4 significant bits, so hi S_hi + lo S_lo reproduces it exactly; smaller
// elements keep an absolute error below 2^-20 of the block maximum.  Two MFMAs (hi
// and lo) then give the product of the bf16 activations with the MXFP4 weights,
// accumulated in fp32.

// round |v| < 448 to e4m3 (OCP E4M3: bias 7, 3 mantissa bits, subnormals of 2^-9),
// nearest-even; returns the code and the rounded value
__device__ __forceinline__ uint32_t e4m3_rne(float v, float& rounded) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  if (a < 0x1p-6f) {
    const float q = rintf(a * 512.f);  // exact scaling; 0..8, 8 is the smallest normal
    rounded = __uint_as_float(__float_as_uint(q * 0x1p-9f) | (sign << 24));
    return sign | (uint32_t)q;
  }
  uint32_t u = __float_as_uint(a);
  u += 0x7FFFFu + ((u >> 20) & 1u);  // nearest-even on the 3 kept mantissa bits
  u &= 0xFFF00000u;
  rounded = __uint_as_float(u | (sign << 24));
  return sign | ((((u >> 23) - 127u + 7u) & 15u) << 3) | ((u >> 20) & 7u);
}

// power-of-two exponent of |a| > 0 (subnormals included)
__device__ __forceinline__ int exponent_of(float a) {
  const uint32_t u = __float_as_uint(a) & 0x7FFFFFFFu;
  if (u >= 0x00800000u) return (int)(u >> 23) - 127;
  return -118 - (int)__clz(u);  // subnormal: value = u * 2^-149
}

__device__ __forceinline__ float pow2f(int e) {  // 2^e for -149 <= e <= 127
  if (e >= -126) return __uint_as_float((uint32_t)(e + 127) << 23);
  return __uint_as_float(1u << (e + 149));
}

// e8m0 byte for a block whose largest magnitude is amax: 2^(E-7), clamped to the
// e8m0 range; returns the byte and the scale's reciprocal as fp32
__device__ __forceinline__ uint32_t block_scale(float amax, float& inv) {
  if (!(amax > 0.f)) {
    inv = 1.f;
    return 127u;
  }
  int se = exponent_of(amax) - 7;
  if (se < -127) se = -127;
  if (se > 127) se = 127;
  inv = pow2f(-se);
  return (uint32_t)(se + 127);
}

// The split of one 32-value block held by the 4 lanes of a quad (8 consecutive values
// each; quad = lanes 4j..4j+3): the block maxima are combined with two quad permutes.
// Returns this lane's 8 hi and 8 lo codes (value i in byte i % 4 of dword i / 4) and
// the block's two scale bytes.
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, dpp_f32<DPP_QUAD_1032>(v, 0.f));
  return fmaxf(v, dpp_f32<DPP_QUAD_2301>(v, 0.f));
}
// |v| for a finite v, 0 for NaN and +-inf: block maxima are taken over the finite values
__device__ __forceinline__ float finite_abs(float v) {
  const float a = fabsf(v);
  return a <= 0x1.fffffep127f ? a : 0.f;
}
// E4M3 NaN (S.1111.111): a non-finite activation enters the matrix cores as NaN, so every
// product that reads it is NaN (an infinity cannot be encoded in E4M3)
constexpr uint32_t E4M3_NAN = 0x7Fu;

// Four values (a scaled block element each, |a| < 256, or 0) to their e4m3 codes in one
// dword (value j in byte j) and their rounded values, on the hardware conversion
// (v_cvt_pk_fp8_f32 rounds to nearest even like e4m3_rne: checked equal on every bf16
// value below 448, codes and rounded values, which covers every input here: bf16 values
// and their exact residuals times powers of two).
__device__ __forceinline__ uint32_t e4m3x4_hw(float a0, float a1, float a2, float a3, float (&q)[4]) {
  int d = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
  d = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, d, true);
  q[0] = __builtin_amdgcn_cvt_f32_fp8(d, 0);
  q[1] = __builtin_amdgcn_cvt_f32_fp8(d, 1);
  q[2] = __builtin_amdgcn_cvt_f32_fp8(d, 2);
  q[3] = __builtin_amdgcn_cvt_f32_fp8(d, 3);
  return (uint32_t)d;
}

__device__ __forceinline__ void quantize_quad8(const float (&v)[8], uint32_t (&hi)[2], uint32_t (&lo)[2], uint32_t& shi,
                                               uint32_t& slo) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, finite_abs(v[i]));
  amax = quad_max(amax);
  float inv;
  shi = block_scale(amax, inv);
  const float s_hi = 1.f / inv;
  float r[8];
  float rmax = 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    bool fin[4];
    float a[4], q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x = v[4 * h + j];
      fin[j] = finite_abs(x) == fabsf(x);
      a[j] = fin[j] ? x * inv : 0.f;
    }
    uint32_t d = e4m3x4_hw(a[0], a[1], a[2], a[3], q);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (!fin[j]) d = (d & ~(0xFFu << (8 * j))) | (E4M3_NAN << (8 * j));
      r[4 * h + j] = fin[j] ? v[4 * h + j] - q[j] * s_hi : 0.f;
      rmax = fmaxf(rmax, fabsf(r[4 * h + j]));
    }
    hi[h] = d;
  }
  rmax = quad_max(rmax);
  slo = block_scale(rmax, inv);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float q[4];
    lo[h] = e4m3x4_hw(r[4 * h] * inv, r[4 * h + 1] * inv, r[4 * h + 2] * inv, r[4 * h + 3] * inv, q);
  }
}

// MXFP8 of one 32-value block held by a quad (the activation format of the MXFP8 mode,
// OCP Microscaling v1.0 convention): shared exponent X = floor(log2 max|v|) - 8 over the
// finite values, e8m0 byte X + 127 (clamped to the e8m0 range; 0 for a block of zeros),
// codes = v / 2^X rounded to nearest-even E4M3 and saturated to +-448, the E4M3 NaN code
// for NaN and +-inf.  Written into the hi term; the lo
// term is zero (codes 0, scale byte 127), so the two-term kernels compute the same
// product and the grouped GEMMs skip it.
__device__ __forceinline__ void quantize_quad8_mx(const float (&v)[8], uint32_t (&hi)[2], uint32_t (&lo)[2],
                                                  uint32_t& shi, uint32_t& slo) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, finite_abs(v[i]));
  amax = quad_max(amax);
  int X = -127;
  if (amax > 0.f) {
    X = exponent_of(amax) - 8;
    X = X < -127 ? -127 : X > 127 ? 127 : X;
  }
  shi = (uint32_t)(X + 127);
  const float inv = pow2f(-X);
  hi[0] = hi[1] = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float q;
    const bool fin = finite_abs(v[i]) == fabsf(v[i]);
    const float t = fminf(fmaxf(fin ? v[i] * inv : 0.f, -448.f), 448.f);  // exact scaling, then saturation
    hi[i / 4] |= (fin ? e4m3_rne(t, q) : E4M3_NAN) << (8 * (i % 4));
  }
  lo[0] = lo[1] = 0u;
  slo = 127u;
}

// the activation split of the layer's format: two exact e4m3 terms, or MXFP8
__device__ __forceinline__ void quantize_quad8_fmt(const float (&v)[8], uint32_t (&hi)[2], uint32_t (&lo)[2],
                                                   uint32_t& shi, uint32_t& slo, bool mxfp8) {
  if (mxfp8)
    quantize_quad8_mx(v, hi, lo, shi, slo);
  else
    quantize_quad8(v, hi, lo, shi, slo);
}

// Quantised activation rows: codes [rows][K] (hi and lo) and e8m0 scales [rows][K/32].
struct QRows {
  uint8_t* hi;
  uint8_t* lo;
  uint8_t* shi;
  uint8_t* slo;
};

// Quantise n bf16 values (n a multiple of 32) in groups of 8, one group per lane:
// groups j0, j0 + jstride, ... (j0 and jstride chosen so that the four groups of a scale
// block sit in one quad of lanes).  All loads of a lane are issued before any group is
// converted.
__device__ __forceinline__ void quantize_quads(const uint16_t* __restrict__ src, QRows q, int64_t n, int64_t j0,
                                               int64_t jstride, bool mxfp8 = false) {
  constexpr int U = 2;
  const int64_t ng = n / 8;
  for (int64_t base = j0; base < ng; base += U * jstride) {
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = base + u * jstride;
      raw[u] = j < ng ? *reinterpret_cast<const uint4*>(src + 8 * j) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = base + u * jstride;
      if (j < ng) {
        const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
        float v[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = bf16lo(w[i]);
          v[2 * i + 1] = bf16hi(w[i]);
        }
        uint32_t hi[2], lo[2], shi, slo;
        quantize_quad8_fmt(v, hi, lo, shi, slo, mxfp8);
        *reinterpret_cast<uint2*>(q.hi + 8 * j) = make_uint2(hi[0], hi[1]);
        *reinterpret_cast<uint2*>(q.lo + 8 * j) = make_uint2(lo[0], lo[1]);
        if ((j & 3) == 0) {
          q.shi[j >> 2] = (uint8_t)shi;
          q.slo[j >> 2] = (uint8_t)slo;
        }
      }
    }
  }
}

}  // namespace moe
