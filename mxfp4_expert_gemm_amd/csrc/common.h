// Shared device helpers for the gfx950 kernels of the MXFP4 Stable-LatentMoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_layer.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

// ---------------------------------------------------------------- bf16 bits

__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }

// acc + a.lo*b.lo + a.hi*b.hi
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(b), acc, false);
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

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }

__host__ __device__ constexpr inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ constexpr inline size_t align_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

}  // namespace moe
