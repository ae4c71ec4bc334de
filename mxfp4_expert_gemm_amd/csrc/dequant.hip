// Bit-exact MXFP4 -> fp32 dequantisation of one [rows][cols] matrix.
//
// Format (kimi-k3-in-c post, "experts that are already 4-bit MXFP4"; kimi-k3-mlx
// digest, quantisation tiers): a weight is a 4-bit E2M1 code, element 2j of a row
// in the low nibble of byte j; 32 consecutive weights of a row share one e8m0
// exponent byte.  Codes of all rows come first, then the scales.
#include "common.h"
#include "kernels.h"

namespace moe {

// E2M1 code -> fp32 bits: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa;
// exponent field 0 gives 0 or 0.5.
__device__ __forceinline__ float e2m1_f32(uint32_t code) {
  uint32_t mag = code & 7u, ex = mag >> 1, man = mag & 1u;
  uint32_t bits;
  if (ex == 0)
    bits = man ? 0x3F000000u : 0u;                 // 0.5 or 0
  else
    bits = ((ex - 1u + 127u) << 23) | (man << 22);  // (1 + man/2) * 2^(ex-1)
  return __uint_as_float(bits | ((code & 8u) << 28));
}

// One thread per code byte: two weights.  The fp32 product of the E2M1 value and
// 2^(s-127) is exact (two significant bits) unless it overflows, where it rounds
// to +-inf; s = 255 gives NaN through the NaN scale.
__global__ void __launch_bounds__(256) dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales, int64_t rows,
                                                      int32_t cols, float* __restrict__ out) {
  const int64_t row_bytes = cols / 2;
  const int64_t n = rows * row_bytes;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    int64_t r = i / row_bytes;
    int64_t jb = i - r * row_bytes;
    uint32_t byte = codes[i];
    float sc = e8m0_to_f32(scales[r * (cols / 32) + jb / 16]);
    float2 v;
    v.x = e2m1_f32(byte & 15u) * sc;
    v.y = e2m1_f32(byte >> 4) * sc;
    *reinterpret_cast<float2*>(out + 2 * i) = v;
  }
}

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t cols,
                          float* out, hipStream_t st) {
  int64_t n = rows * (int64_t)(cols / 2);
  if (n == 0) return hipSuccess;
  int64_t blocks = ceil_div(n, 256);
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, st, codes, scales, rows, cols,
                     out);
  return hipGetLastError();
}

}  // namespace moe
