// MXFP8 weight quantization (section Quantization of the paper: weight-only
// MXFP8 by post-training quantization with standard maximum scaling).
//
// Format (OCP microscaling): each block of 32 consecutive elements along a
// weight row (the reduction dimension) shares a power-of-two scale stored as
// an 8-bit biased exponent (value 2^(code - 127)); elements are FP8 E4M3
// (bias 7, 3 mantissa bits, largest finite 448, subnormals m * 2^-9).
// Scale rule: shared exponent floor(log2(max |w|)) - 8, clamped to >= -126
// (every scale is a normal float). Elements: w * 2^-shared rounded to the
// nearest E4M3 value, ties to the even encoding, saturating at 448; the sign
// of a value rounding to zero is kept.
//
// One thread per block: it reads the block's 32 bf16 weights (64 bytes),
// writes 32 codes, the scale code and, optionally, the 32 dequantized values
// as bf16 (exact: an E4M3 value times a power of two in the float32 range is
// a bf16 value).
#include "common.h"
#include "kernels.h"

namespace dory {

namespace {

// Nearest E4M3 code of a float, ties to even, saturating.
__device__ __forceinline__ uint32_t e4m3_encode(float q) {
  const uint32_t sign = (__float_as_uint(q) >> 24) & 0x80u;
  const float a = fabsf(q);
  uint32_t code;
  if (!(a < 448.f)) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {
    // below the smallest normal 2^-6: multiples of 2^-9 (8 * 2^-9 is 2^-6,
    // whose code is 8 as well)
    code = (uint32_t)__builtin_rintf(a * 512.f);
  } else {
    int e = (int)((__float_as_uint(a) >> 23) & 255u) - 127;  // floor(log2 a), -6 .. 8
    uint32_t m = (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 3 - e));  // 8 .. 16
    if (m == 16u) { m = 8u; ++e; }
    code = ((uint32_t)(e + 7) << 3) | (m - 8u);
  }
  return code | sign;
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float v = e == 0 ? (float)m * 0.001953125f : __builtin_ldexpf((float)(8u + m), (int)e - 10);
  return (c & 0x80u) ? -v : v;
}

__global__ void __launch_bounds__(256)
mx_quantize_kernel(const uint16_t* __restrict__ w, int64_t nblocks, int cols,
                   uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                   uint16_t* __restrict__ deq) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= nblocks) return;
  const int bpr = cols / 32;
  const int64_t row = t / bpr;
  const int64_t off = row * cols + (t - row * bpr) * 32;
  float f[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = reinterpret_cast<const uint4*>(w + off)[i];
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[8 * i + 2 * j] = __uint_as_float(u[j] << 16);
      f[8 * i + 2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(f[i]));
  // floor(log2 amax) from the exponent field; zero and float32 subnormals
  // (field 0) fall under the clamp
  const int fl = (int)((__float_as_uint(amax) >> 23) & 255u) - 127;
  const int se = max(fl - 8, -126);
  scales[t] = (uint8_t)(se + 127);
  uint32_t packed[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) packed[i] = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i)
    packed[i >> 2] |= e4m3_encode(__builtin_ldexpf(f[i], -se)) << (8 * (i & 3));
  uint4* cdst = reinterpret_cast<uint4*>(codes + off);
  cdst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  cdst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  if (deq) {
    uint32_t d2[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t c0 = (packed[(2 * i) >> 2] >> (8 * ((2 * i) & 3))) & 255u;
      const uint32_t c1 = (packed[(2 * i + 1) >> 2] >> (8 * ((2 * i + 1) & 3))) & 255u;
      const uint32_t b0 = __float_as_uint(__builtin_ldexpf(e4m3_value(c0), se)) >> 16;
      const uint32_t b1 = __float_as_uint(__builtin_ldexpf(e4m3_value(c1), se)) >> 16;
      d2[i] = b0 | (b1 << 16);
    }
    uint4* ddst = reinterpret_cast<uint4*>(deq + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) ddst[i] = make_uint4(d2[4 * i], d2[4 * i + 1], d2[4 * i + 2], d2[4 * i + 3]);
  }
}

}  // namespace

hipError_t launch_mx_quantize(const uint16_t* w, int64_t rows, int cols, uint8_t* codes,
                              uint8_t* scales, uint16_t* deq, hipStream_t st) {
  if (rows < 1 || cols < 32 || cols % 32 != 0) return hipErrorInvalidValue;
  const int64_t nblocks = rows * (cols / 32);
  const int64_t grid = (nblocks + 255) / 256;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mx_quantize_kernel, dim3((unsigned)grid), dim3(256), 0, st, w, nblocks, cols,
                     codes, scales, deq);
  return hipGetLastError();
}

}  // namespace dory
