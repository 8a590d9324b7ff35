// Shared device helpers for the gfx950 (CDNA4) kernels of the looped nGPT
// forward pass. Everything here is wave64-specific.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dory {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf2f(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Sum over all threads of a block of NT threads (NT multiple of 64, <= 1024).
// `red` must hold NT/64 floats; returns the total to every thread.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) t += red[i];
  __syncthreads();
  return t;
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

}  // namespace dory

namespace dory {

// Workgroup barrier that waits only for this wave's own LDS operations.
// Pipelines that stage tiles with global->LDS DMA wait for the DMA they need
// with an explicit vmcnt before calling it, so that younger DMA (the next
// tiles) stays in flight across the barrier; __syncthreads() would drain it.
// The memory clobber keeps the compiler from moving LDS accesses across.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Attention visibility: a query at position p sees key u iff u <= p and, for
// a sliding-window layer (window > 0), p - u < window.
__device__ __forceinline__ bool key_visible(int64_t p, int64_t u, int window) {
  return u <= p && (window == 0 || p - u < window);
}

}  // namespace dory
