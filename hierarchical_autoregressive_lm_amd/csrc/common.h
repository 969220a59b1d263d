// Shared device helpers: bf16 storage, rounding, wave reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>


typedef uint16_t bf16_t;

// bf16 -> fp32 is exact (the bf16 bits are the high half of the fp32 bits).
__device__ __forceinline__ float bf2f(bf16_t v) {
  return __uint_as_float(((uint32_t)v) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (NaN stays a quiet NaN).
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// Storage traits: T is float (fp32 models) or bf16_t (bf16 models).
template <typename T> struct St;
template <> struct St<float> {
  static __device__ __forceinline__ float ld(float v) { return v; }
  static __device__ __forceinline__ float st(float f) { return f; }
};
template <> struct St<bf16_t> {
  static __device__ __forceinline__ float ld(bf16_t v) { return bf2f(v); }
  static __device__ __forceinline__ bf16_t st(float f) { return f2bf(f); }
};

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

// Exact GELU, z * Phi(z), with the library erff.
__device__ __forceinline__ float gelu_f(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}
