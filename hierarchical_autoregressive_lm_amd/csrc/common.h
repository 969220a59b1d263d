// Shared device helpers: bf16 storage, rounding, wave reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>


typedef uint16_t bf16_t;

// bf16 -> fp32 is exact (the bf16 bits are the high half of the fp32 bits).
__device__ __forceinline__ float bf2f(bf16_t v) {
  return __uint_as_float(((uint32_t)v) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (NaN stays a NaN): gfx950's
// v_cvt_pk_bf16_f32, which a __bf16 conversion compiles to.  It gives the
// same bits as rounding the fp32 bit pattern in integer arithmetic (add
// 0x7fff plus the lowest kept bit, truncate) for every non-NaN input,
// checked on the GPU over 2^25 inputs including every tie.
__device__ __forceinline__ bf16_t f2bf(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
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

// DPP moves inside 16-lane rows (lanes 16k .. 16k+15): a VALU operand
// modifier, so no trip through the LDS crossbar that a shuffle takes.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a row, every lane receiving the total: pairs
// inside each quad (quad_perm 1,0,3,2), the two pairs of a quad (2,3,0,1),
// the two quads of each half row (row_half_mirror), the two half rows
// (row_mirror).  At each step both lanes of a pair add the same two values,
// so the 16 results are bit-identical.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  return v;
}

// The value of lane c ^ 8 of the same 16-lane row (row_ror by 8).
__device__ __forceinline__ float row16_swap8(float v) { return dpp_mov<0x128>(v); }

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
