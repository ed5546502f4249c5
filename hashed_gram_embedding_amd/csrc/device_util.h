// Small device helpers: bfloat16 conversions and wavefront reductions (gfx950,
// 64-lane wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace engram {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// float -> bfloat16 bits with gfx950's conversion instruction
// (v_cvt_pk_bf16_f32): round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two floats -> two bfloat16 in one word (lo in bits 0-15), one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// SiLU(x) = x / (1 + e^-x) from the hardware exp2 and reciprocal (about one
// ulp each): e^-x = 2^(-x log2 e).  Large |x| saturate correctly: 2^(+big)
// = inf gives x * 0, 2^(-big) = 0 gives x.
__device__ __forceinline__ float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504088896341f * x));
}

// ---- MXFP8: E4M3 elements (bias 7, largest finite 448, subnormals of 2^-9),
// one power-of-two scale per 32 consecutive values along the contraction
// axis, stored as a biased exponent byte.  The scale is the smallest power of
// two that keeps the block's largest magnitude within 448: with
// amax = m 2^E (0.5 <= m < 1) the exponent is E - 9, plus one when m > 0.875.

// Nearest-even E4M3 code of x, |x| <= 448.  Below 2^-6 the quantum is 2^-9
// (the code is the multiple of 2^-9, and 8 is also the smallest normal's
// code); above, the float's top 3 mantissa bits are rounded in place.
__device__ __forceinline__ uint32_t e4m3_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  const uint32_t ab = b & 0x7fffffffu;
  const float a = __uint_as_float(ab);
  uint32_t code;
  if (a < 0.015625f) code = static_cast<uint32_t>(rintf(a * 512.0f));
  else code = ((ab + 0x7ffffu + ((ab >> 20) & 1u)) >> 20) - (120u << 3);
  return code | ((b >> 24) & 0x80u);
}

// Scale exponent of a block whose largest magnitude is amax (> 0), clamped
// to the byte's range.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  int E;
  const float m = frexpf(amax, &E);
  int e = E - 9 + (m > 0.875f ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Quantise 8 values held by each lane of an aligned group of 4 lanes (one
// 32-value block): returns the 8 codes packed little-endian and sets *sbyte
// to the block's scale byte (0 for an all-zero block).
__device__ __forceinline__ uint2 mx_quantize8(const float* f, uint32_t* sbyte) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  if (amax == 0.f) {
    *sbyte = 0;
    return make_uint2(0u, 0u);
  }
  const int e = mx_scale_exp(amax);
  *sbyte = static_cast<uint32_t>(e + 127);
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i >> 2] |= e4m3_rne(ldexpf(f[i], -e)) << (8 * (i & 3));
  return make_uint2(w[0], w[1]);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Unpack 8 bf16 held in a uint4 into floats.
__device__ __forceinline__ void unpack8(const uint4& q, float* f) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ uint4 pack8(const float* f) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace engram
