// device.h -- device-side number formats and wave helpers for the gfx950
// kernels of the block-FP8 MoE library.  Internal header, HIP device code only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bfp8 {

constexpr int kGroup = 128;          // quant group / weight block edge
constexpr float kE4M3Max = 448.0f;   // largest finite OCP E4M3FN magnitude
constexpr float kAmaxFloor = 1e-10f; // amax floor before the scale is formed

// ---------------------------------------------------------------- BF16

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> BF16 bits, round to nearest even; NaN -> quiet NaN with its sign.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return ((b >> 16) & 0x8000u) | 0x7FC0u;
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------- E4M3FN

// fp32 -> OCP E4M3FN byte, round to nearest even on the fp32 bit fields;
// |x| >= 448 saturates to 448, NaN -> 0x7F | sign, sign of zero kept.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  uint32_t b = __float_as_uint(x);
  uint32_t sign = (b >> 24) & 0x80u;
  uint32_t a = b & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;           // 448.0f
  if (a < 0x3C800000u) {                                 // below 2^-6: step 2^-9
    float v = __uint_as_float(a) * 512.0f;               // exact power-of-two scaling
    return sign | (uint32_t)__builtin_rintf(v);          // rint: nearest even; 8 carries into 2^-6
  }
  uint32_t exp8 = (a >> 23) - 127u + 7u;                 // 1..15
  uint32_t man = a & 0x7FFFFFu;
  uint32_t m3 = man >> 20;
  uint32_t rest = man & 0xFFFFFu;
  m3 += (rest > 0x80000u) | ((rest == 0x80000u) & (m3 & 1u));
  // m3 == 8 carries into the exponent: (exp8 << 3) + 8 == ((exp8 + 1) << 3)
  return sign | ((exp8 << 3) + m3);
}

// ---------------------------------------------------------------- scales

// Group scale from the group's amax; fmt 0: amax/448, fmt 1: rounded up to a
// power of two through the fp32 exponent field.
__device__ __forceinline__ float group_scale(float amax, int fmt) {
  float a = amax > kAmaxFloor ? amax : kAmaxFloor;
  float v = a / kE4M3Max;
  if (fmt == 1) {
    uint32_t b = __float_as_uint(v);
    uint32_t e = (b >> 23) + ((b & 0x7FFFFFu) != 0u);
    v = __uint_as_float(e << 23);
  }
  return v;
}

// ---------------------------------------------------------------- SwiGLU

// bf16(silu(g) * u) with the optional finite clamp.  exp(-g) is evaluated in
// fp64 and rounded once to fp32, which is the correctly rounded fp32 value for
// every BF16 gate (the fp64 result sits far from any fp32 rounding boundary).
__device__ __forceinline__ float swiglu_bf16(float g, float u, float limit, bool clamp) {
  if (clamp) {
    g = g > limit ? limit : g;
    u = u > limit ? limit : u;
    u = u < -limit ? -limit : u;
  }
  float e = (float)exp(-(double)g);
  float d = 1.0f + e;
  float sg = g / d;
  float h = sg * u;
  return bf16_to_f32(f32_to_bf16(h));
}

// ---------------------------------------------------------------- waves

__device__ __forceinline__ float max_over_16(float v) {
  // reduce within aligned groups of 16 lanes
  v = fmaxf(v, __shfl_xor(v, 8, 16));
  v = fmaxf(v, __shfl_xor(v, 4, 16));
  v = fmaxf(v, __shfl_xor(v, 2, 16));
  v = fmaxf(v, __shfl_xor(v, 1, 16));
  return v;
}

}  // namespace bfp8
