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
// |x| >= 448 saturates to 448, NaN -> 0x7F | sign, sign of zero kept.  This is
// the definition the hardware conversion used by encode8_scaled was checked
// against.
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

// Quantise 8 BF16-valued floats of one group with scale s: E4M3FN(RN32(x/s)).
//
// Division: RN32(x * RN64(1/s)) equals RN32(x/s) for every BF16 x and fp32 s.
// Write x = A 2^a (|A| < 2^8), s = B 2^b (B < 2^24).  x/s is never an fp32
// rounding midpoint (a midpoint has a 25-bit odd significand 2C+1; x/s equal to
// it would need 2C+1 to divide A), and when it is not one its relative
// distance to the nearest midpoint is at least 2^-49 (|A 2^j - B(2C+1)| >= 1
// over B 2^25 in relative terms), while RN64(1/s) and the fp64 product add a
// relative error of at most 2^-52.  So both sides of every midpoint agree and
// the fp32 results are identical; the cost is one fp64 division per group and
// three cheap operations per value instead of an fp32 division per value.
//
// Encoding: V_CVT_PK_FP8_F32 (round to nearest even, OCP E4M3) gives the same
// byte as e4m3_encode for every finite fp32 of magnitude below 464 (checked
// exhaustively on gfx950), and a quantised value never exceeds 448 * (1 +
// 2^-24) in magnitude because s >= amax / 448 rounded.
__device__ __forceinline__ uint2 encode8_scaled(const float (&f)[8], float s) {
  const double rs = 1.0 / (double)s;
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; i++) q[i] = (float)((double)f[i] * rs);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], hi, true);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
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
