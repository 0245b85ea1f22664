// mfma.h -- FP8 MFMA fragments for gfx950 (CDNA4).  Internal header.
//
// V_MFMA_SCALE_F32_16X16X128_F8F6F4 with unit E8M0 scales (127) and both
// operands in OCP E4M3: C[16x16] += A[16x128] * B[128x16], fp32 accumulate.
//
// Operand fragment of lane l (64 lanes): row (A) or column (B) index l % 16,
// K slot group kq = l / 16, 32 bytes in 8 VGPRs.  The hardware's K order of
// an E4M3 fragment (measured through the FP4 x FP8 form, where it shows) is,
// for a 128-wide K chunk starting at k0:
//     bytes  0..15 of lane l  <- k0 + 16*kq + [0, 16)
//     bytes 16..31 of lane l  <- k0 + 64 + 16*kq + [0, 16)
// so that one 16-byte load per lane reads 64 contiguous bytes of each of the
// 16 rows, and the two loads together cover the rows' 128-byte chunk.  An
// E2M1 fragment (16 bytes in 4 VGPRs) holds K k0 + 32*kq + [0, 32) in order,
// element 2j in the low nibble of byte j.
//
// Result fragment: lane l holds C[4*(l/16) + v][l % 16], v = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bfp8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma_f8_16x16x128(const v8i& a, const v8i& b, const v4f& c) {
  // cbsz = blgp = 0: E4M3 operands; scale operands 127 = 2^0.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// A in E2M1 (cbsz 4: the low 16 bytes of a, 32 elements, element 2j in the
// low nibble of byte j), B in E4M3 (the order above); scale_a the E8M0 byte
// of the lane's A slice, B unscaled (127).  The scales act per lane, and a
// lane's A slice, K 32 (l / 16) .. + 31 of its row, is one MX block of 32.
__device__ __forceinline__ v4f mfma_f4f8_16x16x128(const v8i& a, const v8i& b, int scale_a, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, scale_a, 0, 127);
}

// Load the 32-byte fragment of a 128-byte chunk at p (16-byte aligned) for
// K slot group kq.
__device__ __forceinline__ v8i load_frag(const uint8_t* p, int kq) {
  const uint4 lo = *reinterpret_cast<const uint4*>(p + 16 * kq);
  const uint4 hi = *reinterpret_cast<const uint4*>(p + 64 + 16 * kq);
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

__device__ __forceinline__ v8i zero_frag() {
  v8i f;
#pragma unroll
  for (int i = 0; i < 8; i++) f[i] = 0;
  return f;
}

}  // namespace bfp8
