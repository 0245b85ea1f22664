// w8a8.hip -- the W8A8 variant's per-row quantisation kernels for gfx950: one
// scale per activation row (the row's amax / 448 over all of it, or a static
// per-tensor scale), for the hidden states and for the SwiGLU output.
//
// [P2 Reviewed changes: w8a8.py, the static FP8 MoE backend]
// [P4 Pull request overview: the W8A8 fused MoE ends with moe_reduce]
//   [P2] lmdeploy PR "perf(pytorch): optimize compact blocked FP8 MoE and route
//        preparation"
//   [P4] lmdeploy PR "Moe Reduce kernel"
//
// Work mapping: one 256-thread workgroup per row; thread t holds the 8-value
// pieces t, t + 256, ... of the row (at most four: rows of up to 8192 values)
// in registers, so the row is read once; the row amax is a wave butterfly and
// a 4-entry LDS step.  Quantisation as quant_fp8 (fp64 reciprocal product,
// hardware conversion), with the quotient clamped to +-448 for static scales.
#include "device.h"
#include "internal.h"

namespace bfp8 {

namespace {

constexpr int kRowThreads = 256;
constexpr int kMaxPieces = 4;  // pieces of 8 values per thread: rows up to 8192

__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// Largest value over the workgroup (all threads call it).
__device__ __forceinline__ float block_max(float v) {
  __shared__ float s_m[kRowThreads / 64];
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) v = fmaxf(v, __shfl_xor(v, d));
  if ((threadIdx.x & 63) == 0) s_m[threadIdx.x >> 6] = v;
  __syncthreads();
  v = s_m[0];
#pragma unroll
  for (int w = 1; w < kRowThreads / 64; w++) v = fmaxf(v, s_m[w]);
  return v;
}

// Quantise this thread's pieces of a row held in v[p] (BF16-valued floats)
// with the row's scale; thread 0 stores the scale.
__device__ __forceinline__ void quant_row_pieces(const float (&v)[kMaxPieces][8], int pieces, int fmt,
                                                 float static_scale, uint8_t* __restrict__ qrow,
                                                 float* __restrict__ srow) {
  float sc;
  if (static_scale > 0.0f) {
    sc = static_scale;
  } else {
    float m = 0.0f;
#pragma unroll
    for (int p = 0; p < kMaxPieces; p++)
      if (threadIdx.x + kRowThreads * p < pieces)
#pragma unroll
        for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(v[p][i]));
    sc = group_scale(block_max(m), fmt);
  }
#pragma unroll
  for (int p = 0; p < kMaxPieces; p++) {
    const int c = threadIdx.x + kRowThreads * p;
    if (c < pieces)
      *reinterpret_cast<uint2*>(qrow + 8 * (size_t)c) =
          static_scale > 0.0f ? encode8_scaled_sat(v[p], sc) : encode8_scaled(v[p], sc);
  }
  if (threadIdx.x == 0) *srow = sc;
}

__global__ __launch_bounds__(kRowThreads) void quant_rows_kernel(const uint16_t* __restrict__ x, int K, int fmt,
                                                                 float static_scale, uint8_t* __restrict__ q,
                                                                 float* __restrict__ s) {
  const int64_t r = blockIdx.x;
  const int pieces = K / 8;
  float v[kMaxPieces][8];
#pragma unroll
  for (int p = 0; p < kMaxPieces; p++) {
    const int c = threadIdx.x + kRowThreads * p;
    if (c < pieces) unpack8(*reinterpret_cast<const uint4*>(x + (size_t)r * K + 8 * (size_t)c), v[p]);
  }
  quant_row_pieces(v, pieces, fmt, static_scale, q + (size_t)r * K, s + r);
}

__global__ __launch_bounds__(kRowThreads) void silu_and_mul_quant_rows_kernel(
    const uint16_t* __restrict__ gu, int I, RowFilter filt, float limit, int clamp, int fmt, float static_scale,
    uint8_t* __restrict__ q, float* __restrict__ s) {
  const int64_t r = blockIdx.x;
  if (!row_live(filt, r)) return;  // the whole workgroup: the row is left untouched
  const int pieces = I / 8;
  const uint16_t* row = gu + (size_t)r * 2 * I;
  float v[kMaxPieces][8];
#pragma unroll
  for (int p = 0; p < kMaxPieces; p++) {
    const int c = threadIdx.x + kRowThreads * p;
    if (c < pieces) {
      float g[8], u[8];
      unpack8(*reinterpret_cast<const uint4*>(row + 8 * (size_t)c), g);
      unpack8(*reinterpret_cast<const uint4*>(row + I + 8 * (size_t)c), u);
#pragma unroll
      for (int i = 0; i < 8; i++) v[p][i] = swiglu_bf16(g[i], u[i], limit, clamp != 0);
    }
  }
  quant_row_pieces(v, pieces, fmt, static_scale, q + (size_t)r * I, s + r);
}

}  // namespace

bool rows_quant_fits(int K) { return K > 0 && K % 128 == 0 && K <= 8 * kRowThreads * kMaxPieces; }

hipError_t launch_quant_fp8_rows(const uint16_t* x, int64_t rows, int K, int fmt, float static_scale, uint8_t* q,
                                 float* s, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (!rows_quant_fits(K) || rows > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)rows), dim3(kRowThreads), 0, stream, x, K, fmt, static_scale,
                     q, s);
  return hipGetLastError();
}

hipError_t launch_silu_and_mul_quant_rows(const uint16_t* gu, int64_t rows, int I, const RowFilter& f, float limit,
                                          int fmt, float static_scale, uint8_t* q, float* s, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (!rows_quant_fits(I) || rows > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int clamp = __builtin_isfinite(limit) ? 1 : 0;
  hipLaunchKernelGGL(silu_and_mul_quant_rows_kernel, dim3((unsigned)rows), dim3(kRowThreads), 0, stream, gu, I, f,
                     limit, clamp, fmt, static_scale, q, s);
  return hipGetLastError();
}

}  // namespace bfp8
