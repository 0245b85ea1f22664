// elementwise.hip -- group-128 activation quantisation, SwiGLU, fused
// SwiGLU + quantisation and moe_reduce for gfx950.
//
// Work mapping shared by the quant kernels: one group of 128 values is owned
// by 16 consecutive lanes, each lane holding 8 values (one 16-byte load of
// BF16).  A wave therefore covers 4 groups; the group amax is a 16-lane
// butterfly.  Loads and stores are 16/8-byte vectors, contiguous across lanes.
//
// [P1 Modification, Fused SwiGLU and FP8 quantization] the fused kernel keeps
// the BF16 SwiGLU value in registers and writes only codes and scales.
// [P3 Purpose] clamp, UE8M0 scales and row filtering.
// [P4 Pull request overview] moe_reduce applies the router weights.
//
// Pages cited in brackets, by key and section:
//   [P1] lmdeploy PR "Perf/pytorch block fp8 moe decode"
//   [P2] lmdeploy PR "perf(pytorch): optimize compact blocked FP8 MoE and route
//        preparation"
//   [P3] vLLM PR "[Kernel][Perf] Fuse clamped MoE activation and UE8M0 FP8 block
//        quantization"
//   [P4] lmdeploy PR "Moe Reduce kernel"
#include <algorithm>

#include "device.h"
#include "internal.h"

namespace bfp8 {

namespace {

constexpr int kThreads = 256;                 // 4 waves, 16 groups per workgroup
constexpr int kGroupsPerBlock = kThreads / 16;
// SwiGLU exp by table from this many groups of 128 up: below it the kernels
// are bound by latency, and the table's dependent load costs more than the
// fp64 exp it saves (measured: 8 to 2,048 rows of width 512, 128 rows of 256;
// the table wins at 4,096 rows of 768 and 16,384 of 1,024)
constexpr int64_t kTableMinGroups = 16384;

__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ float lane_amax8(const float (&f)[8]) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(f[i]));
  return m;
}

__global__ __launch_bounds__(kThreads) void quant_fp8_kernel(const uint16_t* __restrict__ x, int64_t n_groups,
                                                             int gpr, int fmt, uint8_t* __restrict__ q,
                                                             float* __restrict__ s) {
  const int64_t gid = (int64_t)blockIdx.x * kGroupsPerBlock + (threadIdx.x >> 4);
  if (gid >= n_groups) return;  // whole 16-lane group leaves together
  quant_group8(x, gid, threadIdx.x & 15, fmt, q, s);  // rows are contiguous groups
  (void)gpr;
}

// SwiGLU of this lane's 8 outputs of group g in row r (gate at column
// g*128 + 8*l16, up I columns later); returns them as BF16-valued floats.
template <bool kTable>
__device__ __forceinline__ void swiglu8(const uint16_t* __restrict__ gu, int64_t r, int I, int g, int l16,
                                        float limit, bool clamp, float (&a)[8]) {
  const uint16_t* row = gu + (size_t)r * 2 * I + (size_t)g * kGroup + (size_t)l16 * 8;
  uint4 gv = *reinterpret_cast<const uint4*>(row);
  uint4 uv = *reinterpret_cast<const uint4*>(row + I);
  float gf[8], uf[8];
  unpack8(gv, gf);
  unpack8(uv, uf);
#pragma unroll
  for (int i = 0; i < 8; i++) a[i] = swiglu_bf16<kTable>(gf[i], uf[i], limit, clamp);
}

template <bool kTable>
__global__ __launch_bounds__(kThreads) void silu_and_mul_kernel(const uint16_t* __restrict__ gu, int64_t n_groups,
                                                                int I, float limit, int clamp,
                                                                uint16_t* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * kGroupsPerBlock + (threadIdx.x >> 4);
  const int l16 = threadIdx.x & 15;
  if (gid >= n_groups) return;
  const int gpr = I / kGroup;
  const int64_t r = gid / gpr;
  const int g = (int)(gid - r * gpr);
  float a[8];
  swiglu8<kTable>(gu, r, I, g, l16, limit, clamp != 0, a);
  uint4 o;
  o.x = f32_to_bf16(a[0]) | (f32_to_bf16(a[1]) << 16);
  o.y = f32_to_bf16(a[2]) | (f32_to_bf16(a[3]) << 16);
  o.z = f32_to_bf16(a[4]) | (f32_to_bf16(a[5]) << 16);
  o.w = f32_to_bf16(a[6]) | (f32_to_bf16(a[7]) << 16);
  *reinterpret_cast<uint4*>(out + (size_t)r * I + (size_t)g * kGroup + (size_t)l16 * 8) = o;
}

template <bool kTable>
__global__ __launch_bounds__(kThreads) void silu_and_mul_quant_kernel(const uint16_t* __restrict__ gu,
                                                                      int64_t n_groups, int I, RowFilter filt,
                                                                      float limit, int clamp, int fmt,
                                                                      uint8_t* __restrict__ q,
                                                                      float* __restrict__ s) {
  const int64_t gid = (int64_t)blockIdx.x * kGroupsPerBlock + (threadIdx.x >> 4);
  const int l16 = threadIdx.x & 15;
  if (gid >= n_groups) return;
  const int gpr = I / kGroup;
  const int64_t r = gid / gpr;
  const int g = (int)(gid - r * gpr);
  if (!row_live(filt, r)) return;  // masked rows are left untouched
  float a[8];
  swiglu8<kTable>(gu, r, I, g, l16, limit, clamp != 0, a);
  float amax = max_over_16(lane_amax8(a));
  float sc = group_scale(amax, fmt);
  *reinterpret_cast<uint2*>(q + (size_t)r * I + (size_t)g * kGroup + (size_t)l16 * 8) = encode8_scaled(a, sc);
  if (l16 == 0) s[(size_t)r * gpr + g] = sc;
}

// Act+quant over a filtered row set or a row list, one item per 16-lane
// group: item f in [0, n gpr) is group f % gpr of position f / gpr.  Its
// loads leave in dependent steps: the position's row (list entry, or row id
// and then the id's map entry), then the gate/up values when the row is
// live.  Positions are rows under the filter when kList is false, else
// list[p] for p < *count (e.g. route preparation's sorted routes and its kept
// count: the rows past the count cost one count read).  Index arithmetic is
// 32-bit (the host keeps n gpr below 2^31).  Measured at top-k 6, width 2048,
// 1/8 of the rows local, 6 to 6144 rows: several items per lane group, the
// rows compacted per workgroup by ballot, and 512- or 1024-thread
// workgroups were all as fast or slower.
template <bool kTable, bool kList>
__global__ __launch_bounds__(kThreads) void silu_and_mul_quant_items_kernel(
    const uint16_t* __restrict__ gu, int n, const int32_t* __restrict__ list, const int32_t* __restrict__ count,
    RowFilter filt, int I, float limit, int clamp, int fmt, uint8_t* __restrict__ q, float* __restrict__ s) {
  const int l16 = threadIdx.x & 15;
  const unsigned gpr = (unsigned)I / kGroup;
  const unsigned f = blockIdx.x * kGroupsPerBlock + (threadIdx.x >> 4);
  const unsigned n_pos = kList ? (unsigned)max(0, min(*count, n)) : (unsigned)n;
  if (f >= n_pos * gpr) return;  // whole 16-lane group leaves together
  const unsigned pos = f / gpr, g = f - pos * gpr;
  const int32_t v = kList ? list[pos] : filt.ids[pos];
  unsigned row = pos;
  if constexpr (kList) {
    row = (unsigned)v;
  } else {
    const bool local = filt.mode == kRowsLocal;
    const int32_t* map = local ? filt.sel.map : filt.map;
    const int32_t E = local ? filt.sel.E : filt.E;
    bool ok;
    if (local && !map) {
      const int64_t e = (int64_t)v - filt.sel.offset;
      ok = e >= 0 && e < filt.sel.L;
    } else {
      ok = v >= 0 && v < E;
      if (ok && map) {
        const int32_t m = map[v];
        ok = m >= 0 && (!local || m < filt.sel.L);
      }
    }
    if (!ok) return;  // masked rows are left untouched
  }
  const uint16_t* src = gu + (size_t)row * 2 * I + g * kGroup + l16 * 8;
  const uint4 gv = *reinterpret_cast<const uint4*>(src);
  const uint4 uv = *reinterpret_cast<const uint4*>(src + I);
  float gf[8], uf[8], a[8];
  unpack8(gv, gf);
  unpack8(uv, uf);
#pragma unroll
  for (int i = 0; i < 8; i++) a[i] = swiglu_bf16<kTable>(gf[i], uf[i], limit, clamp != 0);
  const float sc = group_scale(max_over_16(lane_amax8(a)), fmt);
  *reinterpret_cast<uint2*>(q + (size_t)row * I + g * kGroup + l16 * 8) = encode8_scaled(a, sc);
  if (l16 == 0) s[(size_t)row * gpr + g] = sc;
}

// One thread per (token, 8 consecutive columns): acc over the k routes in
// order with fmaf, one rounding to BF16.
__global__ __launch_bounds__(kThreads) void moe_reduce_kernel(const uint16_t* __restrict__ y,
                                                              const float* __restrict__ w,
                                                              const int32_t* __restrict__ ids, ExpertSel sel,
                                                              int64_t M, int k, int H, uint16_t* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int h8 = H / 8;
  if (idx >= M * h8) return;
  const int64_t t = idx / h8;
  const int c = (int)(idx - t * h8) * 8;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; i++) acc[i] = 0.0f;
  for (int j = 0; j < k; j++) {
    const int64_t r = t * k + j;
    if (ids && local_of(sel, ids[r]) < 0) continue;
    const float wt = w[r];
    uint4 v = *reinterpret_cast<const uint4*>(y + (size_t)r * H + c);
    float f[8];
    unpack8(v, f);
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = __builtin_fmaf(wt, f[i], acc[i]);
  }
  uint4 o;
  o.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
  o.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
  o.z = f32_to_bf16(acc[4]) | (f32_to_bf16(acc[5]) << 16);
  o.w = f32_to_bf16(acc[6]) | (f32_to_bf16(acc[7]) << 16);
  *reinterpret_cast<uint4*>(out + (size_t)t * H + c) = o;
}

inline unsigned blocks_for(int64_t n, int64_t per) { return (unsigned)((n + per - 1) / per); }

// The filtered / listed act+quant: the item kernel while n * gpr fits its
// 32-bit indexing (always, for the layer's route lists), else the flat
// kernel with the filter (list form: rejected).
hipError_t launch_items(const uint16_t* gu, int64_t n, const int32_t* list, const int32_t* count,
                        const RowFilter& f, int I, float limit, int fmt, uint8_t* q, float* s, hipStream_t stream) {
  const int clamp = __builtin_isfinite(limit) ? 1 : 0;
  const int64_t items = n * (I / kGroup);
  const dim3 grid(blocks_for(items, kGroupsPerBlock));
  const bool table = items >= kTableMinGroups;
  if (items > 0x7FFFFFFF) {
    if (list) return hipErrorInvalidValue;
    if (table)
      hipLaunchKernelGGL(silu_and_mul_quant_kernel<true>, grid, dim3(kThreads), 0, stream, gu, items, I, f, limit,
                         clamp, fmt, q, s);
    else
      hipLaunchKernelGGL(silu_and_mul_quant_kernel<false>, grid, dim3(kThreads), 0, stream, gu, items, I, f, limit,
                         clamp, fmt, q, s);
    return hipGetLastError();
  }
  const int nn = (int)n;
#define BFP8_ITEMS(T, LST)                                                                                    \
  hipLaunchKernelGGL((silu_and_mul_quant_items_kernel<T, LST>), grid, dim3(kThreads), 0, stream, gu, nn, list, \
                     count, f, I, limit, clamp, fmt, q, s)
  if (list) {
    if (table)
      BFP8_ITEMS(true, true);
    else
      BFP8_ITEMS(false, true);
  } else {
    if (table)
      BFP8_ITEMS(true, false);
    else
      BFP8_ITEMS(false, false);
  }
#undef BFP8_ITEMS
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_fp8(const uint16_t* x, int64_t rows, int K, int fmt, uint8_t* q, float* s,
                            hipStream_t stream) {
  const int64_t ng = rows * (K / kGroup);
  if (ng == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_fp8_kernel, dim3(blocks_for(ng, kGroupsPerBlock)), dim3(kThreads), 0, stream, x, ng,
                     K / kGroup, fmt, q, s);
  return hipGetLastError();
}

hipError_t launch_silu_and_mul(const uint16_t* gu, int64_t rows, int I, float limit, uint16_t* out,
                               hipStream_t stream) {
  const int64_t ng = rows * (I / kGroup);
  if (ng == 0) return hipSuccess;
  const int clamp = __builtin_isfinite(limit) ? 1 : 0;
  if (ng >= kTableMinGroups)
    hipLaunchKernelGGL(silu_and_mul_kernel<true>, dim3(blocks_for(ng, kGroupsPerBlock)), dim3(kThreads), 0, stream,
                       gu, ng, I, limit, clamp, out);
  else
    hipLaunchKernelGGL(silu_and_mul_kernel<false>, dim3(blocks_for(ng, kGroupsPerBlock)), dim3(kThreads), 0, stream,
                       gu, ng, I, limit, clamp, out);
  return hipGetLastError();
}

hipError_t launch_silu_and_mul_quant(const uint16_t* gu, int64_t rows, int I, const RowFilter& f, float limit,
                                     int fmt, uint8_t* q, float* s, hipStream_t stream) {
  const int64_t ng = rows * (I / kGroup);
  if (ng == 0) return hipSuccess;
  if (f.mode != kRowsAll) return launch_items(gu, rows, nullptr, nullptr, f, I, limit, fmt, q, s, stream);
  const int clamp = __builtin_isfinite(limit) ? 1 : 0;
  if (ng >= kTableMinGroups)
    hipLaunchKernelGGL(silu_and_mul_quant_kernel<true>, dim3(blocks_for(ng, kGroupsPerBlock)), dim3(kThreads), 0,
                       stream, gu, ng, I, f, limit, clamp, fmt, q, s);
  else
    hipLaunchKernelGGL(silu_and_mul_quant_kernel<false>, dim3(blocks_for(ng, kGroupsPerBlock)), dim3(kThreads), 0,
                       stream, gu, ng, I, f, limit, clamp, fmt, q, s);
  return hipGetLastError();
}

hipError_t launch_silu_and_mul_quant_list(const uint16_t* gu, const int32_t* list, const int32_t* count,
                                          int64_t n_list, int I, float limit, int fmt, uint8_t* q, float* s,
                                          hipStream_t stream) {
  if (n_list == 0) return hipSuccess;
  return launch_items(gu, n_list, list, count, RowFilter{}, I, limit, fmt, q, s, stream);
}

hipError_t launch_moe_reduce(const uint16_t* y, const float* w, const int32_t* ids, const ExpertSel& sel, int64_t M,
                             int k, int H, uint16_t* out, hipStream_t stream) {
  const int64_t n = M * (H / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(moe_reduce_kernel, dim3(blocks_for(n, kThreads)), dim3(kThreads), 0, stream, y, w, ids, sel, M,
                     k, H, out);
  return hipGetLastError();
}

}  // namespace bfp8
