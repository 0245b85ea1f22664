// stream_probe.hip -- read-bandwidth probe of the memory system (measurement
// only; no part of the layer).  It streams a device buffer in two shapes and
// keeps nothing but an unreachable store, so a launch costs what its loads
// cost:
//  - contiguous: workgroup b reads bytes [b S, (b + 1) S) of the buffer, S =
//    512 KiB, every thread 16 bytes per load, four loads in flight;
//  - tile: the buffer is rows of row_bytes, workgroup b reads rows 128 b ..
//    128 b + 127 as a grouped GEMM reads a weight tile: each of its 4 waves
//    takes 32 rows and walks K in pieces of `piece` bytes per row, each load
//    instruction covering 1024 / piece rows of one piece (8 rows x 128 bytes
//    at piece 128, the GEMM's shape), four loads in flight per wave;
//  - tile, rotated: as tile, but workgroup b starts its walk along K at piece
//    b mod (row_bytes / piece) and wraps around, so that workgroups running
//    side by side read different column ranges.
// Dynamic LDS (unused) sets how many workgroups share a compute unit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace bfp8 {

namespace {

constexpr int kProbeThreads = 256;
constexpr size_t kSlabBytes = 512 << 10;
constexpr int kInFlight = 4;
typedef unsigned int pu4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void probe_contig_kernel(const pu4* __restrict__ p, uint32_t* sink) {
  extern __shared__ uint32_t s_pad[];
  const size_t slab16 = kSlabBytes / 16;
  const pu4* b = p + (size_t)blockIdx.x * slab16;
  pu4 acc = {0u, 0u, 0u, 0u};
  for (size_t i = threadIdx.x; i < slab16; i += kProbeThreads * kInFlight) {
    pu4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; u++) v[u] = b[i + u * kProbeThreads];
#pragma unroll
    for (int u = 0; u < kInFlight; u++) acc ^= v[u];
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) {  // practically never: keeps the loads
    s_pad[0] = acc.x;
    sink[blockIdx.x] = s_pad[0];
  }
}

template <int P, bool kRotate>
__global__ __launch_bounds__(kProbeThreads) void probe_tile_kernel(const uint8_t* __restrict__ W, int K,
                                                                   uint32_t* sink) {
  extern __shared__ uint32_t s_pad[];
  constexpr int LPR = P / 16, RPI = 64 / LPR, RG = 32 / RPI;  // lanes per row, rows per load, row groups
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint8_t* base = W + ((size_t)blockIdx.x * 128 + wave * 32 + lane / LPR) * K + (lane % LPR) * 16;
  const int n_loads = K / 32;  // 1 KiB per load instruction, 32 rows of K bytes per wave
  const int n_pieces = K / P;
  const int rot = kRotate ? (int)(blockIdx.x % (unsigned)n_pieces) : 0;  // the workgroup's first piece
  auto ld = [&](int j) {
    j = j < n_loads - 1 ? j : n_loads - 1;
    int g = j / RG + rot;
    g = g < n_pieces ? g : g - n_pieces;
    const int rg = j % RG;
    return *reinterpret_cast<const pu4*>(base + (size_t)rg * RPI * K + (size_t)g * P);
  };
  pu4 a[kInFlight], c[kInFlight], acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int d = 0; d < kInFlight; d++) a[d] = ld(d);
  for (int j = kInFlight; j < n_loads; j += 2 * kInFlight) {
#pragma unroll
    for (int d = 0; d < kInFlight; d++) c[d] = ld(j + d);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < kInFlight; d++) acc ^= a[d];
#pragma unroll
    for (int d = 0; d < kInFlight; d++) a[d] = ld(j + kInFlight + d);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < kInFlight; d++) acc ^= c[d];
  }
#pragma unroll
  for (int d = 0; d < kInFlight; d++) acc ^= a[d];
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) {
    s_pad[0] = acc.x;
    sink[blockIdx.x] = s_pad[0];
  }
}

}  // namespace

int64_t stream_probe_grid(size_t bytes, int pattern, int row_bytes) {
  if (pattern == 0) return (int64_t)(bytes / kSlabBytes);
  return row_bytes > 0 ? (int64_t)(bytes / ((size_t)128 * row_bytes)) : 0;
}

hipError_t launch_stream_probe(const uint8_t* buf, size_t bytes, int pattern, int row_bytes, int piece,
                               int lds_bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t grid = stream_probe_grid(bytes, pattern, row_bytes);
  if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid), b(kProbeThreads);
  if (pattern == 0) {
    hipLaunchKernelGGL(probe_contig_kernel, g, b, lds_bytes, stream, reinterpret_cast<const pu4*>(buf), sink);
    return hipGetLastError();
  }
#define BFP8_PROBE_TILE(PC)                                                                                  \
  if (pattern == 2)                                                                                          \
    hipLaunchKernelGGL((probe_tile_kernel<PC, true>), g, b, lds_bytes, stream, buf, row_bytes, sink);         \
  else                                                                                                       \
    hipLaunchKernelGGL((probe_tile_kernel<PC, false>), g, b, lds_bytes, stream, buf, row_bytes, sink);
  switch (piece) {
    case 128:
      BFP8_PROBE_TILE(128)
      break;
    case 256:
      BFP8_PROBE_TILE(256)
      break;
    case 1024:
      BFP8_PROBE_TILE(1024)
      break;
    default:
      return hipErrorInvalidValue;
  }
#undef BFP8_PROBE_TILE
  return hipGetLastError();
}

}  // namespace bfp8
