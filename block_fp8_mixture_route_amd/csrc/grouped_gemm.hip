// grouped_gemm.hip -- block-FP8 grouped GEMM over compact route blocks, gfx950.
//
// [P3 Purpose] W8A8 with [128, 128] weight blocks and 1x128 activation groups.
// [P1 Modification, Active-expert block scheduling] one workgroup tile per
// (compact block, 128 output rows); tiles past the device-side block count
// exit at once, so inactive experts cost nothing but an early return.
// [P2 Changes] small-M tiles use the MMA with operand roles swapped: expert
// weight rows fill the MFMA's 16-row A slot and routes its 16-column B slot.
//
// Tile: 128 weight rows x BM routes, 4 waves of 32 rows each.  The K loop walks
// 128-wide chunks, exactly one scale group: each chunk's MFMA result is
// multiplied by a_scale(route, g) * w_scale(row block, g) and added to the fp32
// accumulator.  Operands come straight from global memory into registers (see
// mfma.h for the K slot order that keeps each load 64-byte contiguous per row);
// the activation fragments are shared by the 4 waves through L1.
//
// Pages cited in brackets, by key and section:
//   [P1] lmdeploy PR "Perf/pytorch block fp8 moe decode"
//   [P2] lmdeploy PR "perf(pytorch): optimize compact blocked FP8 MoE and route
//        preparation"
//   [P3] vLLM PR "[Kernel][Perf] Fuse clamped MoE activation and UE8M0 FP8 block
//        quantization"
//   [P4] lmdeploy PR "Moe Reduce kernel"
#include "device.h"
#include "internal.h"
#include "mfma.h"

namespace bfp8 {

namespace {

constexpr int kThreads = 256;
constexpr int kBN = 128;      // weight rows per workgroup (one scale block)
constexpr int kWN = 32;       // weight rows per wave
constexpr int kRT = kWN / 16; // row tiles per wave
constexpr int kXcd = 8;       // MI355X: workgroups are dealt round-robin to 8 XCDs

template <int BM>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, int a_row_div, const uint8_t* __restrict__ B,
    const float* __restrict__ Bs, int N, int K, const int32_t* __restrict__ sorted_routes,
    const int32_t* __restrict__ expert_offsets, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ block_start, const int32_t* __restrict__ num_blocks, int64_t n_tiles_total,
    uint16_t* __restrict__ C) {
  constexpr int CT = BM / 16;  // route tiles
  const int n_tiles = N / kBN;
  // XCD-aware order: XCD x works on a contiguous range of logical tiles, with
  // the 128-row tiles of one block adjacent, so one expert's weights and one
  // block's activations stay within one XCD's L2.
  const int64_t per_xcd = (n_tiles_total + kXcd - 1) / kXcd;
  const int64_t logical = (int64_t)(blockIdx.x % kXcd) * per_xcd + blockIdx.x / kXcd;
  if (logical >= n_tiles_total) return;
  const int64_t blk = logical / n_tiles;
  const int nt = (int)(logical - blk * n_tiles);
  if (blk >= *num_blocks) return;

  const int e = block_expert[blk];
  const int start = block_start[blk];
  const int end_e = expert_offsets[e + 1];
  const int len = min(BM, end_e - start);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kq = lane >> 4;
  const int G = K / kGroup;

  // activation rows of this lane's routes
  const uint8_t* arow[CT];
  const float* asrow[CT];
  int route[CT];
#pragma unroll
  for (int t = 0; t < CT; t++) {
    const int j = t * 16 + col;
    route[t] = j < len ? sorted_routes[start + j] : -1;
    const int64_t ar = route[t] >= 0 ? route[t] / a_row_div : 0;
    arow[t] = A + (size_t)ar * K;
    asrow[t] = As + (size_t)ar * G;
  }
  // weight rows of this lane
  const int n0 = nt * kBN + wave * kWN;
  const uint8_t* wrow[kRT];
#pragma unroll
  for (int t = 0; t < kRT; t++) wrow[t] = B + ((size_t)e * N + n0 + t * 16 + col) * K;
  const float* ws = Bs + ((size_t)e * n_tiles + nt) * G;

  v4f acc[kRT][CT];
#pragma unroll
  for (int i = 0; i < kRT; i++)
#pragma unroll
    for (int t = 0; t < CT; t++) acc[i][t] = v4f{0.f, 0.f, 0.f, 0.f};

  v8i wa[kRT], xb[CT];
#pragma unroll
  for (int i = 0; i < kRT; i++) wa[i] = load_frag(wrow[i], kq);
#pragma unroll
  for (int t = 0; t < CT; t++) xb[t] = route[t] >= 0 ? load_frag(arow[t], kq) : zero_frag();

  for (int g = 0; g < G; g++) {
    // prefetch the next chunk while this one is multiplied
    v8i wn[kRT], xn[CT];
    const int gn = g + 1 < G ? g + 1 : g;
#pragma unroll
    for (int i = 0; i < kRT; i++) wn[i] = load_frag(wrow[i] + (size_t)gn * kGroup, kq);
#pragma unroll
    for (int t = 0; t < CT; t++) xn[t] = route[t] >= 0 ? load_frag(arow[t] + (size_t)gn * kGroup, kq) : zero_frag();

    const float wsc = ws[g];
    float asc[CT];
#pragma unroll
    for (int t = 0; t < CT; t++) asc[t] = route[t] >= 0 ? asrow[t][g] * wsc : 0.0f;

#pragma unroll
    for (int i = 0; i < kRT; i++) {
#pragma unroll
      for (int t = 0; t < CT; t++) {
        v4f p = mfma_f8_16x16x128(wa[i], xb[t], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int v = 0; v < 4; v++) acc[i][t][v] = __builtin_fmaf(p[v], asc[t], acc[i][t][v]);
      }
    }
#pragma unroll
    for (int i = 0; i < kRT; i++) wa[i] = wn[i];
#pragma unroll
    for (int t = 0; t < CT; t++) xb[t] = xn[t];
  }

  // epilogue: lane holds rows n0 + 16*i + 4*kq + v (v = 0..3) of route[t]
#pragma unroll
  for (int t = 0; t < CT; t++) {
    if (route[t] < 0) continue;
    uint16_t* crow = C + (size_t)route[t] * N + n0;
#pragma unroll
    for (int i = 0; i < kRT; i++) {
      uint2 o;
      o.x = f32_to_bf16(acc[i][t][0]) | (f32_to_bf16(acc[i][t][1]) << 16);
      o.y = f32_to_bf16(acc[i][t][2]) | (f32_to_bf16(acc[i][t][3]) << 16);
      *reinterpret_cast<uint2*>(crow + i * 16 + 4 * kq) = o;
    }
  }
}

}  // namespace

hipError_t launch_grouped_gemm(const uint8_t* A, const float* As, int a_row_div, const uint8_t* B,
                               const float* Bs, int N, int K, const int32_t* sorted_routes,
                               const int32_t* expert_offsets, const int32_t* block_expert,
                               const int32_t* block_start, const int32_t* num_blocks, int64_t max_blocks,
                               int block_m, uint16_t* C, hipStream_t stream) {
  const int64_t total = max_blocks * (N / kBN);
  if (total == 0) return hipSuccess;
  const int64_t grid = (total + kXcd - 1) / kXcd * kXcd;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
#define BFP8_GEMM_CASE(BMV)                                                                                   \
  case BMV:                                                                                                   \
    hipLaunchKernelGGL(grouped_gemm_kernel<BMV>, dim3((unsigned)grid), dim3(kThreads), 0, stream, A, As,      \
                       a_row_div, B, Bs, N, K, sorted_routes, expert_offsets, block_expert, block_start,     \
                       num_blocks, total, C);                                                                \
    break;
  switch (block_m) {
    BFP8_GEMM_CASE(16)
    BFP8_GEMM_CASE(32)
    BFP8_GEMM_CASE(64)
    default:
      return hipErrorInvalidValue;
  }
#undef BFP8_GEMM_CASE
  return hipGetLastError();
}

}  // namespace bfp8
