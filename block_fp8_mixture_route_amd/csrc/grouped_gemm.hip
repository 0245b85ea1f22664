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
// accumulator.  Weight chunks are loaded as whole 128-byte lines and turned
// into MFMA fragments through a per-wave LDS slice; activation fragments come
// straight from global memory into registers (see mfma.h for the K slot
// order) and are shared by the 4 waves through L1.
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

// Route blocks scheduled together on one XCD (see the kernel): pairs from
// 512 possible blocks up (64 per XCD), single blocks below, where the
// balance across XCDs counts for more than shared weight reads (measured).
inline int gemm_group_blocks(int64_t max_blocks) { return max_blocks >= 64 * kXcd ? 2 : 1; }

// Workgroups per XCD for max_blocks route blocks of n_tiles tiles each in
// groups of gb: every XCD gets the same number of groups (the last groups
// may be partial or past the end: their workgroups return at once).
inline int64_t gemm_slots_per_xcd(int64_t max_blocks, int n_tiles, int gb) {
  const int64_t groups = (max_blocks + gb - 1) / gb;
  return (groups + kXcd - 1) / kXcd * gb * n_tiles;
}

template <int BM>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, int a_row_div, const uint8_t* __restrict__ B,
    const float* __restrict__ Bs, int N, int K, const int32_t* __restrict__ sorted_routes,
    const int32_t* __restrict__ expert_offsets, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ block_start, const int32_t* __restrict__ num_blocks, int64_t max_blocks,
    int group_blocks, uint16_t* __restrict__ C) {
  constexpr int CT = BM / 16;  // route tiles
  const int n_tiles = N / kBN;
  // XCD-aware order.  Route blocks form groups of group_blocks consecutive
  // blocks, dealt round-robin to the XCDs, so that the blocks in use (a
  // prefix of max_blocks) keep every XCD busy.  An XCD runs its groups one
  // after another, and within a group the tile index outermost: the same
  // weight tile of consecutive blocks -- one expert's blocks are consecutive
  // -- is read by adjacent workgroups on one XCD, and its second read is an
  // L2 hit; a block's activations are reused by its tiles on that XCD too.
  const int64_t slot = blockIdx.x / kXcd;
  const int64_t T = (int64_t)group_blocks * n_tiles;
  const int64_t b0 = ((slot / T) * kXcd + blockIdx.x % kXcd) * group_blocks;
  if (b0 >= max_blocks) return;
  const int gb = (int)min((int64_t)group_blocks, max_blocks - b0);  // blocks in this group
  const int within = (int)(slot % T);
  if (within >= gb * n_tiles) return;
  const int64_t blk = b0 + within % gb;
  const int nt = within / gb;
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
  const uint8_t* wrow0 = B + ((size_t)e * N + n0) * K;  // the wave's first weight row
  const float* ws = Bs + ((size_t)e * n_tiles + nt) * G;

  v4f acc[kRT][CT];
#pragma unroll
  for (int i = 0; i < kRT; i++)
#pragma unroll
    for (int t = 0; t < CT; t++) acc[i][t] = v4f{0.f, 0.f, 0.f, 0.f};

  // Weight chunks travel as full 128-byte lines: load i of a lane reads row
  // 8 i + lane / 8 of the wave's 32 rows, bytes 16 (lane % 8) .. + 15 of the
  // chunk (each load instruction covers 8 whole lines; the MFMA fragment
  // pattern would cover 16 half lines and stream about a quarter slower).  The
  // wave writes the chunk to its own LDS slice -- 16-byte piece p of row r at
  // piece p ^ (r & 7), against bank conflicts -- and reads its fragments
  // back.  Only the wave itself touches its slice, and LDS accesses of one
  // wave are carried out in order, so no barrier is needed.
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  __shared__ __align__(16) u32x4 s_w[kThreads / 64][kWN * 8];
  u32x4* sw = s_w[wave];
  const uint8_t* wl = wrow0 + (size_t)(lane >> 3) * K + 16 * (lane & 7);  // load i adds 8 i rows

  // One K step: request chunk gn into (wn, xn, sn, wsn), then multiply the
  // chunk held in (wc, xc, sc, wsc).  Two register sets alternate, so nothing is
  // copied.  Every load is unconditional -- a lane without a route reads
  // activation row 0 and its columns are never stored -- and the next
  // chunk's loads are all issued before the current chunk is used, so the
  // wait before the multiply covers the current chunk only.
  auto step = [&](int gn, u32x4 (&wc)[4], v8i (&xc)[CT], float (&sc)[CT], float wsc, u32x4 (&wn)[4],
                  v8i (&xn)[CT], float (&sn)[CT], float& wsn) __attribute__((always_inline)) {
    wsn = ws[gn];
#pragma unroll
    for (int t = 0; t < CT; t++) sn[t] = asrow[t][gn];
#pragma unroll
    for (int i = 0; i < 4; i++) wn[i] = *reinterpret_cast<const u32x4*>(wl + (size_t)(8 * i) * K + (size_t)gn * kGroup);
#pragma unroll
    for (int t = 0; t < CT; t++) xn[t] = load_frag(arow[t] + (size_t)gn * kGroup, kq);
    __builtin_amdgcn_sched_barrier(0);  // the loads leave before anything waits
    // this chunk through the wave's LDS slice into MFMA fragments (K slots
    // as in load_frag: pieces kq and 4 + kq of the fragment's row)
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = 8 * i + (lane >> 3);
      sw[r * 8 + ((lane & 7) ^ (r & 7))] = wc[i];
    }
    v8i wa[kRT];
#pragma unroll
    for (int i = 0; i < kRT; i++) {
      const int r = 16 * i + col;
      const u32x4 lo = sw[r * 8 + (kq ^ (r & 7))];
      const u32x4 hi = sw[r * 8 + ((4 + kq) ^ (r & 7))];
      wa[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int t = 0; t < CT; t++) {
      const float asc = route[t] >= 0 ? sc[t] * wsc : 0.0f;
#pragma unroll
      for (int i = 0; i < kRT; i++) {
        const v4f p = mfma_f8_16x16x128(wa[i], xc[t], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int v = 0; v < 4; v++) acc[i][t][v] = __builtin_fmaf(p[v], asc, acc[i][t][v]);
      }
    }
  };

  u32x4 w0[4], w1[4];
  v8i x0[CT], x1[CT];
  float s0[CT], s1[CT];
  float ws0 = ws[0], ws1 = 0.0f;
#pragma unroll
  for (int t = 0; t < CT; t++) s0[t] = asrow[t][0];
#pragma unroll
  for (int i = 0; i < 4; i++) w0[i] = *reinterpret_cast<const u32x4*>(wl + (size_t)(8 * i) * K);
#pragma unroll
  for (int t = 0; t < CT; t++) x0[t] = load_frag(arow[t], kq);
  // both steps of an iteration run unconditionally (a step in a branch would
  // have its loads moved into that branch, after the other step's wait); an
  // odd chunk count ends with one more step.  The last step's request
  // repeats the last chunk (cache hits, unused).
  int g = 0;
  for (; g + 1 < G; g += 2) {
    step(g + 1, w0, x0, s0, ws0, w1, x1, s1, ws1);
    step(min(g + 2, G - 1), w1, x1, s1, ws1, w0, x0, s0, ws0);
  }
  if (g < G) step(g, w0, x0, s0, ws0, w1, x1, s1, ws1);

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
  if (max_blocks == 0 || N / kBN == 0) return hipSuccess;
  const int gb = gemm_group_blocks(max_blocks);
  const int64_t grid = gemm_slots_per_xcd(max_blocks, N / kBN, gb) * kXcd;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
#define BFP8_GEMM_CASE(BMV)                                                                                   \
  case BMV:                                                                                                   \
    hipLaunchKernelGGL(grouped_gemm_kernel<BMV>, dim3((unsigned)grid), dim3(kThreads), 0, stream, A, As,      \
                       a_row_div, B, Bs, N, K, sorted_routes, expert_offsets, block_expert, block_start,     \
                       num_blocks, max_blocks, gb, C);                                                       \
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
