// grouped_gemm.hip -- block-FP8 grouped GEMM over compact route blocks, gfx950.
//
// [P3 Purpose] W8A8 with [128, 128] weight blocks and 1x128 activation groups;
// [P2 Reviewed changes: w8a8.py] also per-row activation and per-channel
// weight scales (the W8A8 variant).
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
// into MFMA fragments through a per-wave LDS slice; for blocks of 32 or 64
// routes the workgroup loads each chunk of the block's activation rows once,
// as whole lines, into a shared LDS buffer that all 4 waves read their
// fragments from (see mfma.h for the K slot order).  The block's activation
// scales and the tile's weight scales are staged in LDS once per workgroup,
// and blocks of 16 and 32 routes keep two K chunks in flight.
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

// Most consecutive blocks of one expert whose workgroups share each weight
// tile through one XCD's L2 (a chunk; see the kernel).
constexpr int kChunkBlocks = 8;

// Dynamic LDS of the staged scales (grouped_gemm_kernel with kStage): BM
// rows of G + 1 activation scales and G weight scales, G = K / 128.  Staged
// from kStageMinGroups K steps (with fewer, the staging's own round trip
// costs more than the per-step loads it saves: measured) up to
// kStageMaxBytes (K up to 15,360 at 32 routes per block, 7,936 at 64), so
// that the workgroup's LDS stays well inside the 64 KB a launch gets.
constexpr int kStageMinGroups = 4;
constexpr size_t kStageMaxBytes = 16384;
inline size_t gemm_stage_bytes(int bm, int K) {
  const size_t G = (size_t)K / kGroup;
  return ((size_t)bm * (G + 1) + G) * sizeof(float);
}
inline bool gemm_stages(int bm, int K) {
  return K / kGroup >= kStageMinGroups && gemm_stage_bytes(bm, K) <= kStageMaxBytes;
}

// Workgroups per XCD for at most max_blocks route blocks of n_tiles tiles
// each: an XCD's range holds at most ceil(max_blocks / 8) blocks (workgroups
// past the range in use return at once).
inline int64_t gemm_slots_per_xcd(int64_t max_blocks, int n_tiles) {
  return (max_blocks + kXcd - 1) / kXcd * n_tiles;
}

// XCD-aware order of the work.  Workgroup i runs on XCD i % 8 as that XCD's
// slot i / 8 (workgroups are dealt to the XCDs round robin and each XCD takes
// its own in order).  The blocks in use [0, nb) are cut into 8 contiguous
// ranges of equal size, one per XCD; one expert's blocks are consecutive, so
// a range holds whole experts but at its two ends.  Within a range, each
// expert's blocks form chunks of up to kChunkBlocks consecutive blocks, run
// in order, and inside a chunk the tile index is outermost: the chunk's
// workgroups for one weight tile run side by side on one XCD, so the tile
// leaves HBM once per chunk and its other reads hit that XCD's L2, and a
// chunk's activation rows stay in L2 across its tiles.  Item s of the XCD
// lies in the chunk of block gq = lo + s / n_tiles (the chunk's items fill
// slots n_tiles (c0 - lo) .. n_tiles (c1 - lo) - 1).  Returns false for a
// workgroup past the work in use; else its weight tile nt and its block: the
// block's expert e, first position start in sorted_routes and route count
// len.  Block i of an expert starts at its segment start + i BM (the layout
// route preparation writes), so the block's own entries are not read again:
// the chain of dependent loads before the first weight load is the block
// count, then gq's expert and start, then that expert's segment bounds.
template <int BM>
__device__ __forceinline__ bool gemm_work(int n_tiles, const int32_t* __restrict__ expert_offsets,
                                          const int32_t* __restrict__ block_expert,
                                          const int32_t* __restrict__ block_start,
                                          const int32_t* __restrict__ num_blocks, int& nt, int& e, int& start,
                                          int& len) {
  // 32-bit index arithmetic: block counts are int32 and the grid is below
  // 2^31 workgroups (64-bit division is a long loop on this target)
  const unsigned x = blockIdx.x % kXcd;
  const unsigned slot = blockIdx.x / kXcd;
  const int64_t nb = *num_blocks;
  const int lo = (int)(nb * x / kXcd), hi = (int)(nb * (x + 1) / kXcd);
  if ((int64_t)slot >= (int64_t)(hi - lo) * n_tiles) return false;
  const int gq = lo + (int)(slot / (unsigned)n_tiles);
  const int eg = block_expert[gq];
  const int sq = block_start[gq];
  const int off_e = expert_offsets[eg];
  const int end_e = expert_offsets[eg + 1];
  const int ig = (sq - off_e) / BM;                        // gq among its expert's blocks
  const int nbe = (end_e - off_e + BM - 1) / BM;           // the expert's blocks
  const int cq = ig / kChunkBlocks * kChunkBlocks;         // chunk's first, in the expert
  const int c0 = max(gq - ig + cq, lo);
  const int c1 = min(gq - ig + min(cq + kChunkBlocks, nbe), hi);
  const unsigned r = slot - (unsigned)(c0 - lo) * (unsigned)n_tiles;
  const unsigned span = (unsigned)(c1 - c0);
  nt = (int)(r / span);
  const int blk = c0 + (int)(r % span);
  e = eg;
  start = off_e + (ig + blk - gq) * BM;
  len = min(BM, end_e - start);
  return true;
}

// Stages a block's activation scales in LDS: s_as[j * (G + 1) + g] for block
// row j (0 for a row without a route; the stride G + 1 keeps the 16 rows of
// one read in distinct banks).  Wave w writes rows w BM/4 .. (w + 1) BM/4 - 1;
// each lane takes items lane + 64 i (row, group) of its wave's rows, so one
// load instruction reads whole scale rows, and gets the row's route from the
// lane of its wave that holds it (route[t] of lane c is row 16 t + c).  The
// caller's next barrier makes them whole.
template <int BM>
__device__ __forceinline__ void stage_act_scales(float* __restrict__ s_as, const float* __restrict__ As,
                                                 int a_row_div, int G, const int (&route)[BM / 16], int lane,
                                                 int wave) {
  constexpr int CT = BM / 16, kRW = BM / 4;  // route tiles, rows per wave
  const int n_items = kRW * G;
  for (int b = 0; b < n_items; b += 64 * 8) {
    float v[8];
    int dst[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int it = b + lane + 64 * i;
      const int jw = min(it / G, kRW - 1), g = it - (it / G) * G;
      const int j = wave * kRW + jw;
      int rj = -1;
#pragma unroll
      for (int t = 0; t < CT; t++) {
        const int v_t = __shfl(route[t], j & 15);
        if ((j >> 4) == t) rj = v_t;
      }
      const bool ok = it < n_items && rj >= 0;
      v[i] = ok ? As[(size_t)(rj / a_row_div) * G + g] : 0.0f;
      dst[i] = it < n_items ? j * (G + 1) + g : -1;
    }
#pragma unroll
    for (int i = 0; i < 8; i++)
      if (dst[i] >= 0) s_as[dst[i]] = v[i];
  }
}

// Activation registers of one K step: 16-byte line pieces (shared path) or
// MFMA fragments (direct path).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <bool kShared, int XL, int CT>
struct XRegs {
  typedef u32x4_t type[XL];
};
template <int XL, int CT>
struct XRegs<false, XL, CT> {
  typedef v8i type[CT];
};

// kChannel (the W8A8 variant): As holds one scale per activation row and Bs
// one per weight row (output channel); the K loop adds the chunks' sums
// unscaled and the epilogue applies a_scale(route) * w_scale(row).
// kStage: the block's activation scales and the tile's weight scales are
// staged in LDS once (dynamic LDS of gemm_stage_bytes) instead of loaded per
// K step: a step's activation-scale loads touch one line per route, as many
// line requests as the weight chunk itself.
template <int BM, bool kChannel, bool kStage>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(BM == 64 ? 3 : 1))) void grouped_gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, int a_row_div, const uint8_t* __restrict__ B,
    const float* __restrict__ Bs, int N, int K, const int32_t* __restrict__ sorted_routes,
    const int32_t* __restrict__ expert_offsets, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ block_start, const int32_t* __restrict__ num_blocks, uint16_t* __restrict__ C) {
  constexpr int CT = BM / 16;                // route tiles
  constexpr int kAhead = BM <= 32 ? 2 : 1;   // K chunks in flight
  const int n_tiles = N / kBN;
  int nt, e, start, len;
  if (!gemm_work<BM>(n_tiles, expert_offsets, block_expert, block_start, num_blocks, nt, e, start, len)) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kq = lane >> 4;
  const int G = K / kGroup;

  // weight rows of this lane, and the first chunk's weight loads: they need
  // only the expert and the tile, so they leave before the route loads
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const int n0 = nt * kBN + wave * kWN;
  const uint8_t* wrow0 = B + ((size_t)e * N + n0) * K;  // the wave's first weight row
  const float* ws = kChannel ? Bs + (size_t)e * N + n0 : Bs + ((size_t)e * n_tiles + nt) * G;
  const uint8_t* wl = wrow0 + (size_t)(lane >> 3) * K + 16 * (lane & 7);  // load i adds 8 i rows
  u32x4 w0[4], w1[4];
#pragma unroll
  for (int i = 0; i < 4; i++) w0[i] = *reinterpret_cast<const u32x4*>(wl + (size_t)(8 * i) * K);
  float ws0 = kChannel || kStage ? 1.0f : ws[0], ws1 = 0.0f;

  // The activation chunks of blocks of 32 or 64 routes go through a buffer
  // shared by the workgroup; with 16 routes each wave loads its fragments
  // itself, which costs less than the barrier (measured).
  constexpr bool kSharedX = BM >= 32;
  // the routes of this lane's MFMA columns (route tile t, column col): their
  // activation rows and activation-scale rows
  const uint8_t* arow[CT];
  const float* asrow[CT];
  int route[CT];
  // shared path: the activation rows this thread loads, row tid / 8 + 32 x
  // of the block, bytes 16 (tid % 8) .. + 15 of each chunk (full 128-byte
  // lines; a row without a route reads activation row 0, and its columns are
  // never stored)
  constexpr int XL = kSharedX ? BM * 8 / kThreads : 1;  // 16-byte activation loads per thread
  const int tid = threadIdx.x;
  // Every route load is unconditional (position start + 0 stands in for a
  // column past the block's routes) and all leave before the first is used.
  int sr[CT], sx[XL];
#pragma unroll
  for (int t = 0; t < CT; t++) {
    const int j = t * 16 + col;
    sr[t] = sorted_routes[start + (j < len ? j : 0)];
  }
#pragma unroll
  for (int x = 0; x < XL; x++) {
    const int r = kSharedX ? (tid >> 3) + 32 * x : 0;
    sx[x] = sorted_routes[start + (r < len ? r : 0)];
  }
#pragma unroll
  for (int t = 0; t < CT; t++) {
    route[t] = t * 16 + col < len ? sr[t] : -1;
    const int64_t ar = route[t] >= 0 ? route[t] / a_row_div : 0;
    arow[t] = A + (size_t)ar * K;
    asrow[t] = As + (size_t)ar * (kChannel ? 1 : G);
  }
  const uint8_t* xrow[XL];
#pragma unroll
  for (int x = 0; x < XL; x++) {
    const int r = kSharedX ? (tid >> 3) + 32 * x : 0;
    const int rt = r < len ? sx[x] : -1;
    xrow[x] = A + (size_t)(rt >= 0 ? rt / a_row_div : 0) * K + 16 * (tid & 7);
  }

  // Staged scales: the block's activation scales (stage_act_scales), then
  // the tile's weight scales s_ws[g], written by wave 0.  The first step's
  // barrier (or, with no shared activation buffer, the one below) makes them
  // whole.
  extern __shared__ float s_dyn[];
  float* s_as = s_dyn;
  float* s_ws = s_dyn + BM * (G + 1);
  if constexpr (kStage) {
    stage_act_scales<BM>(s_as, As, a_row_div, G, route, lane, wave);
    if (wave == 0)
      for (int g = lane; g < G; g += 64) s_ws[g] = ws[g];
    if constexpr (!kSharedX) __syncthreads();
  }

  v4f acc[kRT][CT];
#pragma unroll
  for (int i = 0; i < kRT; i++)
#pragma unroll
    for (int t = 0; t < CT; t++) acc[i][t] = v4f{0.f, 0.f, 0.f, 0.f};

  // Chunks travel as full 128-byte lines and are turned into MFMA fragments
  // in LDS, 16-byte piece p of row r stored at piece p ^ (r & 7) against bank
  // conflicts (fragment reads take pieces kq and 4 + kq of the fragment's
  // rows, the K slot order of load_frag).
  //  - Weights: load i of a lane reads row 8 i + lane / 8 of the wave's 32
  //    rows (each load instruction covers 8 whole lines; the MFMA fragment
  //    pattern would cover 16 half lines and stream about a quarter slower).
  //    The wave writes the chunk to its own LDS slice and reads its fragments
  //    back; LDS accesses of one wave are carried out in order, so no barrier
  //    is needed.
  //  - Activations (shared path): the workgroup loads the block's rows once
  //    (not once per wave) into one of two shared buffers, alternating by
  //    step; one barrier per step makes the buffer whole before any wave
  //    reads it, and the barrier of the step before has seen every read of
  //    the buffer's previous contents.  Direct path: each wave loads its
  //    fragments (mfma.h K slot order), shared by the 4 waves through L1.
  __shared__ __align__(16) u32x4 s_w[kThreads / 64][kWN * 8];
  __shared__ __align__(16) u32x4 s_x[2][kSharedX ? BM * 8 : 1];
  u32x4* sw = s_w[wave];

  // The K loop keeps kAhead chunks in flight: chunk c is multiplied from
  // register set c % (kAhead + 1) while the loads of the next kAhead chunks
  // are out (two measured a little faster than one at blocks of 16 and 32
  // routes; blocks of 64 routes keep one, for registers).  fetch
  // requests chunk gn into (wn, xn, sn, wsn); use multiplies the chunk held
  // in (wc, xc, sc, wsc) through shared buffer xb.  The sets rotate, so
  // nothing is copied, and every load is issued before the chunk kAhead
  // steps older is used, so the wait before a multiply covers that chunk.
  auto fetch = [&](int gn, u32x4 (&wn)[4], auto& xn, float (&sn)[CT], float& wsn) __attribute__((always_inline)) {
    if constexpr (!kChannel && !kStage) {
      wsn = ws[gn];
#pragma unroll
      for (int t = 0; t < CT; t++) sn[t] = asrow[t][gn];
    }
#pragma unroll
    for (int i = 0; i < 4; i++) wn[i] = *reinterpret_cast<const u32x4*>(wl + (size_t)(8 * i) * K + (size_t)gn * kGroup);
    if constexpr (kSharedX) {
#pragma unroll
      for (int x = 0; x < XL; x++) xn[x] = *reinterpret_cast<const u32x4*>(xrow[x] + (size_t)gn * kGroup);
    } else {
#pragma unroll
      for (int t = 0; t < CT; t++) xn[t] = load_frag(arow[t] + (size_t)gn * kGroup, kq);
    }
  };
  auto use = [&](int gc, u32x4 (&wc)[4], auto& xc, float (&sc)[CT], float wsc, u32x4* xb)
      __attribute__((always_inline)) {
    if constexpr (kSharedX) {
#pragma unroll
      for (int x = 0; x < XL; x++) {
        const int r = (tid >> 3) + 32 * x;
        xb[r * 8 + ((tid & 7) ^ (r & 7))] = xc[x];
      }
    }
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
    if constexpr (kSharedX) {
      // the shared activation buffer is whole (LDS traffic only: the next
      // chunk's loads stay in flight)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
#pragma unroll
    for (int t = 0; t < CT; t++) {
      v8i xf;
      if constexpr (kSharedX) {
        const int r = 16 * t + col;
        const u32x4 lo = xb[r * 8 + (kq ^ (r & 7))];
        const u32x4 hi = xb[r * 8 + ((4 + kq) ^ (r & 7))];
        xf = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      } else {
        xf = xc[t];
      }
      float asc;
      if constexpr (kChannel)
        asc = route[t] >= 0 ? 1.0f : 0.0f;
      else if constexpr (kStage)
        asc = s_as[(16 * t + col) * (G + 1) + gc] * s_ws[gc];
      else
        asc = route[t] >= 0 ? sc[t] * wsc : 0.0f;
#pragma unroll
      for (int i = 0; i < kRT; i++) {
        const v4f p = mfma_f8_16x16x128(wa[i], xf, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int v = 0; v < 4; v++) acc[i][t][v] = __builtin_fmaf(p[v], asc, acc[i][t][v]);
      }
    }
  };

  typedef typename XRegs<kSharedX, XL, CT>::type XR;
  XR x0, x1;
  float s0[CT], s1[CT];
#pragma unroll
  for (int t = 0; t < CT; t++) s0[t] = kChannel || kStage ? 1.0f : asrow[t][0];
  if constexpr (kSharedX) {
#pragma unroll
    for (int x = 0; x < XL; x++) x0[x] = *reinterpret_cast<const u32x4*>(xrow[x]);
  } else {
#pragma unroll
    for (int t = 0; t < CT; t++) x0[t] = load_frag(arow[t], kq);
  }
  // The steps of an iteration run unconditionally (a fetch in a branch would
  // be moved into that branch, after the other steps' waits); requests past
  // the last chunk repeat it (cache hits, unused), and the chunks left after
  // the loop are already in their sets.  Chunk c goes through shared buffer
  // c % 2.
  int g = 0;
  if constexpr (kAhead == 2) {
    u32x4 w2[4];
    XR x2;
    float s2[CT], ws2 = 0.0f;
    fetch(min(1, G - 1), w1, x1, s1, ws1);
    for (; g + 2 < G; g += 3) {
      fetch(g + 2, w2, x2, s2, ws2);
      __builtin_amdgcn_sched_barrier(0);  // the loads leave before anything waits
      use(g, w0, x0, s0, ws0, s_x[g & 1]);
      fetch(min(g + 3, G - 1), w0, x0, s0, ws0);
      __builtin_amdgcn_sched_barrier(0);
      use(g + 1, w1, x1, s1, ws1, s_x[(g + 1) & 1]);
      fetch(min(g + 4, G - 1), w1, x1, s1, ws1);
      __builtin_amdgcn_sched_barrier(0);
      use(g + 2, w2, x2, s2, ws2, s_x[g & 1]);
    }
    if (g < G) use(g, w0, x0, s0, ws0, s_x[g & 1]);
    if (g + 1 < G) use(g + 1, w1, x1, s1, ws1, s_x[(g + 1) & 1]);
  } else {
    for (; g + 1 < G; g += 2) {
      fetch(g + 1, w1, x1, s1, ws1);
      __builtin_amdgcn_sched_barrier(0);
      use(g, w0, x0, s0, ws0, s_x[0]);
      fetch(min(g + 2, G - 1), w0, x0, s0, ws0);
      __builtin_amdgcn_sched_barrier(0);
      use(g + 1, w1, x1, s1, ws1, s_x[1]);
    }
    if (g < G) use(g, w0, x0, s0, ws0, s_x[0]);
  }

  // epilogue: lane holds rows n0 + 16*i + 4*kq + v (v = 0..3) of route[t]
  if constexpr (kChannel) {
    float4 wsv[kRT];
#pragma unroll
    for (int i = 0; i < kRT; i++) wsv[i] = *reinterpret_cast<const float4*>(ws + i * 16 + 4 * kq);
#pragma unroll
    for (int t = 0; t < CT; t++) {
      const float a_s = asrow[t][0];
#pragma unroll
      for (int i = 0; i < kRT; i++) {
        acc[i][t][0] *= a_s * wsv[i].x;
        acc[i][t][1] *= a_s * wsv[i].y;
        acc[i][t][2] *= a_s * wsv[i].z;
        acc[i][t][3] *= a_s * wsv[i].w;
      }
    }
  }
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

// ------------------------------------------------------------------ MXFP4 weights
//
// [P2 Reviewed changes: v4_fp4_grouped_gemm.py] the FP4-weight grouped GEMM.
// Reading (OCP Microscaling Formats v1.0): weight rows of E2M1 elements, two
// to a byte (the even element in the low nibble), one E8M0 scale byte per 32
// along K; activations E4M3 with one scale per 128, as in the block-FP8 GEMM.
// The MFMA takes A in FP4 and B in FP8 with an E8M0 scale per lane (mfma.h):
// a lane's FP4 slice is 32 consecutive K, one MX block, and its scale byte is
// that block's; its FP8 slice pairs with it in the hardware's FP8 order.
// Tile, order and pipeline as grouped_gemm_kernel; the K loop walks 256-wide
// chunks (two activation groups, eight MX blocks), so that a chunk of a
// packed weight row is one 128-byte line.  Per chunk and half h (K 128 h ..
// + 127 of the chunk) one MFMA per (row tile, route tile), its sum times the
// activation scale of group 2 c + h added to the fp32 accumulator.  The
// activation chunk (BM rows of 256 bytes) goes through a shared LDS buffer,
// 16-byte piece p of row r stored at p ^ (r & 15).
// kStage: the block's activation scales staged in LDS once (dynamic LDS of
// gemm_stage_bytes), as in grouped_gemm_kernel.  kStageW: the tile's weight
// scale bytes (128 rows x K / 32) staged in LDS once, for K / 128 a power of
// two from 4 to 32: per K step they were one
// 8-byte load per fragment row, 16 rows' lines per instruction.
template <int BM, bool kStage, bool kStageW>
__global__ __launch_bounds__(kThreads) void grouped_gemm_mxfp4_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, int a_row_div, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, int N, int K, const int32_t* __restrict__ sorted_routes,
    const int32_t* __restrict__ expert_offsets, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ block_start, const int32_t* __restrict__ num_blocks, uint16_t* __restrict__ C) {
  constexpr int CT = BM / 16;              // route tiles
  constexpr int XL = BM * 16 / kThreads;   // 16-byte activation pieces per thread per chunk
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const int n_tiles = N / kBN;
  int nt, e, start, len;
  if (!gemm_work<BM>(n_tiles, expert_offsets, block_expert, block_start, num_blocks, nt, e, start, len)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, kq = lane >> 4;
  const int G = K / kGroup, KB = K / 2, NS = K / 32;  // groups, packed row bytes, scale bytes per row
  const int nch = K / 256;                            // K chunks

  // weight rows: load i of a lane reads row 8 i + lane / 8 of the wave's 32,
  // bytes 16 (lane % 8) .. + 15 of the chunk's line; the scale bytes of the
  // lane's fragment rows 16 i + col.  The first chunk's weight loads leave
  // before the route loads (they need only the expert and the tile).
  const int n0 = nt * kBN + wave * kWN;
  const uint8_t* wl = B + ((size_t)e * N + n0 + (lane >> 3)) * KB + 16 * (lane & 7);
  const uint8_t* wsr[kRT];
#pragma unroll
  for (int i = 0; i < kRT; i++) wsr[i] = Bs + ((size_t)e * N + n0 + 16 * i + col) * NS;
  u32x4 w0[4], w1[4];
  uint2 b0[kRT], b1[kRT];
#pragma unroll
  for (int i = 0; i < 4; i++) w0[i] = *reinterpret_cast<const u32x4*>(wl + (size_t)(8 * i) * KB);
  if constexpr (!kStageW) {
#pragma unroll
    for (int i = 0; i < kRT; i++) b0[i] = *reinterpret_cast<const uint2*>(wsr[i]);
  }

  // the routes of this lane's MFMA columns and their activation-scale rows,
  // and the activation pieces this thread loads: piece q = tid + 256 x of
  // the block's BM x 16, row q / 16, global piece q % 16 (a row without a
  // route reads activation row 0; its columns are never stored).  Route
  // loads are unconditional and all leave first, as in grouped_gemm_kernel.
  int sr[CT], sx[XL];
#pragma unroll
  for (int t = 0; t < CT; t++) {
    const int j = t * 16 + col;
    sr[t] = sorted_routes[start + (j < len ? j : 0)];
  }
#pragma unroll
  for (int x = 0; x < XL; x++) {
    const int r = (tid + kThreads * x) >> 4;
    sx[x] = sorted_routes[start + (r < len ? r : 0)];
  }
  const float* asrow[CT];
  int route[CT];
#pragma unroll
  for (int t = 0; t < CT; t++) {
    route[t] = t * 16 + col < len ? sr[t] : -1;
    asrow[t] = As + (size_t)(route[t] >= 0 ? route[t] / a_row_div : 0) * G;
  }
  const uint8_t* xrow[XL];
#pragma unroll
  for (int x = 0; x < XL; x++) {
    const int q = tid + kThreads * x, r = q >> 4;
    const int rt = r < len ? sx[x] : -1;
    xrow[x] = A + (size_t)(rt >= 0 ? rt / a_row_div : 0) * K + 16 * (q & 15);
  }

  v4f acc[kRT][CT];
#pragma unroll
  for (int i = 0; i < kRT; i++)
#pragma unroll
    for (int t = 0; t < CT; t++) acc[i][t] = v4f{0.f, 0.f, 0.f, 0.f};

  __shared__ __align__(16) u32x4 s_w[kThreads / 64][kWN * 8];
  __shared__ __align__(16) u32x4 s_x[2][BM * 16];
  u32x4* sw = s_w[wave];

  // One K step: request chunk cn into the next register set, then multiply
  // the chunk held in the current one through shared buffer xb (as in
  // grouped_gemm_kernel: two sets alternate, every load unconditional and
  // issued before the current chunk is used).
  extern __shared__ float s_dyn[];
  float* s_as = s_dyn;
  if constexpr (kStage) stage_act_scales<BM>(s_as, As, a_row_div, G, route, lane, wave);
  // staged weight scale bytes: word w of tile row r (bytes 4 w .. 4 w + 3 of
  // its NS) at word w ^ (r % NW) of the row, NW = NS / 4 words per row (a
  // power of two), so that the 16 rows of one read fall in distinct banks;
  // the rows of a tile are contiguous in Bs, read 16 bytes per thread
  __shared__ uint32_t s_wsc[kStageW ? kBN * 32 : 1];
  const int NW = NS / 4;
  if constexpr (kStageW) {
    const uint8_t* wt = Bs + ((size_t)e * N + (size_t)nt * kBN) * NS;
    for (int q = tid; q < kBN * NS / 16; q += kThreads) {
      const uint4 v = *reinterpret_cast<const uint4*>(wt + 16 * (size_t)q);
      const int r = 16 * q / NS, w = (16 * q - r * NS) / 4;
      uint32_t* row = s_wsc + r * NW;
      row[(w + 0) ^ (r & (NW - 1))] = v.x;
      row[(w + 1) ^ (r & (NW - 1))] = v.y;
      row[(w + 2) ^ (r & (NW - 1))] = v.z;
      row[(w + 3) ^ (r & (NW - 1))] = v.w;
    }
  }

  auto step = [&](int cn, int cc, u32x4 (&wc)[4], u32x4 (&xc)[XL], float (&sc)[CT][2], uint2 (&bc)[kRT],
                  u32x4 (&wn)[4], u32x4 (&xn)[XL], float (&sn)[CT][2], uint2 (&bn)[kRT], u32x4* xb)
      __attribute__((always_inline)) {
    if constexpr (!kStage) {
#pragma unroll
      for (int t = 0; t < CT; t++) {
        sn[t][0] = asrow[t][2 * cn];
        sn[t][1] = asrow[t][2 * cn + 1];
      }
    }
    if constexpr (!kStageW) {
#pragma unroll
      for (int i = 0; i < kRT; i++) bn[i] = *reinterpret_cast<const uint2*>(wsr[i] + 8 * cn);
    }
#pragma unroll
    for (int i = 0; i < 4; i++) wn[i] = *reinterpret_cast<const u32x4*>(wl + (size_t)(8 * i) * KB + (size_t)cn * 128);
#pragma unroll
    for (int x = 0; x < XL; x++) xn[x] = *reinterpret_cast<const u32x4*>(xrow[x] + (size_t)cn * 256);
    __builtin_amdgcn_sched_barrier(0);  // the loads leave before anything waits
#pragma unroll
    for (int x = 0; x < XL; x++) {
      const int q = tid + kThreads * x, r = q >> 4;
      xb[r * 16 + ((q & 15) ^ (r & 15))] = xc[x];
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = 8 * i + (lane >> 3);
      sw[r * 8 + ((lane & 7) ^ (r & 7))] = wc[i];
    }
    // A fragments: row 16 i + col, bytes 64 h + 16 kq .. + 15 (piece 4 h + kq)
    v8i wa[kRT][2];
#pragma unroll
    for (int i = 0; i < kRT; i++) {
      const int r = 16 * i + col;
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const u32x4 v = sw[r * 8 + ((4 * h + kq) ^ (r & 7))];
        wa[i][h] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      }
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the shared buffer is written
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int t = 0; t < CT; t++) {
      const int r = 16 * t + col;
#pragma unroll
      for (int h = 0; h < 2; h++) {
        // B fragment: route row r, bytes 128 h + 16 kq .. + 15 and 128 h + 64
        // + 16 kq .. + 15 (pieces 8 h + kq and 8 h + 4 + kq)
        const u32x4 lo = xb[r * 16 + ((8 * h + kq) ^ (r & 15))];
        const u32x4 hi = xb[r * 16 + ((8 * h + 4 + kq) ^ (r & 15))];
        const v8i xf = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        const float asc = kStage ? s_as[(16 * t + col) * (G + 1) + 2 * cc + h] : route[t] >= 0 ? sc[t][h] : 0.0f;
#pragma unroll
        for (int i = 0; i < kRT; i++) {
          int e8;
          if constexpr (kStageW) {
            // MX block 8 cc + 4 h + kq of tile row wave 32 + 16 i + col: byte kq of word 2 cc + h
            const int r = wave * kWN + 16 * i + col;
            e8 = (int)((s_wsc[r * NW + ((2 * cc + h) ^ (r & (NW - 1)))] >> (8 * kq)) & 0xFFu);
          } else {
            e8 = (int)(((h ? bc[i].y : bc[i].x) >> (8 * kq)) & 0xFFu);
          }
          const v4f p = mfma_f4f8_16x16x128(wa[i][h], xf, e8, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int v = 0; v < 4; v++) acc[i][t][v] = __builtin_fmaf(p[v], asc, acc[i][t][v]);
        }
      }
    }
  };

  u32x4 x0[XL], x1[XL];
  float s0[CT][2], s1[CT][2];
#pragma unroll
  for (int t = 0; t < CT; t++) {
    s0[t][0] = kStage ? 1.0f : asrow[t][0];
    s0[t][1] = kStage ? 1.0f : asrow[t][1];
  }
#pragma unroll
  for (int x = 0; x < XL; x++) x0[x] = *reinterpret_cast<const u32x4*>(xrow[x]);
  int c = 0;
  for (; c + 1 < nch; c += 2) {
    step(c + 1, c, w0, x0, s0, b0, w1, x1, s1, b1, s_x[0]);
    step(min(c + 2, nch - 1), c + 1, w1, x1, s1, b1, w0, x0, s0, b0, s_x[1]);
  }
  if (c < nch) step(c, c, w0, x0, s0, b0, w1, x1, s1, b1, s_x[0]);

  // epilogue: lane holds rows n0 + 16 i + 4 kq + v (v = 0..3) of route[t]
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
                               int block_m, uint16_t* C, hipStream_t stream, bool channel) {
  if (max_blocks == 0 || N / kBN == 0) return hipSuccess;
  const int64_t grid = gemm_slots_per_xcd(max_blocks, N / kBN) * kXcd;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
#define BFP8_GEMM_CASE(BMV)                                                                                     \
  case BMV:                                                                                                     \
    if (channel)                                                                                                \
      hipLaunchKernelGGL((grouped_gemm_kernel<BMV, true, false>), dim3((unsigned)grid), dim3(kThreads), 0, stream, \
                         A, As, a_row_div, B, Bs, N, K, sorted_routes, expert_offsets, block_expert, block_start,    \
                         num_blocks, C);                                                                       \
    else if (gemm_stages(BMV, K))                                                                               \
      hipLaunchKernelGGL((grouped_gemm_kernel<BMV, false, true>), dim3((unsigned)grid), dim3(kThreads),          \
                         gemm_stage_bytes(BMV, K), stream, A, As, a_row_div, B, Bs, N, K, sorted_routes,          \
                         expert_offsets, block_expert, block_start, num_blocks, C);                              \
    else                                                                                                        \
      hipLaunchKernelGGL((grouped_gemm_kernel<BMV, false, false>), dim3((unsigned)grid), dim3(kThreads), 0,       \
                         stream, A, As, a_row_div, B, Bs, N, K, sorted_routes, expert_offsets, block_expert,      \
                         block_start, num_blocks, C);                                                          \
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

hipError_t launch_grouped_gemm_mxfp4(const uint8_t* A, const float* As, int a_row_div, const uint8_t* B,
                                     const uint8_t* Bs, int N, int K, const int32_t* sorted_routes,
                                     const int32_t* expert_offsets, const int32_t* block_expert,
                                     const int32_t* block_start, const int32_t* num_blocks, int64_t max_blocks,
                                     int block_m, uint16_t* C, hipStream_t stream) {
  if (max_blocks == 0 || N / kBN == 0) return hipSuccess;
  if (K % 256 != 0) return hipErrorInvalidValue;  // the caller checks
  const int64_t grid = gemm_slots_per_xcd(max_blocks, N / kBN) * kXcd;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  // the tile's weight scales staged from K = 512 to 4096 with K / 128 a power of two
  const int kg = K / kGroup;
  const bool stage_w = kg >= 4 && kg <= 32 && (kg & (kg - 1)) == 0;
#define BFP8_MX_LAUNCH(BMV, ST, SW)                                                                            \
  hipLaunchKernelGGL((grouped_gemm_mxfp4_kernel<BMV, ST, SW>), dim3((unsigned)grid), dim3(kThreads),           \
                     ST ? (size_t)BMV * (K / kGroup + 1) * sizeof(float) : 0, stream, A, As, a_row_div, B, Bs, N,  \
                     K, sorted_routes, expert_offsets, block_expert, block_start, num_blocks, C)
#define BFP8_MX_CASE(BMV)                                                                                      \
  case BMV:                                                                                                    \
    if (gemm_stages(BMV, K) && stage_w)                                                                        \
      BFP8_MX_LAUNCH(BMV, true, true);                                                                         \
    else if (gemm_stages(BMV, K))                                                                              \
      BFP8_MX_LAUNCH(BMV, true, false);                                                                        \
    else if (stage_w)                                                                                          \
      BFP8_MX_LAUNCH(BMV, false, true);                                                                        \
    else                                                                                                       \
      BFP8_MX_LAUNCH(BMV, false, false);                                                                       \
    break;
  switch (block_m) {
    BFP8_MX_CASE(16)
    BFP8_MX_CASE(32)
    BFP8_MX_CASE(64)
    default:
      return hipErrorInvalidValue;
  }
#undef BFP8_MX_CASE
#undef BFP8_MX_LAUNCH
  return hipGetLastError();
}

}  // namespace bfp8
