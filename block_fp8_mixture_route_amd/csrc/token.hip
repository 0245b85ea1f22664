// token.hip -- the block-FP8 MoE layer for a few tokens (M <= 32, the decode
// regime) on gfx950 as two weight-streaming kernels.
//
// [P1 Motivation] at M = 1, top-k 8, E = 256 at most eight experts are active
// and the layer is pure weight streaming: 44 MB of W13 + W2 at the 7168 x 256
// decode shape against 88 MFLOP.  Both projections are matrix-vector
// products, so they run on the vector ALUs from row-contiguous loads (every
// wave load instruction reads 1 KB of one weight row), not on MFMA tiles whose
// operand layout scatters each load over 16 rows.
// [P1 Modification, Active-expert block scheduling] only the active routes'
// rows are read: gate/up workgroups exist per route, and a route whose expert
// lies outside the local slice exits at once.
// [P1 Modification, Fused SwiGLU and FP8 quantization] SwiGLU is applied in the
// gate/up epilogue; its BF16 output is group-quantised where the down
// projection consumes it.
// [P4 Pull request overview] the down projection ends with the top-k weighted
// reduction, routes in order.
//
// The column waves' wait for the hidden row is bounded; running out of it
// ends the kernel normally and sets a device flag the host can read
// (bfp8moe_wait_faults).
//
// gate/up kernel: workgroup (route j, slice q) computes columns n = 8 q .. 8 q
//   + 7 of route j's SwiGLU row (route j = t k + r belongs to token t), one
//   column (gate row n and up row I + n) per column wave, each written as one
//   BF16 value into act[j]; the other 8 waves prepare the token's quantised
//   hidden row in LDS.  Each route reads its expert's rows: with top-k routing
//   the routes of one token have distinct experts, and at a few tokens the
//   rows that two tokens share are a small part of the stream.
// With the router folded in ([P2 Changes: the fused single-group top-k router
//   feeds the layer]), one wave of each gate/up workgroup ranks the token's
//   logits up to the route's rank first, and one wave per token writes the
//   routing the down kernel reads.
// down kernel: workgroup (b, t) computes output rows DR b .. DR b + DR - 1 of
//   token t for its k routes from their W2 pieces (1 KB units: route, kRpl
//   rows of I bytes), quantises the k SwiGLU rows itself, and ends with the
//   weighted reduction.
//
// The kernel boundary is the only exchange.  Within one kernel a compute unit
// serves its memory requests roughly in order, so any store or poll that hands
// the SwiGLU row from gate/up workgroups to down workgroups waits behind the
// weight loads its compute unit issued earlier; the next launch in the stream
// costs less than that wait.  Every load a kernel needs is issued as soon as
// its address is known, before any of its data is used, so that the memory
// counter waits (in order) for the small operands never include weight loads.
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
#include "router.h"

namespace bfp8 {

namespace {

constexpr int kUpThreads = 1024;    // gate/up kernel: 8 column waves + 8 hidden-row waves
constexpr int kUpWaves = kUpThreads / 64;
constexpr int kColumnWaves = 8;
constexpr int kDownThreads = 1024;  // down kernel: 16 waves
constexpr int kDownWaves = kDownThreads / 64;
constexpr int kMaxK = 16;  // routes per token; the down kernel is built for 8 and for 16
constexpr int kMaxTokens = 32;  // tokens per call on this path
constexpr int kMaxH = 8192;
constexpr int kUnitsPerWave = 4;                            // 1 KB W2 units per down wave
constexpr int kMxUnitsPerWave = 2;  // the same with MXFP4 rows (a unit holds twice the elements)
constexpr int kMaxUnits = kDownWaves * kUnitsPerWave;       // per down workgroup
constexpr int kMxMaxUnits = kDownWaves * kMxUnitsPerWave;
constexpr int kMaxDownRows = 64;
constexpr int kDownTarget = 256;  // down workgroups aimed at (one per compute unit of MI355X)
constexpr unsigned kSpinLimit = 1u << 20;  // bound of the LDS waits (about 0.03 s)
// Weight formats of the two kernels (the C ABI's weight_scale_mode values):
// E4M3 rows with fp32 scales per 128 x 128 block; E4M3 rows with one fp32
// scale per row (W8A8: the activations then take one scale per row too);
// E2M1 rows with an E8M0 scale per 32 elements (MXFP4).
constexpr int kWBlock = 0, kWChannel = 1, kWMx = 2;

}  // namespace

// Bit 0: a column wave of the gate/up kernel ran out of its bounded wait for
// the hidden row (its column's value is then unspecified).  Bit 1: a
// hidden-row wave of the W8A8 form ran out of its wait for the other
// hidden-row waves' maxima (the row's scale is then unspecified).  Set with a
// device atomic, never cleared by the kernels; read and cleared by
// read_wait_faults (bfp8moe_wait_faults in the C ABI).
__device__ unsigned int g_wait_faults = 0;

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// Workgroup barrier that waits for LDS traffic only (no vector-memory wait),
// so that waves with weight loads in flight are not held up.  The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void wg_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): vmcnt and expcnt left at their maximum
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ float amax8(const float (&f)[8]) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(f[i]));
  return m;
}

// Quantise 8 BF16-valued floats of one group (scale sc) and store the E4M3
// values dec(E4M3(x / sc)) as four FP16 pairs (every E4M3 value is exact in
// FP16, subnormals included) at dst (LDS, 16-byte aligned).  sat: the scale
// may be below amax / 448 (a static one), quotients beyond saturate.
__device__ __forceinline__ void quant_store8(const float (&f)[8], float sc, h2* dst, bool sat = false) {
  const uint2 q = sat ? encode8_scaled_sat(f, sc) : encode8_scaled(f, sc);
  const h2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)q.x, 1.0f, false);
  const h2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)q.x, 1.0f, true);
  const h2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)q.y, 1.0f, false);
  const h2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)q.y, 1.0f, true);
  dst[0] = a; dst[1] = b; dst[2] = c; dst[3] = d;
}

// Activation rows in LDS (the gate/up kernel's hidden row, the down kernel's
// SwiGLU rows): FP16 pair i (elements 2 i, 2 i + 1) is stored at act_swz(i).
// The 16-byte units (4 pairs) of each run of 16 are permuted by XOR with the
// run's index, so that reads where lane l takes the 8 or 16 pairs of its 16 or
// 32 consecutive elements spread a 16-lane pass over all banks instead of a
// half, a quarter or a sixteenth of them.
__device__ __forceinline__ int act_swz(int i) { return i ^ (((i >> 6) & 15) << 2); }

// Four FP16 pairs (one 16-byte unit) of the swizzled hidden row from pair i
// (a multiple of 4).
__device__ __forceinline__ void act_unit(const h2* row, int i, h2 (&a)[4]) {
  const uint4 v = *reinterpret_cast<const uint4*>(row + act_swz(i));
  a[0] = __builtin_bit_cast(h2, v.x);
  a[1] = __builtin_bit_cast(h2, v.y);
  a[2] = __builtin_bit_cast(h2, v.z);
  a[3] = __builtin_bit_cast(h2, v.w);
}

// sum_i dec(w_i) * a_i over 16 E4M3 weights (one 16-byte load) and 16 E4M3
// activations held as FP16 pairs in LDS: pairs i .. i + 7 of a row stored
// with act_swz (dot16_row).  Weight bytes are widened to FP16 pairs (exact),
// and each v_dot2 product of two E4M3 values is exact in FP32; only the FP32
// additions round.  Two chains.
__device__ __forceinline__ float dot16_pairs(const uint4& w, h2 a0, h2 a1, h2 a2, h2 a3, h2 a4, h2 a5, h2 a6,
                                             h2 a7) {
  float s0 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w.x, 1.0f, false), a0, 0.0f, false);
  float s1 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w.x, 1.0f, true), a1, 0.0f, false);
  s0 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w.y, 1.0f, false), a2, s0, false);
  s1 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w.y, 1.0f, true), a3, s1, false);
  s0 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w.z, 1.0f, false), a4, s0, false);
  s1 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w.z, 1.0f, true), a5, s1, false);
  s0 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w.w, 1.0f, false), a6, s0, false);
  s1 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w.w, 1.0f, true), a7, s1, false);
  return s0 + s1;
}
__device__ __forceinline__ float dot16_row(const uint4& w, const h2* row, int i) {
  h2 a[4], b[4];
  act_unit(row, i, a);
  act_unit(row, i + 4, b);
  return dot16_pairs(w, a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]);
}

// sum_i dec(w_i) * a_i over 32 E2M1 weights (one 16-byte load, two to a
// byte, the even element in the low nibble) and 32 E4M3 activations held as
// FP16 pairs in LDS: pairs i .. i + 15 of a row stored with act_swz
// (dot32_fp4_row).  Each weight byte widens to an FP16 pair (exact, unit
// scale), each v_dot2 product is exact in FP32; only the FP32 additions round.
// Two chains.
__device__ __forceinline__ void dot32_fp4_unit(uint32_t wd, const h2 (&a)[4], float& s0, float& s1) {
  s0 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, 1.0f, 0), a[0], s0, false);
  s1 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, 1.0f, 1), a[1], s1, false);
  s0 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, 1.0f, 2), a[2], s0, false);
  s1 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, 1.0f, 3), a[3], s1, false);
}
__device__ __forceinline__ float dot32_fp4_row(const uint4& w, const h2* row, int i) {
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  h2 a[4][4];
#pragma unroll
  for (int d = 0; d < 4; d++) act_unit(row, i + 4 * d, a[d]);
  float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
  for (int d = 0; d < 4; d++) dot32_fp4_unit(wd[d], a[d], s0, s1);
  return s0 + s1;
}

// An E8M0 scale byte as an fp32 value, 2^(s - 127): exact for every byte
// (2^-127 is an fp32 subnormal); 255 is NaN.
__device__ __forceinline__ float e8m0_f32(uint32_t s) {
  return s == 0u ? __builtin_bit_cast(float, 0x00400000u)
                 : (s == 255u ? __builtin_nanf("") : __builtin_bit_cast(float, s << 23));
}

// Sum (or max) over aligned groups of N lanes (N = 8, 16, 32 or 64), the
// result in every lane of the group.  Within a 16-lane row the exchanges are
// DPP moves (quad swaps, then the half-row and row mirrors); wider groups add
// cross-row shuffles.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm 1,0,3,2
  v += dpp<0x4E>(v);   // quad_perm 2,3,0,1
  v += dpp<0x141>(v);  // row_half_mirror: the other quad of the half row
  if (N >= 16) v += dpp<0x140>(v);  // row_mirror: the other half row
  if (N >= 32) v += __shfl_xor(v, 16);
  if (N >= 64) v += __shfl_xor(v, 32);
  return v;
}
template <int N>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  if (N >= 16) v = fmaxf(v, dpp<0x140>(v));
  if (N >= 32) v = fmaxf(v, __shfl_xor(v, 16));
  if (N >= 64) v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// Two BF16-valued floats of one group quantised with scale sc, returned as
// the FP16 pair of their E4M3 values (same rounding as quant_store8; sat as
// there: quotients beyond +-448 saturate).
__device__ __forceinline__ h2 quant2(float a, float b, float sc, bool sat = false) {
  const double rs = 1.0 / (double)sc;
  float qa = (float)((double)a * rs), qb = (float)((double)b * rs);
  if (sat) {
    qa = fminf(fmaxf(qa, -kE4M3Max), kE4M3Max);
    qb = fminf(fmaxf(qb, -kE4M3Max), kE4M3Max);
  }
  const int q = __builtin_amdgcn_cvt_pk_fp8_f32(qa, qb, 0, false);
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(q, 1.0f, false);
}

// ------------------------------------------------------------------ gate/up
//
// Workgroup (route j, slice q) computes columns 8 q .. 8 q + 7 of route j's
// SwiGLU row.  Waves 0-7 own one column n = 8 q + w each: the dot products of
// the quantised hidden row with gate row n and up row I + n of route j's
// expert, both block scales applied per group of 128, then SwiGLU on their
// BF16 values, stored as act[j][n].  Waves 8-15 quantise the hidden row and
// load the block-scale table into LDS and count themselves done in an LDS
// word.  The column waves wait for that word, not for a workgroup barrier: a
// barrier would also wait for every column wave to have issued its loads,
// which the compute unit's memory queue holds back for microseconds, and no
// wave could start its dot products before then.
template <int RL, int I, bool kRoute, int kW>
__global__ __launch_bounds__(kUpThreads) void token_gate_up_kernel(
    const uint16_t* __restrict__ hidden, int H, const int32_t* __restrict__ ids, int k, ExpertSel sel,
    const uint8_t* __restrict__ w13, const void* __restrict__ w13_sv, int fmt, float a_static, float limit,
    int clamp, uint16_t* __restrict__ act, RouterArgs ra) {
  constexpr int kSlices = I / 8;
  // kMx: MXFP4 rows (H / 2 bytes, E2M1) with an E8M0 scale byte per 32
  // elements; kCh: E4M3 rows with one fp32 scale per row, and the hidden row
  // quantised with one scale (its amax over H, or a_static when > 0); else
  // E4M3 rows (H bytes) with fp32 scales per 128 x 128 block
  constexpr bool kMx = kW == kWMx, kCh = kW == kWChannel;
  const float* __restrict__ w13_s = static_cast<const float*>(w13_sv);
  const uint8_t* __restrict__ w13_mx = static_cast<const uint8_t*>(w13_sv);
  const int RB = kMx ? H / 2 : H;  // bytes per weight row
  __shared__ __align__(16) h2 s_ah[kMaxH / 2];  // quantised hidden row (E4M3 values as FP16)
  __shared__ float s_as[kMaxH / 128];           // its group scales
  __shared__ float s_tab[2 * (kMaxH / 128)];    // W13 block scales: gate row block, then up row block
  __shared__ int s_ready;                       // hidden-row waves done
  __shared__ float s_wmax[kUpWaves - kColumnWaves];  // kCh: each hidden-row wave's amax
  __shared__ int s_nmax;                        // kCh: hidden-row waves whose amax is in s_wmax

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = H / 128;
  const int j = blockIdx.x / kSlices;
  const int n0 = (blockIdx.x - j * kSlices) * 8;
  if (tid == 0) {
    s_ready = 0;
    s_nmax = 0;
  }
  int id_j;
  // the router folded in: wave 0 ranks the token's logits up to this route's
  // rank and hands the expert to the other waves through LDS (no weight load
  // is in flight yet, so the barrier costs only the ranking); in the token's
  // first workgroup wave 8, a hidden-row wave, later ranks all k on its own,
  // forms the weights and writes the routing for the down kernel
  const int tok = j / k, rank = j - tok * k;
  const bool writer = kRoute && rank == 0 && n0 == 0 && wave == 8;
  // LDS for the grouped selection's keys: wave 0 and the writer (wave 8) each
  __shared__ float s_rkey[kRoute ? 2 : 1][kRoute ? 64 + kFoldedRouterMaxE : 1];
  if constexpr (kRoute) {
    __shared__ int s_route;
    if (wave == 0) {
      router::WaveRoute<kFoldedRouterMaxE / 64> r;
      r.load(ra.logits + (size_t)tok * ra.E, ra.E, ra.score_fn, ra.bias, lane, ra.n_group, ra.topk_group,
             s_rkey[0]);
      int ex = 0;
      for (int q = 0; q <= rank; q++) {
        float lv;
        ex = r.take(lane, lv);
      }
      if (lane == 0) s_route = ex;
    }
    wg_sync();
    id_j = s_route;
  } else {
    id_j = ids[j];
  }
  // the writer's work, done once its hidden-row duties are over (or at once
  // when the route is not local): off the column waves' path
  auto write_routing = [&]() {
    router::WaveRoute<kFoldedRouterMaxE / 64> r;
    r.load(ra.logits + (size_t)tok * ra.E, ra.E, ra.score_fn, ra.bias, lane, ra.n_group, ra.topk_group,
           s_rkey[kRoute ? 1 : 0]);
    int my_id = 0;
    float my_logit = 0.0f;
    for (int q = 0; q < k; q++) {
      float lv;
      const int ex = r.take(lane, lv);
      if (lane == q) {
        my_id = ex;
        my_logit = lv;
      }
    }
    const float wt = r.weight(my_logit, lane, ra.E, k, ra.score_fn, ra.renorm, ra.scale);
    if (lane < k) {
      ra.ids[(size_t)tok * k + lane] = my_id;
      ra.w[(size_t)tok * k + lane] = wt;
    }
  };
  const int e = local_of(sel, id_j);
  if (e < 0) {  // route outside the local slice: it contributes nothing
    if (writer) write_routing();
    return;
  }

  // the small operands, loaded by every wave (the column waves' copies go
  // unused) so that the loads are unconditional: hidden groups t/16 and
  // t/16 + 32 (t = tid % 512), 8 values per lane, and one W13 block-scale
  // entry per thread.  Clamped lanes repeat the last group.
  // The pointers pass through empty asm statements: loads through a
  // restrict pointer count as invariant, and the compiler would otherwise
  // sink them past the barrier into the only branch that uses them.
  const int t = tid & 511, l16 = t & 15;
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(1))) const u32x4* g_u32x4;
  typedef __attribute__((address_space(1))) const float* g_float;
  // global address space kept: generic loads would count as LDS traffic too;
  // route j belongs to token j / k
  g_u32x4 hid = (g_u32x4)(hidden + (size_t)(j / k) * H);
  g_float ws13 = (g_float)w13_s;
  asm volatile("" : "+s"(hid), "+s"(ws13));
  uint4 hv[2];
#pragma unroll
  for (int p = 0; p < 2; p++) {
    const int hg = min((t >> 4) + 32 * p, G - 1);
    const u32x4 x = hid[(size_t)hg * 16 + l16];
    hv[p] = make_uint4(x.x, x.y, x.z, x.w);
  }
  const int te = min(t, 2 * G - 1);
  const float tab =
      kW != kWBlock
          ? 0.0f
          : ws13[((size_t)e * (2 * I / 128) + (te < G ? n0 / 128 : (I + n0) / 128)) * G + (te < G ? te : te - G)];
  // every wave's small loads have left before any W13 load: the compute
  // unit returns data roughly in issue order, so they land first
  wg_sync();

  if (wave >= kColumnWaves) {
    // hidden-row waves: quantise into LDS (same arithmetic as quant_fp8, or
    // quant_fp8_rows for kCh), store the table, and count themselves done
    float f[2][8];
#pragma unroll
    for (int p = 0; p < 2; p++) unpack8(hv[p], f[p]);
    float row_sc = 0.0f;
    if constexpr (kCh) {
      // one scale for the row: the 8 waves' maxima meet in LDS (bounded wait)
      row_sc = a_static;
      if (!(a_static > 0.0f)) {
        const float m = group_max<64>(fmaxf(amax8(f[0]), amax8(f[1])));
        if (lane == 0) {
          s_wmax[wave - kColumnWaves] = m;
          __hip_atomic_fetch_add(&s_nmax, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        for (unsigned spins = 0;
             __hip_atomic_load(&s_nmax, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < kUpWaves - kColumnWaves &&
             spins < kSpinLimit;
             spins++)
          __builtin_amdgcn_s_sleep(1);
        if (__hip_atomic_load(&s_nmax, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < kUpWaves - kColumnWaves &&
            lane == 0)
          atomicOr(&g_wait_faults, 2u);  // ran out: report it
        float rm = 0.0f;
#pragma unroll
        for (int w = 0; w < kUpWaves - kColumnWaves; w++) rm = fmaxf(rm, s_wmax[w]);
        row_sc = group_scale(rm, fmt);
      }
    }
#pragma unroll
    for (int p = 0; p < 2; p++) {
      const int hg = min((t >> 4) + 32 * p, G - 1);
      const float sc = kCh ? row_sc : group_scale(max_over_16(amax8(f[p])), fmt);
      quant_store8(f[p], sc, s_ah + act_swz((hg * 128 + l16 * 8) / 2), kCh && a_static > 0.0f);
      if (l16 == 0) s_as[hg] = sc;
    }
    if constexpr (kW == kWBlock) s_tab[te] = tab;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the LDS stores are done
    if (lane == 0) __hip_atomic_fetch_add(&s_ready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (writer) write_routing();
    return;
  }

  // column waves: the gate and up rows of column n0 + wave, 2 x RL 1 KB
  // loads, all issued before any data is used (every chunk but the last lies
  // inside the row; the last is clamped)
  uint4 wg[RL], wu[RL];
  // kMx: each load's E8M0 scale byte (one 32-element block); kCh: the row's fp32 scale (bits)
  uint32_t sg[kMx ? RL : 1], su[kMx ? RL : 1];
  {
    const uint8_t* gsrc = w13 + ((size_t)e * 2 * I + n0 + wave) * RB;
    const uint8_t* usrc = gsrc + (size_t)I * RB;
    const int last = min(1024 * (RL - 1) + 16 * lane, RB - 16);
#pragma unroll
    for (int c = 0; c < RL; c++) {
      const int off = c < RL - 1 ? 1024 * c + 16 * lane : last;
      wg[c] = *reinterpret_cast<const uint4*>(gsrc + off);
      wu[c] = *reinterpret_cast<const uint4*>(usrc + off);
    }
    if constexpr (kCh) {
      sg[0] = __builtin_bit_cast(uint32_t, w13_s[(size_t)e * 2 * I + n0 + wave]);
      su[0] = __builtin_bit_cast(uint32_t, w13_s[(size_t)e * 2 * I + I + n0 + wave]);
    }
    if constexpr (kMx) {
      const uint8_t* gs = w13_mx + ((size_t)e * 2 * I + n0 + wave) * (H / 32);
      const uint8_t* us = gs + (size_t)I * (H / 32);
#pragma unroll
      for (int c = 0; c < RL; c++) {
        const int off = c < RL - 1 ? 1024 * c + 16 * lane : last;
        sg[c] = gs[off / 16];
        su[c] = us[off / 16];
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // the hidden row and the table are in LDS (bounded wait; a run-out leaves
  // the column's value unspecified but ends the kernel)
  for (unsigned spins = 0;
       __hip_atomic_load(&s_ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < kUpWaves - kColumnWaves &&
       spins < kSpinLimit;
       spins++)
    __builtin_amdgcn_s_sleep(1);
  if (__hip_atomic_load(&s_ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < kUpWaves - kColumnWaves &&
      lane == 0)
    atomicOr(&g_wait_faults, 1u);  // ran out: report it

  // gate and up dot products as the data lands
  float ag = 0.0f, au = 0.0f;
#pragma unroll
  for (int c = 0; c < RL; c++) {
    const int kob = 1024 * c + 16 * lane;    // byte offset in the row: past it only in the last chunk,
    const int kof = kMx ? 2 * kob : kob;     // whose terms are dropped; kof: first element
    const int ka = min(kof, H - (kMx ? 32 : 16));  // in range for the dropped lanes' LDS reads
    float pg, pu;
    if constexpr (kMx) {
      const float as = s_as[ka / 128];
      pg = dot32_fp4_row(wg[c], s_ah, ka / 2) * (as * e8m0_f32(sg[c]));
      pu = dot32_fp4_row(wu[c], s_ah, ka / 2) * (as * e8m0_f32(su[c]));
    } else if constexpr (kCh) {
      pg = dot16_row(wg[c], s_ah, ka / 2);  // one scale for the row: applied to the sum below
      pu = dot16_row(wu[c], s_ah, ka / 2);
    } else {
      const float as = s_as[ka / 128];
      pg = dot16_row(wg[c], s_ah, ka / 2) * (as * s_tab[ka / 128]);
      pu = dot16_row(wu[c], s_ah, ka / 2) * (as * s_tab[G + ka / 128]);
    }
    if (c == RL - 1 && kof >= H) pg = pu = 0.0f;
    ag += pg;
    au += pu;
  }
  if constexpr (kCh) {
    ag *= s_as[0] * __builtin_bit_cast(float, sg[0]);
    au *= s_as[0] * __builtin_bit_cast(float, su[0]);
  }
  ag = group_sum<64>(ag);
  au = group_sum<64>(au);

  // SwiGLU of the BF16 gate/up outputs; each wave stores its column
  const float g = bf16_to_f32(f32_to_bf16(ag)), u = bf16_to_f32(f32_to_bf16(au));
  if (lane == 0) act[(size_t)j * I + n0 + wave] = (uint16_t)f32_to_bf16(swiglu_bf16(g, u, limit, clamp != 0));
}

// ------------------------------------------------------------------ down + reduce
//
// Workgroup b: output rows d0 = DR b .. d0 + DR - 1 (DR a multiple of kRpl =
// 1024 / row bytes, at most 64).  Its W2 data is k x DL units of 1 KB (route
// j, piece c: rows d0 + kRpl c .. + kRpl - 1); unit u = wave + 16 i (i below
// 4, or 2 for MXFP4 rows, whose units hold twice the elements) is held by
// that wave, lane l reading row kRpl c + l / kLpr, bytes 16 (l % kLpr) .. + 15.
// Loads leave in the order their data is needed: the SwiGLU rows (they do not
// depend on the routing), the W2 units, the W2 block scale of each lane's
// row and group.  Route ids are read with uniform (scalar) loads by each wave
// that needs them: no barrier stands between the start and the W2 loads.
template <int I, int KMAX, int kW>
__global__ __launch_bounds__(kDownThreads) void token_down_kernel(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ ids, const float* __restrict__ topk_w, int k,
    ExpertSel sel, const uint8_t* __restrict__ w2, const void* __restrict__ w2_sv, int H, int fmt, float q_static,
    int DR, int DL, uint32_t dl_magic, uint16_t* __restrict__ out) {
  // kMx: MXFP4 rows (I / 2 bytes, E2M1) with an E8M0 scale byte per 32
  // elements; kCh: E4M3 rows with one fp32 scale per row, and each SwiGLU
  // row quantised with one scale (its amax over I, or q_static when > 0);
  // else E4M3 rows (I bytes) with fp32 scales per 128 x 128 block
  constexpr bool kMx = kW == kWMx, kCh = kW == kWChannel;
  constexpr int RBI = kMx ? I / 2 : I;  // bytes per W2 row
  constexpr int GI = I / 128, kRpl = 1024 / RBI, kLpr = RBI / 16;
  constexpr int kUpw = kMx ? kMxUnitsPerWave : kUnitsPerWave;  // W2 units per wave
  const float* __restrict__ w2_s = static_cast<const float*>(w2_sv);
  const uint8_t* __restrict__ w2_mx = static_cast<const uint8_t*>(w2_sv);
  constexpr int kActLoads = (KMAX * GI + kDownWaves - 1) / kDownWaves;  // SwiGLU groups per wave
  __shared__ __align__(16) h2 s_qh[KMAX][I / 2];  // quantised SwiGLU rows (E4M3 values as FP16), each
                                                 // swizzled as the gate/up kernel's hidden row (act_swz)
  __shared__ float s_qs[KMAX][GI];                // their group scales
  __shared__ float s_y[KMAX][kMaxDownRows];       // down outputs per route (BF16 values)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = H / 128;
  const int d0 = blockIdx.x * DR, d_end = min(H, d0 + DR);
  const int n_units = k * DL;
  const int kob = 16 * (lane % kLpr);      // the lane's byte offset in its row
  const int kof = kMx ? 2 * kob : kob;     // its first element
  // token blockIdx.y: its k routes, their SwiGLU rows, its output row
  ids += (size_t)blockIdx.y * k;
  topk_w += (size_t)blockIdx.y * k;
  act += (size_t)blockIdx.y * k * I;
  out += (size_t)blockIdx.y * H;

  // 1. the route ids (lane r: route min(r, k - 1)), then the SwiGLU groups
  //    gi = wave + 16 m (route gi / GI, group gi % GI; lane l takes columns
  //    2 l and 2 l + 1), which do not depend on the routing
  const int id_lane = ids[min(lane, k - 1)];
  const float w_lane = topk_w[min(lane, k - 1)];
  __builtin_amdgcn_sched_barrier(0);
  uint32_t av[kActLoads];
#pragma unroll
  for (int m = 0; m < kActLoads; m++) {
    const int gi = min(wave + kDownWaves * m, k * GI - 1);
    av[m] = *reinterpret_cast<const uint32_t*>(act + (size_t)(gi / GI) * I + (gi % GI) * 128 + 2 * lane);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int e_lane = local_of(sel, id_lane);

  // 2. the wave's W2 units (past the last: repeats of it, cache hits).  A
  //    unit of a masked route reads a line of the SwiGLU buffer instead (in
  //    cache) and its result is dropped.
  int eu[kUpw];
#pragma unroll
  for (int i = 0; i < kUpw; i++) {
    const int u = min(wave + kDownWaves * i, n_units - 1);
    eu[i] = __builtin_amdgcn_readlane(e_lane, (int)(((uint32_t)u * dl_magic) >> 16));
  }
  uint4 wb[kUpw];
  const uint8_t* spare = reinterpret_cast<const uint8_t*>(act) + min(16 * lane, k * I * 2 - 16);
#pragma unroll
  for (int i = 0; i < kUpw; i++) {
    const int u = min(wave + kDownWaves * i, n_units - 1);
    const int j = (int)(((uint32_t)u * dl_magic) >> 16), c = u - j * DL;
    const int row = min(d0 + c * kRpl + lane / kLpr, H - 1);
    const uint8_t* src = eu[i] >= 0 ? w2 + ((size_t)eu[i] * H + row) * RBI + kob : spare;
    wb[i] = *reinterpret_cast<const uint4*>(src);
  }
  __builtin_amdgcn_sched_barrier(0);
  float wsc[kUpw];
#pragma unroll
  for (int i = 0; i < kUpw; i++) {
    const int u = min(wave + kDownWaves * i, n_units - 1);
    const int j = (int)(((uint32_t)u * dl_magic) >> 16), c = u - j * DL;
    const int row = min(d0 + c * kRpl + lane / kLpr, H - 1);
    if constexpr (kMx)
      wsc[i] = e8m0_f32(w2_mx[((size_t)max(eu[i], 0) * H + row) * (I / 32) + kof / 32]);
    else if constexpr (kCh)
      wsc[i] = w2_s[(size_t)max(eu[i], 0) * H + row];
    else
      wsc[i] = w2_s[((size_t)max(eu[i], 0) * G + row / 128) * GI + kof / 128];
  }
  __builtin_amdgcn_sched_barrier(0);

  // 3. the live routes' SwiGLU groups quantised into LDS (same arithmetic as
  //    silu_and_mul_quant_fp8, or silu_and_mul_quant_fp8_rows for kCh, whose
  //    row scale takes the maxima of the row's groups, met in LDS) while W2
  //    is in flight
  __shared__ float s_gmax[kCh ? KMAX * GI : 1];
  if constexpr (kCh) {
#pragma unroll
    for (int m = 0; m < kActLoads; m++) {
      const int gi = wave + kDownWaves * m, jq = min(gi / GI, k - 1);
      if (gi < k * GI && __builtin_amdgcn_readlane(e_lane, jq) >= 0) {
        const float gm = group_max<64>(fmaxf(fabsf(bf16_to_f32(av[m] & 0xFFFFu)), fabsf(bf16_to_f32(av[m] >> 16))));
        if (lane == 0) s_gmax[gi] = gm;
      }
    }
    wg_sync();
  }
#pragma unroll
  for (int m = 0; m < kActLoads; m++) {
    const int gi = wave + kDownWaves * m, jq = min(gi / GI, k - 1), g = gi % GI;
    if (gi < k * GI && __builtin_amdgcn_readlane(e_lane, jq) >= 0) {
      const float a0 = bf16_to_f32(av[m] & 0xFFFFu), a1 = bf16_to_f32(av[m] >> 16);
      float sc;
      if constexpr (kCh) {
        float rm = 0.0f;
#pragma unroll
        for (int g2 = 0; g2 < GI; g2++) rm = fmaxf(rm, s_gmax[jq * GI + g2]);
        sc = q_static > 0.0f ? q_static : group_scale(rm, fmt);
      } else {
        sc = group_scale(group_max<64>(fmaxf(fabsf(a0), fabsf(a1))), fmt);
      }
      s_qh[jq][act_swz(g * 64 + lane)] = quant2(a0, a1, sc, kCh && q_static > 0.0f);
      if (lane == 0) s_qs[jq][g] = sc;
    }
  }
  wg_sync();

  // 4. down projection: each row's dot product with its route's quantised
  //    SwiGLU row, both block scales applied per group, reduced over the row's
  //    lanes; live rows go to s_y as BF16 values
  float v[kUpw];
#pragma unroll
  for (int i = 0; i < kUpw; i++) {
    const int u = min(wave + kDownWaves * i, n_units - 1);
    const int j = (int)(((uint32_t)u * dl_magic) >> 16);
    if constexpr (kMx)
      v[i] = dot32_fp4_row(wb[i], s_qh[j], kof / 2) * (s_qs[j][kof / 128] * wsc[i]);
    else
      v[i] = dot16_row(wb[i], s_qh[j], kof / 2) * (s_qs[j][kof / 128] * wsc[i]);
  }
#pragma unroll
  for (int i = 0; i < kUpw; i++) v[i] = group_sum<kLpr>(v[i]);
#pragma unroll
  for (int i = 0; i < kUpw; i++) {
    const int u = wave + kDownWaves * i;
    const int j = (int)(((uint32_t)u * dl_magic) >> 16), c = u - j * DL;
    const int rl = c * kRpl + lane / kLpr;
    if (u < n_units && eu[i] >= 0 && lane % kLpr == 0 && d0 + rl < d_end) s_y[j][rl] = bf16_to_f32(f32_to_bf16(v[i]));
  }
  wg_sync();

  // 5. weighted reduction over the live routes, j ascending, by wave 0 (rows
  //    tid < DR <= 64).  The routing comes from the wave's own lanes, read
  //    while every lane is active; every s_y read is issued before the first
  //    is used.
  float wr[KMAX];
  bool lr[KMAX];
#pragma unroll
  for (int r = 0; r < KMAX; r++) {
    lr[r] = r < k && __builtin_amdgcn_readlane(e_lane, r) >= 0;
    wr[r] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_lane), r));
  }
  if (tid < d_end - d0) {
    float y[KMAX];
#pragma unroll
    for (int r = 0; r < KMAX; r++) y[r] = s_y[r][tid];
    float a = 0.0f;
#pragma unroll
    for (int r = 0; r < KMAX; r++)
      if (lr[r]) a = __builtin_fmaf(wr[r], y[r], a);
    out[d0 + tid] = (uint16_t)f32_to_bf16(a);
  }
}

}  // namespace

// Rows per down workgroup: a multiple of the rows of one 1 KB load (1024 /
// row bytes: I, or I / 2 for MXFP4 rows) giving about 256 workgroups, with at
// most 64 units and 64 rows per workgroup.
int token_down_rows(int H, int I, int k, bool mx) {
  const int rpl = 1024 / (mx ? I / 2 : I);
  int dl = ((H + kDownTarget - 1) / kDownTarget + rpl - 1) / rpl;
  const int max_units = mx ? kMxMaxUnits : kMaxUnits;
  dl = dl < max_units / k ? dl : max_units / k;
  dl = dl < kMaxDownRows / rpl ? dl : kMaxDownRows / rpl;
  return (dl > 1 ? dl : 1) * rpl;
}

hipError_t read_wait_faults(unsigned* flags, bool clear) {
  hipError_t e = hipMemcpyFromSymbol(flags, HIP_SYMBOL(g_wait_faults), sizeof(unsigned), 0, hipMemcpyDeviceToHost);
  if (e == hipSuccess && clear) {
    const unsigned zero = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_wait_faults), &zero, sizeof zero, 0, hipMemcpyHostToDevice);
  }
  return e;
}

bool token_path_fits(int64_t M, int H, int k, int I, int wfmt) {
  if (M < 1 || M > kMaxTokens || k < 1 || k > kMaxK || H < 128 || H > kMaxH || H % 128 != 0) return false;
  if (wfmt == kWMx) return H % 256 == 0 && (I == 256 || I == 512);  // whole 32-element blocks per 16-byte load
  return (wfmt == kWBlock || wfmt == kWChannel) && (I == 128 || I == 256 || I == 512);
}

hipError_t launch_token_layer(const uint16_t* hidden, int64_t M, int H, const int32_t* ids, const float* topk_w,
                              int k, const ExpertSel& sel, const uint8_t* w13, const void* w13_s,
                              const uint8_t* w2, const void* w2_s, int I, int fmt, float limit, uint16_t* act,
                              uint16_t* out, hipStream_t stream, const LaunchHook* hook,
                              const RouterArgs* route, int wfmt, float a1_static, float a2_static) {
  if (!token_path_fits(M, H, k, I, wfmt)) return hipErrorInvalidValue;  // the caller checks token_path_fits
  if (wfmt != kWBlock && route) return hipErrorInvalidValue;  // the routed layer takes block-FP8 weights
  const bool mx = wfmt == kWMx;
  if (route && (route->E < 1 || route->E > kFoldedRouterMaxE || k > route->E)) return hipErrorInvalidValue;
  const RouterArgs ra = route ? *route : RouterArgs{};
  if (route) {
    ids = route->ids;  // written by the gate/up kernel, read by the down kernel
    topk_w = route->w;
  }
  const int clamp = __builtin_isfinite(limit) ? 1 : 0;
  const int rb = mx ? H / 2 : H, rbi = mx ? I / 2 : I;  // bytes per W13 and W2 row
  const int rl = (rb + 1023) / 1024;
  const int dr = token_down_rows(H, I, k, mx);
  const int dl = dr * rbi / 1024;
  // u / dl for u < 64 by multiply and shift (exact: the multiplier's rounding
  // error stays below one step for such u)
  const uint32_t dl_magic = (65536u + dl - 1) / dl;
  const int up_grid = (int)M * k * (I / 8);
  const int down_grid = (H + dr - 1) / dr;
  if (hook) hook->before(0, stream);
  const bool run0 = !hook || hook->run(0), run1 = !hook || hook->run(1);
#define BFP8_TOKEN_CASE(N, II)                                                                                  \
  case N:                                                                                                       \
    if (route)                                                                                                  \
      hipLaunchKernelGGL((token_gate_up_kernel<N, II, true, kWBlock>), dim3(up_grid), dim3(kUpThreads), 0,     \
                         stream, hidden, H, ids, k, sel, w13, w13_s, fmt, a1_static, limit, clamp, act, ra);    \
    else if (wfmt == kWChannel)                                                                                 \
      hipLaunchKernelGGL((token_gate_up_kernel<N, II, false, kWChannel>), dim3(up_grid), dim3(kUpThreads), 0,  \
                         stream, hidden, H, ids, k, sel, w13, w13_s, fmt, a1_static, limit, clamp, act, ra);    \
    else                                                                                                        \
      hipLaunchKernelGGL((token_gate_up_kernel<N, II, false, kWBlock>), dim3(up_grid), dim3(kUpThreads), 0,    \
                         stream, hidden, H, ids, k, sel, w13, w13_s, fmt, a1_static, limit, clamp, act, ra);    \
    break;
#define BFP8_TOKEN_MX_CASE(N, II)                                                                               \
  case N:                                                                                                       \
    hipLaunchKernelGGL((token_gate_up_kernel<N, II, false, kWMx>), dim3(up_grid), dim3(kUpThreads), 0, stream,  \
                       hidden, H, ids, k, sel, w13, w13_s, fmt, a1_static, limit, clamp, act, ra);              \
    break;
#define BFP8_TOKEN_RL(II)   \
  switch (rl) {             \
    BFP8_TOKEN_CASE(1, II)  \
    BFP8_TOKEN_CASE(2, II)  \
    BFP8_TOKEN_CASE(3, II)  \
    BFP8_TOKEN_CASE(4, II)  \
    BFP8_TOKEN_CASE(5, II)  \
    BFP8_TOKEN_CASE(6, II)  \
    BFP8_TOKEN_CASE(7, II)  \
    BFP8_TOKEN_CASE(8, II)  \
  }
#define BFP8_TOKEN_MX_RL(II) \
  switch (rl) {               \
    BFP8_TOKEN_MX_CASE(1, II) \
    BFP8_TOKEN_MX_CASE(2, II) \
    BFP8_TOKEN_MX_CASE(3, II) \
    BFP8_TOKEN_MX_CASE(4, II) \
  }
  if (!run0) {
  } else if (mx) {
    if (I == 256) {
      BFP8_TOKEN_MX_RL(256)
    } else {
      BFP8_TOKEN_MX_RL(512)
    }
  } else if (I == 128) {
    BFP8_TOKEN_RL(128)
  } else if (I == 256) {
    BFP8_TOKEN_RL(256)
  } else {
    BFP8_TOKEN_RL(512)
  }
#undef BFP8_TOKEN_MX_RL
#undef BFP8_TOKEN_RL
#undef BFP8_TOKEN_MX_CASE
#undef BFP8_TOKEN_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (hook) hook->before(1, stream);
#define BFP8_TOKEN_DOWN(II, W)                                                                                   \
  do {                                                                                                           \
    if (k <= 8)                                                                                                  \
      hipLaunchKernelGGL((token_down_kernel<II, 8, W>), dim3(down_grid, (unsigned)M), dim3(kDownThreads), 0,    \
                         stream, act, ids, topk_w, k, sel, w2, w2_s, H, fmt, a2_static, dr, dl, dl_magic, out);  \
    else                                                                                                         \
      hipLaunchKernelGGL((token_down_kernel<II, 16, W>), dim3(down_grid, (unsigned)M), dim3(kDownThreads), 0,   \
                         stream, act, ids, topk_w, k, sel, w2, w2_s, H, fmt, a2_static, dr, dl, dl_magic, out);  \
  } while (0)
#define BFP8_TOKEN_DOWN_I(W)      \
  do {                            \
    if (I == 128)                 \
      BFP8_TOKEN_DOWN(128, W);    \
    else if (I == 256)            \
      BFP8_TOKEN_DOWN(256, W);    \
    else                          \
      BFP8_TOKEN_DOWN(512, W);    \
  } while (0)
  if (!run1) {
  } else if (mx) {
    if (I == 256)
      BFP8_TOKEN_DOWN(256, kWMx);
    else
      BFP8_TOKEN_DOWN(512, kWMx);
  } else if (wfmt == kWChannel) {
    BFP8_TOKEN_DOWN_I(kWChannel);
  } else {
    BFP8_TOKEN_DOWN_I(kWBlock);
  }
#undef BFP8_TOKEN_DOWN_I
#undef BFP8_TOKEN_DOWN
  e = hipGetLastError();
  if (hook) hook->before(2, stream);
  return e;
}

}  // namespace bfp8
