// token.hip -- the whole block-FP8 MoE layer for one token (M = 1) in one
// persistent kernel on gfx950.
//
// [P1 Motivation] at M = 1, top-k 8, E = 256 at most eight experts are active
// and the layer is pure weight streaming: 44 MB of W13 + W2 at the 7168 x 256
// decode shape against 88 MFLOP.  Both projections are matrix-vector
// products, so they run on the vector ALUs from row-contiguous loads (every
// wave load instruction reads 1 KB of one weight row), not on MFMA tiles whose
// operand layout scatters each load over 16 rows.
// [P1 Modification, Active-expert block scheduling] only the active experts'
// rows are read; workgroups are laid out per active-expert slot.
// [P1 Modification, Fused SwiGLU and FP8 quantization] SwiGLU is applied in the
// gate/up epilogue; its BF16 output is group-quantised where the down
// projection consumes it.
// [P4 Pull request overview] the down projection ends with the top-k weighted
// reduction, routes in order.
//
// Grid: one 1024-thread workgroup per compute unit, all resident.  Workgroup w
// serves
//   gate/up unit w: active-expert slot w / (I/8) (experts in ascending order),
//     gate rows n0 = 8 (w % (I/8)) .. n0+7 and up rows I+n0 .. I+n0+7, one row
//     per wave;
//   down unit w: output rows DR w .. DR w + DR - 1 for all k routes, as k x DL
//     pieces of 1 KB spread four per wave.
// Every wave runs the same straight-line load sequence -- block-scale tables,
// its W13 row, its four W2 pieces -- so that the waits the compiler places
// for the W13 data never include the W2 loads issued after them (the memory
// counter is in order), and the W2 stream overlaps the gate/up work.
//
// No grid barrier: the SwiGLU outputs are written as 8-byte words holding two
// BF16 values and a 32-bit launch tag, into state kept at the start of the
// workspace.  A consumer polls the words it needs until every tag equals the
// current launch's tag, so data and completion travel in one store.  The tag
// of a launch is gen + 1, where gen is read by every workgroup at its start;
// each workgroup then records that it has read gen, and workgroup 0 advances
// gen once every workgroup has done so.  Zero-filled state is valid, tags
// never repeat within 2^32 launches, and no other use of the workspace
// touches this state.  Bounded waits: a wait that runs out sets an expiry
// word and lets the kernel finish.
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

namespace bfp8 {

namespace {

constexpr int kThreads = 1024;  // 16 waves
constexpr int kWaves = kThreads / 64;
constexpr int kMaxK = 8;
constexpr int kMaxH = 8192;
constexpr int kMaxRowLoads = kMaxH / 1024;  // 1 KB loads per W13 row
constexpr int kMaxI = 512;
constexpr int kMaxDownLoads = 8;            // 1 KB W2 loads per route per workgroup
constexpr int kW2PerWave = 8;               // (route, 1 KB piece) W2 units per down wave
constexpr int kMaxGrid = 512;               // 64 flags per down wave
constexpr int kReplicas = 8;                // copies of the polled state, read by workgroup b from copy b % 8
constexpr int kTabSlots = 2 * (kMaxH / 128) + kMaxK * 2 * (kMaxI / 128) + 1;

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// Launch state at the start of the workspace.  Words that many workgroups
// poll at once are kept in kReplicas copies so that no single memory line
// serves the whole grid.  The SwiGLU output depends only on the expert and
// the column (one token), so it is kept per active-expert slot: row s holds
// slot s's I columns as 64-bit words of two columns each.  Workgroup (slot s,
// slice q) writes its 8 columns as one 32-byte piece from one wave.  Writes
// here are whole pieces from one wave: small writes that many workgroups aim
// at one memory line are serialised by the memory system and stall the
// weight stream.  A producer's tagged piece also shows that it has read gen;
// only workgroups without a slot write a separate flag.
struct TokenState {
  uint32_t gen[kReplicas][32];               // tag of the last completed launch, one copy per 128-byte line
  uint32_t expired;                          // set when a bounded wait ran out
  uint32_t pad[31];
  uint32_t pad2[(8192 - kReplicas * 128 - 128) / 4];
  uint32_t flag[kMaxGrid][16];               // workgroups without a slot: 64 bytes of tag once they have read gen
  uint64_t act[kReplicas][kMaxK * kMaxI / 2];  // [slot][column pair]: 2 BF16 (low half) + tag (high half)
};
static_assert(sizeof(TokenState) <= kTokenStateBytes, "token state");
static_assert(offsetof(TokenState, flag) == 8192 && offsetof(TokenState, act) == 8192 + 64 * kMaxGrid, "layout");

constexpr unsigned kSpinLimit = 1u << 22;

#define ATOMIC_LD(p) __hip_atomic_load((p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
#define ATOMIC_ST(p, v) __hip_atomic_store((p), (v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)

// Workgroup-wide barrier that waits for LDS traffic only (no vector-memory
// wait), so that waves with weight loads in flight are not held up.
__device__ __forceinline__ void wg_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): vmcnt and expcnt left at their maximum
  __builtin_amdgcn_s_barrier();
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
// FP16, subnormals included) at dst (LDS, 16-byte aligned).
__device__ __forceinline__ void quant_store8(const float (&f)[8], float sc, h2* dst) {
  const uint2 q = encode8_scaled(f, sc);
  const h2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)q.x, 1.0f, false);
  const h2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)q.x, 1.0f, true);
  const h2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)q.y, 1.0f, false);
  const h2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)q.y, 1.0f, true);
  dst[0] = a; dst[1] = b; dst[2] = c; dst[3] = d;
}

// sum_i dec(w_i) * a_i over 16 E4M3 weights (one 16-byte load) and 16 E4M3
// activations held as FP16 pairs at p (LDS, 16-byte aligned).  Weight bytes
// are widened to FP16 pairs (exact), and each v_dot2 product of two E4M3
// values is exact in FP32; only the FP32 additions round.  Two chains.
__device__ __forceinline__ float dot16(const uint4& w, const h2* p) {
  const h2* q = p;
  const h2 a0 = q[0], a1 = q[1], a2 = q[2], a3 = q[3], a4 = q[4], a5 = q[5], a6 = q[6], a7 = q[7];
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
// the FP16 pair of their E4M3 values (same rounding as quant_store8).
__device__ __forceinline__ h2 quant2(float a, float b, float sc) {
  const double rs = 1.0 / (double)sc;
  const int q = __builtin_amdgcn_cvt_pk_fp8_f32((float)((double)a * rs), (float)((double)b * rs), 0, false);
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(q, 1.0f, false);
}

// Gate/up wave d (0..7), once it has published: wait until every SwiGLU
// word of its groups gi = d, d + 8, ... (route j = gi / (I/128), group g,
// read from the row of route j's slot) carries tag T -- and, in workgroup 0,
// until the flags of workgroups 64 d .. 64 d + 63 without a slot do -- then
// quantise the groups into LDS.  Lane l takes the word of columns 2l and
// 2l + 1 of a group.  All loads of a round go out together.
template <int I>
__device__ __forceinline__ void take_groups(TokenState* st, int rep, int d, int k, const int* s_e, const int* s_slot,
                                           int n_slots, uint32_t T, int fmt, h2 (*s_qh)[I / 2],
                                           float (*s_qs)[I / 128], int lane) {
  constexpr int GI = I / 128;
  constexpr int NG = GI;  // groups per wave at k = 8
  bool live[NG];
  const uint64_t* src[NG];
#pragma unroll
  for (int m = 0; m < NG; m++) {
    const int gi = d + 8 * m;
    const int j = min(gi / GI, k - 1), g = gi - (gi / GI) * GI;
    live[m] = gi < k * GI && s_e[j] >= 0;
    src[m] = &st->act[rep][s_slot[j] * (kMaxI / 2) + g * 64 + lane];
  }
  const bool chk_flags = blockIdx.x == 0 && 64 * d < (int)gridDim.x;
  const int fi = min(64 * d + lane, (int)gridDim.x - 1);
  const bool fi_has_slot = fi / (I / 8) < n_slots;  // such a workgroup's SwiGLU piece is checked instead
  uint64_t w[NG];
  unsigned spins = 0;
#pragma nounroll
  for (;;) {
#pragma unroll
    for (int m = 0; m < NG; m++) w[m] = ATOMIC_LD(src[m]);
    const uint32_t f = ATOMIC_LD(&st->flag[fi][0]);
    bool ok = !chk_flags || fi_has_slot || f == T;
#pragma unroll
    for (int m = 0; m < NG; m++) ok = ok && (!live[m] || (uint32_t)(w[m] >> 32) == T);
    if (__all(ok)) break;
    if (++spins == kSpinLimit) {
      ATOMIC_ST(&st->expired, 1u);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
#pragma unroll
  for (int m = 0; m < NG; m++) {
    if (!live[m]) continue;
    const int gi = d + 8 * m, j = gi / GI, g = gi - j * GI;
    const float a0 = bf16_to_f32((uint32_t)w[m] & 0xFFFFu), a1 = bf16_to_f32(((uint32_t)w[m] >> 16) & 0xFFFFu);
    const float sc = group_scale(group_max<64>(fmaxf(fabsf(a0), fabsf(a1))), fmt);
    s_qh[j][g * 64 + lane] = quant2(a0, a1, sc);
    if (lane == 0) s_qs[j][g] = sc;
  }
}

typedef __attribute__((address_space(1))) const void* global_ptr;
typedef __attribute__((address_space(3))) void* lds_ptr;

// W2 units u = d + 8 i (down wave d = wave - 8) of the workgroup's down
// rows, copied by direct-to-LDS loads into s_w2[u] (1 KB each): route u / DL,
// 1 KB piece u % DL, i.e. kRpl rows of I bytes; lane l's 16 bytes land at
// byte 16 l of the unit.  Units past the last repeat it (a cache hit);
// masked routes read expert 0.  Completion is counted by the wave's memory
// counter.
template <int I>
__device__ __forceinline__ void issue_w2(uint8_t* s_w2, int wave, int k, int DL, uint32_t dl_magic, const int* s_e,
                                         const uint8_t* __restrict__ w2, int H, int d0, int lane) {
  constexpr int kRpl = 1024 / I, kLpr = I / 16;
  const uint8_t* src[kW2PerWave];
#pragma unroll
  for (int i = 0; i < kW2PerWave; i++) {
    const int u = min((wave - 8) + 8 * i, k * DL - 1);
    const int j = (int)(((uint32_t)u * dl_magic) >> 16), c = u - j * DL;
    const int ej = max(s_e[j], 0);
    const int row = min(d0 + c * kRpl + lane / kLpr, H - 1);
    src[i] = w2 + ((size_t)ej * H + row) * I + 16 * (lane % kLpr);
  }
#pragma unroll
  for (int i = 0; i < kW2PerWave; i++)
    __builtin_amdgcn_global_load_lds((global_ptr)src[i], (lds_ptr)(s_w2 + ((wave - 8) + 8 * i) * 1024), 16, 0, 0);
}

// Down projection of wave w's W2 units u = w + 16 i (read from LDS): each
// row's dot product with the quantised SwiGLU row of its route, both block
// scales applied per group, reduced over the row's lanes; live rows go to
// s_y as BF16-valued floats.
template <int I>
__device__ __forceinline__ void down_units(const uint8_t* s_w2, int wave, int k, int DL, uint32_t dl_magic,
                                           const int* s_e, const float* s_tab, const h2 (*s_qh)[I / 2],
                                           const float (*s_qs)[I / 128], float (*s_y)[64], int G, int H, int d0,
                                           int d_end, int rb0, int lane) {
  constexpr int GI = I / 128, kRpl = 1024 / I, kLpr = I / 16;
  constexpr int kUnits = 8 * kW2PerWave / kWaves;
  const int kof = 16 * (lane % kLpr);
  float v[kUnits];
#pragma unroll
  for (int i = 0; i < kUnits; i++) {
    const int u = min(wave + kWaves * i, k * DL - 1);
    const int j = (int)(((uint32_t)u * dl_magic) >> 16), c = u - j * DL;
    const int row = min(d0 + c * kRpl + lane / kLpr, H - 1);
    const float w2sc = s_tab[2 * G + (j * 2 + (row / 128 == rb0 ? 0 : 1)) * GI + kof / 128];
    const uint4 wv = *reinterpret_cast<const uint4*>(s_w2 + u * 1024 + 16 * lane);
    v[i] = dot16(wv, &s_qh[j][kof / 2]) * (s_qs[j][kof / 128] * w2sc);
  }
#pragma unroll
  for (int i = 0; i < kUnits; i++) v[i] = group_sum<kLpr>(v[i]);
#pragma unroll
  for (int i = 0; i < kUnits; i++) {
    const int u = wave + kWaves * i;
    const int j = (int)(((uint32_t)u * dl_magic) >> 16), c = u - j * DL;
    const int rl = c * kRpl + lane / kLpr;
    if (u < k * DL && lane % kLpr == 0 && d0 + rl < d_end && s_e[j] >= 0) s_y[j][rl] = bf16_to_f32(f32_to_bf16(v[i]));
  }
}

template <int RL, int I>
__global__ __launch_bounds__(kThreads) void token_layer_kernel(
    const uint16_t* __restrict__ hidden, int H, const int32_t* __restrict__ ids, const float* __restrict__ topk_w,
    int k, int32_t offset, int32_t L, const uint8_t* __restrict__ w13, const float* __restrict__ w13_s,
    const uint8_t* __restrict__ w2, const float* __restrict__ w2_s, int fmt, float limit, int clamp,
    int down_rows, int DL, uint32_t dl_magic, uint32_t tab_magic, TokenState* st, uint16_t* __restrict__ out) {
  constexpr int GI = I / 128;
  constexpr int kSlices = I / 8;     // gate/up units per expert
  __shared__ __align__(16) int s_e[kMaxK];
  __shared__ int s_slot[kMaxK];                    // active-expert slot of each route
  __shared__ float s_w[kMaxK];
  __shared__ uint32_t s_tag;
  __shared__ uint32_t s_pub[8];                    // this workgroup's 8 SwiGLU columns (BF16)
  __shared__ int s_pub_count;
  __shared__ int s_expert, s_nslots;
  __shared__ __align__(16) h2 s_ah[kMaxH / 2];     // quantised hidden row (E4M3 values as FP16)
  __shared__ float s_as[kMaxH / 128];              // its group scales
  __shared__ __align__(16) h2 s_qh[kMaxK][I / 2];  // quantised SwiGLU rows (E4M3 values as FP16)
  __shared__ float s_qs[kMaxK][GI];
  __shared__ float s_y[kMaxK][64];
  __shared__ float s_tab[kTabSlots];               // block-scale tables (+ a spare slot)
  __shared__ __align__(16) uint8_t s_w2[8 * kW2PerWave * 1024];  // the workgroup's W2 units

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = H / 128;
  const int slot = blockIdx.x / kSlices;
  const int n0 = (blockIdx.x - slot * kSlices) * 8;
  const int d0 = blockIdx.x * down_rows;  // >= H: no down unit
  const int d_end = min(H, d0 + down_rows);
  const int l16 = tid & 15;
  const int rep = blockIdx.x % kReplicas;

  // 0. the hidden row (group tid/16, 8 values per lane), the routing through
  //    scalar loads (one request per wave, not one per lane) and, in wave 0,
  //    gen.  The hidden load is unconditional (clamped index): a vector load
  //    in a branch makes the compiler wait for it where the branch joins.
  const int hg = min(tid >> 4, G - 1);
  const uint4 hv = *reinterpret_cast<const uint4*>(hidden + (size_t)hg * 128 + l16 * 8);
  int32_t id_raw[kMaxK];
  float w_raw[kMaxK];
#pragma unroll
  for (int r = 0; r < kMaxK; r++) {
    id_raw[r] = r < k ? ids[r] : -1;
    w_raw[r] = r < k ? topk_w[r] : 0.0f;
  }
  uint32_t gen = 0;
  if (wave == 0) gen = ATOMIC_LD(&st->gen[rep][0]);

  // 1. quantise the hidden row into LDS while the routing settles
  if ((tid >> 4) < G) {
    float f[8];
    unpack8(hv, f);
    const float sc = group_scale(max_over_16(amax8(f)), fmt);
    quant_store8(f, sc, s_ah + (hg * 128 + l16 * 8) / 2);
    if (l16 == 0) s_as[hg] = sc;
  }
  if (tid < kMaxK) {
    int32_t id = id_raw[0];
    float wt = w_raw[0];
#pragma unroll
    for (int r = 1; r < kMaxK; r++)
      if (tid == r) {
        id = id_raw[r];
        wt = w_raw[r];
      }
    const int64_t e = (int64_t)id - offset;
    s_e[tid] = (tid < k && e >= 0 && e < L) ? (int)e : -1;
    s_w[tid] = wt;
  }
  if (tid == 0) {
    s_tag = gen + 1;
    s_pub_count = 0;
    s_expert = -1;
  }
  wg_sync();

  // 2. this workgroup's active-expert slot: the distinct live experts in
  //    ascending order.  Lane r < k of wave 0 works out route r's rank
  //    (vector code: the scalar unit is shared by all waves of the CU).
  if (wave == 0) {
    int ev[kMaxK];
    {
      const int4 a = *reinterpret_cast<const int4*>(s_e), b = *reinterpret_cast<const int4*>(s_e + 4);
      ev[0] = a.x; ev[1] = a.y; ev[2] = a.z; ev[3] = a.w; ev[4] = b.x; ev[5] = b.y; ev[6] = b.z; ev[7] = b.w;
    }
    const int r = min(lane, kMaxK - 1);
    int er = ev[0];
#pragma unroll
    for (int q = 1; q < kMaxK; q++) er = r == q ? ev[q] : er;
    bool first = lane < kMaxK && er >= 0;
    int rank = 0;
#pragma unroll
    for (int q = 0; q < kMaxK; q++) {
      bool q_first = ev[q] >= 0;
#pragma unroll
      for (int p2 = 0; p2 < q; p2++) q_first = q_first && ev[p2] != ev[q];
      first = first && !(q < r && ev[q] == er);
      rank += (q_first && ev[q] < er) ? 1 : 0;
    }
    const uint64_t firsts = __ballot(first);
    if (lane < kMaxK) s_slot[lane] = rank;  // a route's expert has this rank among the distinct live experts
    if (first && rank == slot) s_expert = er;
    if (lane == 0) s_nslots = __popcll(firsts);
  }
  wg_sync();
  const int e = __builtin_amdgcn_readfirstlane(s_expert);  // -1: no gate/up unit
  const int n_slots = __builtin_amdgcn_readfirstlane(s_nslots);
  const uint32_t T = s_tag;

  const int e_ld = e >= 0 ? e : 0;  // a workgroup without a slot loads expert 0 and discards it
  const int rb0 = min(d0, H - 1) / 128, rb1 = min(max(d_end - 1, d0), H - 1) / 128;

  if (wave >= 8) {
    // 3. down waves: block-scale tables into LDS, one load per thread: W13
    //    scales of the gate and up row blocks (entries 0 .. 2G-1), then the
    //    W2 scales of this unit's (at most two) row blocks for every route
    {
      const int n_tab = 2 * G + k * 2 * GI;
      const int blk_gate = n0 / 128, blk_up = (I + n0) / 128;
      const int t0 = tid - 512;
      const int t = t0 - n_tab * (int)(((uint32_t)t0 * tab_magic) >> 20);  // t0 mod n_tab
      const float* src;
      if (t < 2 * G) {
        src = w13_s + ((size_t)e_ld * (2 * I / 128) + (t < G ? blk_gate : blk_up)) * G + (t < G ? t : t - G);
      } else {
        const int q = t - 2 * G;
        const int j = q / (2 * GI), which = (q / GI) & 1, g2 = q % GI;
        const int ej = s_e[j] >= 0 ? s_e[j] : 0;
        src = w2_s + ((size_t)ej * G + (which ? rb1 : rb0)) * GI + g2;
      }
      s_tab[t0 < n_tab ? t0 : kTabSlots - 1] = *src;  // past the tables: the spare slot
    }
    wg_sync();
    if (d0 >= H) return;
    // 4. their W2 units into LDS, queued behind the W13 loads of the
    //    gate/up waves
    issue_w2<I>(s_w2, wave, k, DL, dl_magic, s_e, w2, H, d0, lane);
    __builtin_amdgcn_s_waitcnt(0);  // the W2 units are in LDS
  } else {
    // 4. gate/up wave w: column n = n0 + w, i.e. gate row n and up row I + n
    //    of expert e, requested as soon as the slot is known
    uint4 wg[RL], wu[RL];
    {
      // every chunk but the last lies inside the row; the last is clamped
      const uint8_t* gsrc = w13 + ((size_t)e_ld * 2 * I + n0 + wave) * H;
      const uint8_t* usrc = gsrc + (size_t)I * H;
      const int last = min(1024 * (RL - 1) + 16 * lane, H - 16);
#pragma unroll
      for (int c = 0; c < RL; c++) {
        const int off = c < RL - 1 ? 1024 * c + 16 * lane : last;
        wg[c] = *reinterpret_cast<const uint4*>(gsrc + off);
        wu[c] = *reinterpret_cast<const uint4*>(usrc + off);
      }
    }
    wg_sync();  // the tables are in LDS

    // 5. gate and up dot products as the data lands, then SwiGLU on their
    //    BF16 values
    float ag = 0.0f, au = 0.0f;
#pragma unroll
    for (int c = 0; c < RL; c++) {
      const int kof = 1024 * c + 16 * lane;  // past H only in the last chunk: its terms are dropped
      const float as = s_as[kof / 128];
      float pg = dot16(wg[c], s_ah + kof / 2) * (as * s_tab[kof / 128]);
      float pu = dot16(wu[c], s_ah + kof / 2) * (as * s_tab[G + kof / 128]);
      if (c == RL - 1 && kof >= H) pg = pu = 0.0f;
      ag += pg;
      au += pu;
    }
    ag = group_sum<64>(ag);
    au = group_sum<64>(au);
    if (e >= 0) {
      // the last of the 8 gate/up waves to finish writes the workgroup's
      // 8 columns, tagged, to every copy
      const float g = bf16_to_f32(f32_to_bf16(ag)), u = bf16_to_f32(f32_to_bf16(au));
      const uint32_t h = f32_to_bf16(swiglu_bf16(g, u, limit, clamp != 0));
      int done = 0;
      if (lane == 0) {
        s_pub[wave] = h;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        done = atomicAdd(&s_pub_count, 1);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      }
      done = __builtin_amdgcn_readfirstlane(done);
      if (done == kWaves / 2 - 1 && lane < 4) {
        const uint64_t word = (uint64_t)(s_pub[2 * lane] | (s_pub[2 * lane + 1] << 16)) | ((uint64_t)T << 32);
#pragma unroll
        for (int x = 0; x < kReplicas; x++) ATOMIC_ST(&st->act[x][slot * (kMaxI / 2) + n0 / 2 + lane], word);
      }
    }
    if (e < 0 && wave == 0 && lane < 16) ATOMIC_ST(&st->flag[blockIdx.x][lane], T);
    if (d0 >= H) return;  // the whole workgroup leaves: no down unit
    // 6. SwiGLU rows into LDS, quantised
    take_groups<I>(st, rep, wave, k, s_e, s_slot, n_slots, T, fmt, s_qh, s_qs, lane);
  }
  wg_sync();  // the quantised SwiGLU rows are in LDS

  // 7. down projection, shared by all 16 waves, then the route rows in s_y
  down_units<I>(s_w2, wave, k, DL, dl_magic, s_e, s_tab, s_qh, s_qs, s_y, G, H, d0, d_end, rb0, lane);
  wg_sync();
  if (blockIdx.x == 0 && tid < kReplicas) ATOMIC_ST(&st->gen[tid][0], T);  // every workgroup has read gen

  // 8. weighted reduction over the routes, j ascending
  if (tid < d_end - d0) {
    float a = 0.0f;
    for (int j = 0; j < k; j++)
      if (s_e[j] >= 0) a = __builtin_fmaf(s_w[j], s_y[j][tid], a);
    out[d0 + tid] = (uint16_t)f32_to_bf16(a);
  }
}

// rows of the down unit: the smallest multiple of the rows per 1 KB load that
// covers H with at most `units` workgroups
int token_down_rows(int H, int I, int units) {
  const int rpl = 1024 / I;
  int dr = (H + units - 1) / units;
  dr = (dr + rpl - 1) / rpl * rpl;
  return dr;
}

}  // namespace

int token_kernel_grid(int H, int k, int32_t L, int I) {
  const int slots = k < L ? k : L;
  const int up = slots * (I / 8);
  const int dr = token_down_rows(H, I, up);
  const int down = (H + dr - 1) / dr;
  return up > down ? up : down;
}

bool token_path_fits(int64_t M, int H, int k, int32_t L, int I, int num_cus) {
  if (M != 1 || k < 1 || k > kMaxK || H > kMaxH || H % 128 != 0) return false;
  if (!(I == 128 || I == 256 || I == 512)) return false;
  const int slots = k < L ? k : L;
  const int up = slots * (I / 8);
  const int dr = token_down_rows(H, I, up);
  if (dr > 64 || dr * I / 1024 > kMaxDownLoads) return false;
  if (k * (dr * I / 1024) > 8 * kW2PerWave) return false;  // W2 units of the 8 down waves
  const int grid = token_kernel_grid(H, k, L, I);
  return grid <= num_cus && grid <= kMaxGrid;
}

hipError_t launch_token_layer(const uint16_t* hidden, int H, const int32_t* ids, const float* topk_w, int k,
                              int32_t offset, int32_t L, const uint8_t* w13, const float* w13_s, const uint8_t* w2,
                              const float* w2_s, int I, int fmt, float limit, void* state, uint16_t* out,
                              hipStream_t stream, const LaunchHook* hook) {
  const int clamp = __builtin_isfinite(limit) ? 1 : 0;
  const int slots = k < L ? k : L;
  const int dr = token_down_rows(H, I, slots * (I / 8));
  const int grid = token_kernel_grid(H, k, L, I);
  const int rl = (H + 1023) / 1024, dl = dr * I / 1024;
  if (!(I == 128 || I == 256 || I == 512) || rl < 1 || rl > kMaxRowLoads || dl < 1 || dl > kMaxDownLoads || k * dl > 8 * kW2PerWave)
    return hipErrorInvalidValue;  // token_path_fits rules these out
  // exact quotients by multiply and shift: u / dl for u < 64 and t / n_tab for
  // t < 1024 (the rounding error of the multiplier stays below one step)
  const uint32_t dl_magic = (65536u + dl - 1) / dl;
  const uint32_t n_tab = 2 * (H / 128) + k * 2 * (I / 128);
  const uint32_t tab_magic = ((1u << 20) + n_tab - 1) / n_tab;
  if (hook) hook->before(0, stream);
#define BFP8_TOKEN_CASE(N, II)                                                                               \
  case N:                                                                                                    \
    hipLaunchKernelGGL((token_layer_kernel<N, II>), dim3(grid), dim3(kThreads), 0, stream, hidden, H, ids,   \
                       topk_w, k, offset, L, w13, w13_s, w2, w2_s, fmt, limit, clamp, dr, dl, dl_magic,     \
                       tab_magic, static_cast<TokenState*>(state), out);                                     \
    break;
#define BFP8_TOKEN_RL(II)                                                                                    \
  switch (rl) {                                                                                              \
    BFP8_TOKEN_CASE(1, II)                                                                                   \
    BFP8_TOKEN_CASE(2, II)                                                                                   \
    BFP8_TOKEN_CASE(3, II)                                                                                   \
    BFP8_TOKEN_CASE(4, II)                                                                                   \
    BFP8_TOKEN_CASE(5, II)                                                                                   \
    BFP8_TOKEN_CASE(6, II)                                                                                   \
    BFP8_TOKEN_CASE(7, II)                                                                                   \
    BFP8_TOKEN_CASE(8, II)                                                                                   \
  }
  if (I == 128) {
    BFP8_TOKEN_RL(128)
  } else if (I == 256) {
    BFP8_TOKEN_RL(256)
  } else {
    BFP8_TOKEN_RL(512)
  }
#undef BFP8_TOKEN_RL
#undef BFP8_TOKEN_CASE
  hipError_t e = hipGetLastError();
  if (hook) hook->before(1, stream);
  return e;
}

}  // namespace bfp8
