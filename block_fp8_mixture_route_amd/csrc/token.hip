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
// Grid: one 1024-thread workgroup per compute unit, all resident.  Small
// straight-line code per wave matters: a dispatch starts with a cold
// instruction cache, so each wave handles one weight row (and up to four 1 KB
// pieces of W2) instead of many unrolled rows.  Workgroup w serves
//   gate/up unit w: active-expert slot w / (I/8) (experts in ascending order),
//     gate rows n0 = 8 (w % (I/8)) .. n0+7 and up rows I+n0 .. I+n0+7;
//   down unit w: output rows DR w .. DR w + DR - 1 for all k routes.
// Timeline per workgroup:
//   ids -> slot's expert -> W13 loads (one row per wave) -> hidden row
//   quantised into LDS -> W2 loads (k x DL units of 1 KB, four per wave over
//   waves 1..15) -> gate/up dot products (need W13 only) -> SwiGLU, act rows
//   to global memory (wave 0, which holds no W2 loads and so waits only for
//   its own stores) -> grid barrier -> act rows of the k routes quantised into
//   LDS (waves 0..7) -> down dot products as the W2 data lands (waves 1..15)
//   -> weighted reduction -> out.
// The barrier and the act exchange overlap the tail of the W2 stream.  Every
// load is issued unconditionally (clamped addresses, counts fixed at compile
// time) and the W2 loads share one straight-line branch with the gate/up work
// of their waves, so that the compiler's waits for W13 data never include the
// W2 loads issued after it.
#include "device.h"
#include "internal.h"

namespace bfp8 {

namespace {

constexpr int kThreads = 1024;  // 16 waves: one W13 row each; waves 8..15 also one route's W2 rows
constexpr int kWaves = kThreads / 64;
constexpr int kMaxK = 8;
constexpr int kMaxH = 8192;
constexpr int kMaxRowLoads = kMaxH / 1024;  // 1 KB loads per W13 row
constexpr int kMaxI = 512;
constexpr int kMaxDownLoads = 8;            // 1 KB W2 loads per route per workgroup
constexpr int kDownUnitsPerWave = 4;        // (route, 1 KB chunk) W2 units per wave 1..15
constexpr int kMaxGrid = 1024;

typedef float v2f __attribute__((ext_vector_type(2)));

// Grid barrier state, at the start of the workspace.  Generation-numbered
// flags: each workgroup publishes gen+1 in its own slot, workgroup 0 waits
// for all of them and then publishes gen+1 itself; everything stays
// consistent across launches without a reset.  Zero-filled memory is a valid
// initial state.
struct TokenBarrier {
  uint32_t gen;
  uint32_t expired;
  uint32_t pad[30];
  uint32_t flag[kMaxGrid];
};
static_assert(sizeof(TokenBarrier) <= 8192, "barrier header");

constexpr unsigned kSpinLimit = 1u << 22;

#define ATOMIC_LD(p) __hip_atomic_load((p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
#define ATOMIC_ST(p, v) __hip_atomic_store((p), (v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)

// Workgroup-wide barrier that waits for LDS traffic only (no vector-memory
// wait), so that waves with weight loads in flight are not held up.
__device__ __forceinline__ void wg_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): vmcnt and expcnt left at their maximum
  __builtin_amdgcn_s_barrier();
}

// Grid barrier.  Before it, every act store of this workgroup must have been
// acknowledged: the act writer (wave 0) waits for its vector memory counter,
// the other waves hold only loads and do not wait.
__device__ void grid_barrier(TokenBarrier* b, unsigned nwg, int wave) {
  __shared__ uint32_t s_gen;
  if (wave == 0) __builtin_amdgcn_s_waitcnt(0);
  wg_sync();
  if (threadIdx.x == 0) {
    const uint32_t g = ATOMIC_LD(&b->gen);
    __builtin_amdgcn_s_waitcnt(0);
    ATOMIC_ST(&b->flag[blockIdx.x], g + 1);
    s_gen = g;
  }
  wg_sync();
  const uint32_t g = s_gen;
  if (blockIdx.x == 0) {
    for (unsigned i = threadIdx.x; i < nwg; i += kThreads) {
      unsigned spins = 0;
      while (ATOMIC_LD(&b->flag[i]) != g + 1) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins == kSpinLimit) {
          ATOMIC_ST(&b->expired, 1u);
          break;
        }
      }
    }
    wg_sync();
    if (threadIdx.x == 0) {
      __builtin_amdgcn_s_waitcnt(0);
      ATOMIC_ST(&b->gen, g + 1);
    }
  } else if (threadIdx.x == 0) {
    unsigned spins = 0;
    while (ATOMIC_LD(&b->gen) == g) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins == kSpinLimit) {
        ATOMIC_ST(&b->expired, 1u);
        break;
      }
    }
  }
  wg_sync();
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

// Quantise 8 BF16-valued floats of one group (scale sc) and return the
// decoded E4M3 values, i.e. dec(E4M3(x / sc)), as fp32.
__device__ __forceinline__ void quant_dequant8(const float (&f)[8], float sc, float (&d)[8]) {
  const uint2 q = encode8_scaled(f, sc);
  const v2f a = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.x, false), b = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.x, true);
  const v2f c = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.y, false), e = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.y, true);
  d[0] = a.x; d[1] = a.y; d[2] = b.x; d[3] = b.y; d[4] = c.x; d[5] = c.y; d[6] = e.x; d[7] = e.y;
}

// sum_i dec(w_i) * a_i over 16 E4M3 weights (one 16-byte load) and 16 fp32
// activations at p (LDS, 16-byte aligned); two interleaved fp32 chains.
__device__ __forceinline__ float dot16(const uint4& w, const float* p) {
  const float4 a0 = *reinterpret_cast<const float4*>(p);
  const float4 a1 = *reinterpret_cast<const float4*>(p + 4);
  const float4 a2 = *reinterpret_cast<const float4*>(p + 8);
  const float4 a3 = *reinterpret_cast<const float4*>(p + 12);
  const v2f w0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false), w1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
  const v2f w2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false), w3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
  const v2f w4 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.z, false), w5 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.z, true);
  const v2f w6 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.w, false), w7 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.w, true);
  float s0 = w0.x * a0.x, s1 = w0.y * a0.y;
  s0 = __builtin_fmaf(w1.x, a0.z, s0); s1 = __builtin_fmaf(w1.y, a0.w, s1);
  s0 = __builtin_fmaf(w2.x, a1.x, s0); s1 = __builtin_fmaf(w2.y, a1.y, s1);
  s0 = __builtin_fmaf(w3.x, a1.z, s0); s1 = __builtin_fmaf(w3.y, a1.w, s1);
  s0 = __builtin_fmaf(w4.x, a2.x, s0); s1 = __builtin_fmaf(w4.y, a2.y, s1);
  s0 = __builtin_fmaf(w5.x, a2.z, s0); s1 = __builtin_fmaf(w5.y, a2.w, s1);
  s0 = __builtin_fmaf(w6.x, a3.x, s0); s1 = __builtin_fmaf(w6.y, a3.y, s1);
  s0 = __builtin_fmaf(w7.x, a3.z, s0); s1 = __builtin_fmaf(w7.y, a3.w, s1);
  return s0 + s1;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// Gate/up dot product of one wave's row from its RL loads (lane-partial).
template <int RL>
__device__ __forceinline__ float gate_up_row(const uint4 (&wa)[RL], const float* s_af, const float* s_as,
                                             const float* wsc, int H, int lane) {
  float acc = 0.0f;
#pragma unroll
  for (int c = 0; c < RL; c++) {
    const int kof = 1024 * c + 16 * lane;
    const int kc = min(kof, H - 16);
    const float sc = kof < H ? s_as[kc / 128] * wsc[kc / 128] : 0.0f;
    acc = __builtin_fmaf(dot16(wa[c], s_af + kc), sc, acc);
  }
  return acc;
}

template <int RL, int DL>
__global__ __launch_bounds__(kThreads) void token_layer_kernel(
    const uint16_t* __restrict__ hidden, int H, const int32_t* __restrict__ ids, const float* __restrict__ topk_w,
    int k, int32_t offset, int32_t L, const uint8_t* __restrict__ w13, const float* __restrict__ w13_s,
    const uint8_t* __restrict__ w2, const float* __restrict__ w2_s, int I, int fmt, float limit, int clamp,
    int down_rows, uint16_t* __restrict__ act, TokenBarrier* bar, uint16_t* __restrict__ out) {
  __shared__ int s_e[kMaxK];
  __shared__ float s_w[kMaxK];
  __shared__ int s_expert;
  __shared__ uint32_t s_route_mask;
  __shared__ __align__(16) float s_af[kMaxH];       // dequantised hidden row
  __shared__ float s_as[kMaxH / 128];               // its group scales
  __shared__ float s_rows[16];                      // gate/up row totals
  __shared__ __align__(16) float s_qf[kMaxK][kMaxI];  // dequantised act rows
  __shared__ float s_qs[kMaxK][kMaxI / 128];
  __shared__ float s_y[kMaxK][64];
  __shared__ float s_tab[2 * (kMaxH / 128) + kMaxK * 2 * (kMaxI / 128)];  // block-scale tables

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = H / 128, GI = I / 128;
  const int slices = I / 8;
  const int slot = blockIdx.x / slices;
  const int n0 = (blockIdx.x - slot * slices) * 8;
  const int rpl = 1024 / I;                       // W2 rows per 1 KB load
  const int lpr = I / 16;                         // lanes per W2 row
  const int d0 = blockIdx.x * down_rows;
  const int d_end = min(H, d0 + down_rows);
  const int l16 = tid & 15;

  // 0. routing and the hidden row (group tid/16, 8 values per lane): issued first
  int e_mine = -1;
  if (tid < k) {
    const int64_t e = (int64_t)ids[tid] - offset;
    e_mine = (e >= 0 && e < L) ? (int)e : -1;
    s_w[tid] = topk_w[tid];
    s_e[tid] = e_mine;
  }
  const int hg = min(tid >> 4, G - 1);
  const uint4 hv = *reinterpret_cast<const uint4*>(hidden + (size_t)hg * 128 + l16 * 8);

  // 1. this workgroup's active-expert slot (distinct live experts, ascending)
  if (tid == 0) { s_expert = -1; s_route_mask = 0; }
  wg_sync();
  if (tid < k && e_mine >= 0) {
    bool first = true;
    int rank = 0;
    for (int r = 0; r < k; r++) {
      const int o = s_e[r];
      if (r < tid && o == e_mine) first = false;
      bool o_first = o >= 0;
      for (int q = 0; q < r; q++) o_first = o_first && (s_e[q] != o);
      rank += (o_first && o < e_mine) ? 1 : 0;
    }
    if (first && rank == slot) s_expert = e_mine;
  }
  wg_sync();
  const int e = __builtin_amdgcn_readfirstlane(s_expert);  // -1: no gate/up unit
  if (tid < k && e >= 0 && e_mine == e) atomicOr(&s_route_mask, 1u << tid);

  // 2. scale tables: W13 block scales of the gate and up row blocks (threads
  //    0..2G-1), W2 block scales of this unit's (at most two) row blocks for
  //    every route (threads 512..).  One unconditional load per thread.
  const int e_ld = e >= 0 ? e : 0;  // a workgroup without a slot loads expert 0 and discards it
  const int blk_gate = n0 / 128, blk_up = (I + n0) / 128;
  const int rb0 = min(d0, H - 1) / 128, rb1 = min(max(d_end - 1, d0), H - 1) / 128;
  float tab;
  int tab_slot;
  {
    const bool is13 = tid < 512;
    const int t13 = min(tid, 2 * G - 1);
    const int b13 = t13 < G ? blk_gate : blk_up, g13 = t13 < G ? t13 : t13 - G;
    const int q = min(max(tid - 512, 0), 2 * kMaxK * GI - 1);
    const int j2 = min(q / (2 * GI), k - 1), which = (q / GI) & 1, g2 = q % GI;
    const int e2 = s_e[j2] >= 0 ? s_e[j2] : 0;
    const float* src = is13 ? w13_s + ((size_t)e_ld * (2 * I / 128) + b13) * G + g13
                            : w2_s + ((size_t)e2 * G + (which ? rb1 : rb0)) * GI + g2;
    tab = *src;
    tab_slot = is13 ? (tid < 2 * G ? tid : -1) : (q == tid - 512 ? 2 * G + q : -1);
  }

  // 3. W13: this wave's row (gate row n0 + w for w < 8, up row I + n0 + w - 8)
  uint4 wa[RL];
  {
    const int row = wave < 8 ? n0 + wave : I + n0 + (wave - 8);
    const uint8_t* src = w13 + ((size_t)e_ld * 2 * I + row) * H;
#pragma unroll
    for (int c = 0; c < RL; c++) wa[c] = *reinterpret_cast<const uint4*>(src + min(1024 * c + 16 * lane, H - 16));
  }
  __builtin_amdgcn_sched_barrier(0);

  // 4. quantise the hidden row, dequantised into LDS; the tables land in LDS
  if ((tid >> 4) < G) {
    float f[8], d[8];
    unpack8(hv, f);
    const float sc = group_scale(max_over_16(amax8(f)), fmt);
    quant_dequant8(f, sc, d);
    float* dst = s_af + hg * 128 + l16 * 8;
    *reinterpret_cast<float4*>(dst) = make_float4(d[0], d[1], d[2], d[3]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(d[4], d[5], d[6], d[7]);
    if (l16 == 0) s_as[hg] = sc;
  }
  if (tab_slot >= 0) s_tab[tab_slot] = tab;
  wg_sync();
  __builtin_amdgcn_sched_barrier(0);

  // 5. gate/up dot products; waves 1..15 first issue their W2 units, in the
  //    same straight-line branch.  Unit u = (wave - 1) + 15 i (i < 4) is route
  //    u / DL, 1 KB chunk u % DL of the down rows; every wave issues exactly
  //    four loads (units past k * DL, masked routes and missing routes load a
  //    valid row and are discarded).
  float part;
  uint4 wb[kDownUnitsPerWave];
  const float* wsc = s_tab + (wave < 8 ? 0 : G);
  if (wave >= 1) {
#pragma unroll
    for (int i = 0; i < kDownUnitsPerWave; i++) {
      const int u = min((wave - 1) + 15 * i, k * DL - 1);
      const int j = u / DL, c = u - j * DL;
      const int ee = s_e[j] >= 0 ? s_e[j] : 0;
      const int row = min(d0 + c * rpl + lane / lpr, H - 1);
      wb[i] = *reinterpret_cast<const uint4*>(w2 + ((size_t)ee * H + row) * I + 16 * (lane % lpr));
    }
    __builtin_amdgcn_sched_barrier(0);
    part = gate_up_row<RL>(wa, s_af, s_as, wsc, H, lane);
  } else {
    part = gate_up_row<RL>(wa, s_af, s_as, wsc, H, lane);
  }
  {
    const float t = wave_sum(part);
    if (lane == 0) s_rows[wave] = t;
  }
  wg_sync();

  // 6. SwiGLU on the BF16 gate/up values; act rows stored by wave 0
  if (e >= 0 && wave == 0 && lane < 2 * kMaxK) {
    const uint32_t mask = s_route_mask;
    const int r_idx = lane >> 1, half = lane & 1;  // lane pairs: route, 4 of the 8 columns
    int r = -1, cnt = 0;
    for (int q = 0; q < k; q++)
      if ((mask >> q) & 1) {
        if (cnt == r_idx) r = q;
        cnt++;
      }
    if (r >= 0) {
      uint32_t h[4];
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const int i = 4 * half + v;
        const float g = bf16_to_f32(f32_to_bf16(s_rows[i]));
        const float u = bf16_to_f32(f32_to_bf16(s_rows[8 + i]));
        h[v] = f32_to_bf16(swiglu_bf16(g, u, limit, clamp != 0));
      }
      const uint64_t o = (uint64_t)(h[0] | (h[1] << 16)) | ((uint64_t)(h[2] | (h[3] << 16)) << 32);
      ATOMIC_ST(reinterpret_cast<uint64_t*>(act + (size_t)r * I + n0 + 4 * half), o);
    }
  }

  // 7. every act row is complete past this point
  grid_barrier(bar, gridDim.x, wave);
  if (d0 >= H) return;

  // 8. the k act rows, quantised per group of 128 and dequantised into LDS,
  //    by waves 0..7 (one group per 16 lanes; waves 8..15 wait for W2 data)
  if (wave < 8) {
    const int gid = tid >> 4;
    if (gid < k * GI) {
      const int j = gid / GI, g = gid - j * GI;
      if (s_e[j] >= 0) {
        const uint64_t* src = reinterpret_cast<const uint64_t*>(act + (size_t)j * I + g * 128 + l16 * 8);
        const uint64_t a0 = ATOMIC_LD(src), a1 = ATOMIC_LD(src + 1);
        const uint4 v = make_uint4((uint32_t)a0, (uint32_t)(a0 >> 32), (uint32_t)a1, (uint32_t)(a1 >> 32));
        float f[8], d[8];
        unpack8(v, f);
        const float sc = group_scale(max_over_16(amax8(f)), fmt);
        quant_dequant8(f, sc, d);
        float* dst = &s_qf[j][g * 128 + l16 * 8];
        *reinterpret_cast<float4*>(dst) = make_float4(d[0], d[1], d[2], d[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(d[4], d[5], d[6], d[7]);
        if (l16 == 0) s_qs[j][g] = sc;
      }
    }
  }
  wg_sync();

  // 9. down projection: each of waves 1..15 finishes its W2 units
  if (wave >= 1) {
#pragma unroll
    for (int i = 0; i < kDownUnitsPerWave; i++) {
      const int u = (wave - 1) + 15 * i;
      if (u >= k * DL) break;
      const int j = u / DL, c = u - j * DL;
      if (s_e[j] < 0) continue;
      const int kof = 16 * (lane % lpr);
      const int row = min(d0 + c * rpl + lane / lpr, H - 1);
      const float w2sc = s_tab[2 * G + (j * 2 + (row / 128 == rb0 ? 0 : 1)) * GI + kof / 128];
      float v = dot16(wb[i], &s_qf[j][kof]) * (s_qs[j][kof / 128] * w2sc);
      for (int m = lpr / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m);
      const int rl = c * rpl + lane / lpr;
      if (lane % lpr == 0 && d0 + rl < d_end) s_y[j][rl] = bf16_to_f32(f32_to_bf16(v));
    }
  }
  wg_sync();

  // 10. weighted reduction over the routes, j ascending
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
  if (dr * I / 1024 != (H + 1023) / 1024) return false;  // kernels are instantiated for equal load counts
  if (k * (dr * I / 1024) > 15 * kDownUnitsPerWave) return false;  // W2 units of waves 1..15
  const int grid = token_kernel_grid(H, k, L, I);
  return grid <= num_cus && grid <= kMaxGrid;
}

hipError_t launch_token_layer(const uint16_t* hidden, int H, const int32_t* ids, const float* topk_w, int k,
                              int32_t offset, int32_t L, const uint8_t* w13, const float* w13_s, const uint8_t* w2,
                              const float* w2_s, int I, int fmt, float limit, uint16_t* act, void* barrier,
                              uint16_t* out, hipStream_t stream, const LaunchHook* hook) {
  const int clamp = __builtin_isfinite(limit) ? 1 : 0;
  const int slots = k < L ? k : L;
  const int dr = token_down_rows(H, I, slots * (I / 8));
  const int grid = token_kernel_grid(H, k, L, I);
  const int rl = (H + 1023) / 1024, dl = dr * I / 1024;
  if (rl != dl || rl < 1 || rl > kMaxRowLoads) return hipErrorInvalidValue;  // token_path_fits rules this out
  if (hook) hook->before(0, stream);
#define BFP8_TOKEN_CASE(N)                                                                                   \
  case N:                                                                                                    \
    hipLaunchKernelGGL((token_layer_kernel<N, N>), dim3(grid), dim3(kThreads), 0, stream, hidden, H, ids,    \
                       topk_w, k, offset, L, w13, w13_s, w2, w2_s, I, fmt, limit, clamp, dr, act,           \
                       static_cast<TokenBarrier*>(barrier), out);                                            \
    break;
  switch (rl) {
    BFP8_TOKEN_CASE(1)
    BFP8_TOKEN_CASE(2)
    BFP8_TOKEN_CASE(3)
    BFP8_TOKEN_CASE(4)
    BFP8_TOKEN_CASE(5)
    BFP8_TOKEN_CASE(6)
    BFP8_TOKEN_CASE(7)
    BFP8_TOKEN_CASE(8)
  }
#undef BFP8_TOKEN_CASE
  hipError_t e = hipGetLastError();
  if (hook) hook->before(1, stream);
  return e;
}

}  // namespace bfp8
