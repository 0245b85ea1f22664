// decode.hip -- the small-batch (decode) path of the fused layer: two kernels
// instead of route prep + quant + GEMM + act/quant + GEMM + reduce.
//
// [P1 Motivation] at M = 1, top-k 8, E = 256 at most eight experts are active;
// the layer is pure weight streaming (44 MB of W13 + W2 at the 7168 x 256
// decode shape), so the design goal is one pass over the active experts'
// weights with as many loads in flight as early as possible.
// [P1 Modification, Active-expert block scheduling] workgroups exist per active
// expert slot; slots past the number of distinct experts exit at once.
// [P1 Modification, Fused SwiGLU and FP8 quantization] the gate/up kernel's
// epilogue applies SwiGLU; the SwiGLU output is group-quantised inside the down
// kernel, per route, without a separate launch.
// [P4 Pull request overview] the down kernel ends with the top-k weighted
// reduction in route order.
//
// gate/up kernel (one workgroup = one active expert x 8 gate + 8 up rows):
//   1. local expert of every route (R <= 64) -> this slot's expert and its
//      routes, ascending, in LDS;
//   2. every wave issues all of its W13 loads at once (its K chunks are
//      w, w+4, w+8, ...), 32 bytes per lane per chunk, straight to registers;
//   3. the hidden rows of the expert's tokens are group-quantised into LDS
//      (same arithmetic as quant_fp8) while those loads are in flight;
//   4. MFMA 16x16x128 per chunk: A = 16 weight rows, B = up to 16 routes;
//      result x (a_scale * w_scale) accumulated in fp32;
//   5. the 4 waves' partial sums are added in wave order in LDS, rounded to
//      BF16 (the gate/up output), and SwiGLU gives act[r, n] in BF16.
// down + reduce kernel (one workgroup = one token x 32 output rows):
//   1. the token's k routes and weights;
//   2. W2 loads for the wave's routes (j = wave, wave + 4) issued at once;
//   3. the k act rows are group-quantised into LDS (same arithmetic as
//      silu_and_mul_quant_fp8);
//   4. MFMA per route, scales, BF16 y values in LDS;
//   5. out[t, n] = bf16(fmaf chain over j ascending) over live routes.
//
// Pages cited in brackets, by key and section:
//   [P1] lmdeploy PR "Perf/pytorch block fp8 moe decode"
//   [P2] lmdeploy PR "perf(pytorch): optimize compact blocked FP8 MoE and route
//        preparation"
//   [P3] vLLM PR "[Kernel][Perf] Fuse clamped MoE activation and UE8M0 FP8 block
//        quantization"
//   [P4] lmdeploy PR "Moe Reduce kernel"
#include <mutex>

#include "device.h"
#include "internal.h"
#include "mfma.h"

namespace bfp8 {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxR = 64;      // routes of the decode path
constexpr int kMaxTok = 8;     // tokens
constexpr int kMaxCpw = 16;    // K chunks per wave in the gate/up kernel (H <= 8192)
constexpr int kMaxK = 8;       // top-k in the down kernel
constexpr int kMaxG2 = 4;      // K chunks of the down projection (I <= 512)
constexpr int kDownRows = 32;  // output rows per down workgroup

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

// LDS fragment load (32 bytes, same K slot order as load_frag).
__device__ __forceinline__ v8i lds_frag(const uint8_t* p, int kq) {
  const uint4 lo = *reinterpret_cast<const uint4*>(p + 16 * kq);
  const uint4 hi = *reinterpret_cast<const uint4*>(p + 64 + 16 * kq);
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

// ------------------------------------------------------------------ gate/up

// Quantise one token row (G groups of 128, G <= 64) held as 4 loads per
// thread: groups p*16 + tid/16, p = 0..3, 8 values per lane.
__device__ __forceinline__ void quant_row_to_lds(const uint4 (&v)[4], int G, int fmt, uint8_t* aq_row,
                                                 float* as_row) {
  const int l16 = threadIdx.x & 15;
#pragma unroll
  for (int p = 0; p < 4; p++) {
    const int g = p * 16 + (threadIdx.x >> 4);
    if (g < G) {  // uniform across each 16-lane group
      float f[8];
      unpack8(v[p], f);
      const float sc = group_scale(max_over_16(amax8(f)), fmt);
      *reinterpret_cast<uint2*>(aq_row + (size_t)g * kGroup + l16 * 8) = encode8_scaled(f, sc);
      if (l16 == 0) as_row[g] = sc;
    }
  }
}

// Issue the 4 loads of one token row (addresses clamped into the row, so the
// loads are unconditional and leave back to back).
__device__ __forceinline__ void load_row(const uint16_t* __restrict__ row, int G, uint4 (&v)[4]) {
  const int l16 = threadIdx.x & 15;
#pragma unroll
  for (int p = 0; p < 4; p++) {
    const int g = min(p * 16 + (int)(threadIdx.x >> 4), G - 1);
    v[p] = *reinterpret_cast<const uint4*>(row + (size_t)g * kGroup + l16 * 8);
  }
}

__global__ __launch_bounds__(kThreads) void decode_gate_up_kernel(
    const uint16_t* __restrict__ hidden, int M, int H, const int32_t* __restrict__ ids, int k, ExpertSel sel,
    const uint8_t* __restrict__ w13, const float* __restrict__ w13_s, int I, int fmt, float limit,
    int clamp, int tile_cap, uint16_t* __restrict__ act) {
  __shared__ int s_e[kMaxR];
  __shared__ int s_first[kMaxR];
  __shared__ int s_routes[kMaxR];
  __shared__ int s_expert, s_nroutes;
  extern __shared__ __align__(16) uint8_t dyn[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, kq = lane >> 4;
  const int R = M * k;
  const int G = H / kGroup;
  const int slot = blockIdx.y;
  const int n0 = blockIdx.x * 8;  // gate rows n0..n0+7, up rows I+n0..I+n0+7
  uint8_t* aq = dyn;                                                  // [M][H]
  float* as = reinterpret_cast<float*>(dyn + (size_t)M * H);          // [M][G]
  float* part = as + (size_t)M * G;                                   // [4][tile_cap][64][4]

  // 0. routing ids, and the first 4 tokens' hidden rows: nothing depends on
  //    anything yet, so all of these loads leave at once
  int e_mine = -1;
  if (tid < R) e_mine = local_of(sel, ids[tid]);
  uint4 hv[4][4];
#pragma unroll
  for (int t = 0; t < 4; t++) load_row(hidden + (size_t)min(t, M - 1) * H, G, hv[t]);

  // 1. which expert this workgroup serves, and its routes
  if (tid == 0) { s_expert = -1; s_nroutes = 0; }
  if (tid < R) s_e[tid] = e_mine;
  __syncthreads();
  if (tid < R) {
    bool first = e_mine >= 0;
    for (int r = 0; r < tid; r++) first = first && (s_e[r] != e_mine);
    s_first[tid] = first ? 1 : 0;
  }
  __syncthreads();
  if (tid < R && s_first[tid]) {
    int rank = 0, cnt = 0;
    for (int r = 0; r < R; r++) {
      rank += (s_first[r] && s_e[r] < e_mine) ? 1 : 0;
      cnt += (s_e[r] == e_mine) ? 1 : 0;
    }
    if (rank == slot) { s_expert = e_mine; s_nroutes = cnt; }
  }
  __syncthreads();
  const int e = __builtin_amdgcn_readfirstlane(s_expert);
  if (e < 0) return;  // slot beyond the number of active experts
  const int nroutes = s_nroutes;
  if (tid < R && e_mine == e) {
    int pos = 0;
    for (int r = 0; r < tid; r++) pos += (s_e[r] == e) ? 1 : 0;
    s_routes[pos] = tid;
  }

  // 2. weight scales (wave-uniform addresses) and all of this wave's W13
  //    fragments; chunk c of wave w is K chunk w + 4c
  const int nc = (G - wave + 3) / 4;
  const float* gs = w13_s + ((size_t)e * (2 * I / kGroup) + n0 / kGroup) * G;
  const float* us = w13_s + ((size_t)e * (2 * I / kGroup) + (I + n0) / kGroup) * G;
  float gsc[kMaxCpw], usc[kMaxCpw];
#pragma unroll
  for (int c = 0; c < kMaxCpw; c++) {
    const int g = min(wave + 4 * c, G - 1);
    gsc[c] = gs[g];
    usc[c] = us[g];
  }
  const int wrow_idx = col < 8 ? n0 + col : I + n0 + (col - 8);
  const uint8_t* wrow = w13 + ((size_t)e * 2 * I + wrow_idx) * H;
  v8i wa[kMaxCpw];
#pragma unroll
  for (int c = 0; c < kMaxCpw; c++)
    if (c < nc) wa[c] = load_frag(wrow + (size_t)(wave + 4 * c) * kGroup, kq);

  // 3. quantise every token's hidden row into LDS (tokens 0..3 already loaded)
#pragma unroll
  for (int t = 0; t < 4; t++)
    if (t < M) quant_row_to_lds(hv[t], G, fmt, aq + (size_t)t * H, as + (size_t)t * G);
  for (int t = 4; t < M; t++) {
    load_row(hidden + (size_t)t * H, G, hv[0]);
    quant_row_to_lds(hv[0], G, fmt, aq + (size_t)t * H, as + (size_t)t * G);
  }
  __syncthreads();

  // 4. MFMA over this wave's chunks, up to 4 tiles of 16 routes
  const int ntiles = (nroutes + 15) / 16;
  int tok[kMaxR / 16];
#pragma unroll
  for (int t = 0; t < kMaxR / 16; t++) {
    const int j = t * 16 + col;
    tok[t] = (t < ntiles && j < nroutes) ? s_routes[j] / k : -1;
  }
  v4f acc[kMaxR / 16];
#pragma unroll
  for (int t = 0; t < kMaxR / 16; t++) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < kMaxCpw; c++) {
    if (c < nc) {
      const int g = wave + 4 * c;
      const float wsc = kq < 2 ? gsc[c] : usc[c];
#pragma unroll
      for (int t = 0; t < kMaxR / 16; t++) {
        if (t < ntiles) {
          v8i b = zero_frag();
          float csc = 0.0f;
          if (tok[t] >= 0) {
            b = lds_frag(aq + (size_t)tok[t] * H + (size_t)g * kGroup, kq);
            csc = as[tok[t] * G + g] * wsc;
          }
          const v4f p = mfma_f8_16x16x128(wa[c], b, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int v = 0; v < 4; v++) acc[t][v] = __builtin_fmaf(p[v], csc, acc[t][v]);
        }
      }
    }
  }

  // 5. add the waves' partial sums in wave order, SwiGLU, store
#pragma unroll
  for (int t = 0; t < kMaxR / 16; t++)
    if (t < ntiles)
      *reinterpret_cast<float4*>(part + (((size_t)wave * tile_cap + t) * 64 + lane) * 4) =
          make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < kMaxR / 16; t++) {
      if (t >= ntiles) break;
      float sum[4] = {0.f, 0.f, 0.f, 0.f};
      for (int w = 0; w < 4; w++) {
        const float4 pw = *reinterpret_cast<const float4*>(part + (((size_t)w * tile_cap + t) * 64 + lane) * 4);
        sum[0] += pw.x; sum[1] += pw.y; sum[2] += pw.z; sum[3] += pw.w;
      }
      // lanes kq = 0, 1 hold gate rows 4kq+v; lanes kq = 2, 3 the matching up rows
      float u[4];
#pragma unroll
      for (int v = 0; v < 4; v++) u[v] = __shfl(sum[v], lane + 32);
      const int j = t * 16 + col;
      if (kq < 2 && j < nroutes) {
        const int r = s_routes[j];
        uint32_t h[4];
#pragma unroll
        for (int v = 0; v < 4; v++) {
          const float g = bf16_to_f32(f32_to_bf16(sum[v]));
          const float up = bf16_to_f32(f32_to_bf16(u[v]));
          h[v] = f32_to_bf16(swiglu_bf16(g, up, limit, clamp != 0));
        }
        uint2 o;
        o.x = h[0] | (h[1] << 16);
        o.y = h[2] | (h[3] << 16);
        *reinterpret_cast<uint2*>(act + (size_t)r * I + n0 + 4 * kq) = o;
      }
    }
  }
}

// ------------------------------------------------------------------ down + reduce

__global__ __launch_bounds__(kThreads) void decode_down_reduce_kernel(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ ids, const float* __restrict__ topk_w, int k,
    ExpertSel sel, const uint8_t* __restrict__ w2, const float* __restrict__ w2_s, int H, int I,
    int fmt, uint16_t* __restrict__ out) {
  __shared__ int s_e[kMaxK];
  __shared__ float s_w[kMaxK];
  __shared__ __align__(16) uint8_t s_q[kMaxK][kMaxG2 * kGroup];
  __shared__ float s_s[kMaxK][kMaxG2];
  __shared__ float s_y[kMaxK][kDownRows];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, kq = lane >> 4;
  const int t = blockIdx.y;
  const int n0 = blockIdx.x * kDownRows;
  const int G2 = I / kGroup;
  const int GH = H / kGroup;
  const int l16 = tid & 15;
  const int ngroups = k * G2;  // <= 32

  // 0. the token's k act rows (written by the gate/up kernel): 2 loads per
  //    thread, addresses clamped so both leave unconditionally
  uint4 av[2];
#pragma unroll
  for (int p = 0; p < 2; p++) {
    const int gid = min(p * 16 + (tid >> 4), ngroups - 1);
    const int j = gid / G2, g = gid - j * G2;
    av[p] = *reinterpret_cast<const uint4*>(act + ((size_t)t * k + j) * I + (size_t)g * kGroup + l16 * 8);
  }
  // 1. this wave's routes (wave-uniform loads), then their W2 fragments and scales
  int ej[2];
#pragma unroll
  for (int jj = 0; jj < 2; jj++) {
    const int j = wave + 4 * jj;
    ej[jj] = -1;
    if (j < k) ej[jj] = local_of(sel, ids[(size_t)t * k + j]);
  }
  const int rblk = n0 / kGroup;
  v8i wb[2][2][kMaxG2];
  float wsc[2][kMaxG2];
#pragma unroll
  for (int jj = 0; jj < 2; jj++) {
    const int ee = ej[jj] >= 0 ? ej[jj] : 0;
#pragma unroll
    for (int c = 0; c < kMaxG2; c++) wsc[jj][c] = w2_s[((size_t)ee * GH + rblk) * G2 + min(c, G2 - 1)];
#pragma unroll
    for (int rt = 0; rt < 2; rt++)
#pragma unroll
      for (int c = 0; c < kMaxG2; c++)
        if (ej[jj] >= 0 && c < G2)
          wb[jj][rt][c] = load_frag(w2 + ((size_t)ej[jj] * H + n0 + rt * 16 + col) * I + (size_t)c * kGroup, kq);
  }

  if (tid < k) {
    s_e[tid] = local_of(sel, ids[(size_t)t * k + tid]);
    s_w[tid] = topk_w[(size_t)t * k + tid];
  }

  // 2. group-quantise the act rows into LDS (masked routes' rows are not used)
#pragma unroll
  for (int p = 0; p < 2; p++) {
    const int gid = p * 16 + (tid >> 4);
    if (gid < ngroups) {  // uniform across the 16-lane group
      const int j = gid / G2, g = gid - j * G2;
      float f[8];
      unpack8(av[p], f);
      const float sc = group_scale(max_over_16(amax8(f)), fmt);
      *reinterpret_cast<uint2*>(&s_q[j][g * kGroup + l16 * 8]) = encode8_scaled(f, sc);
      if (l16 == 0) s_s[j][g] = sc;
    }
  }
  __syncthreads();

  // 3. per route: y = bf16(sum_c mfma * scale) for 32 rows
#pragma unroll
  for (int jj = 0; jj < 2; jj++) {
    const int j = wave + 4 * jj;
    if (j >= k || ej[jj] < 0) continue;
#pragma unroll
    for (int rt = 0; rt < 2; rt++) {
      v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < kMaxG2; c++) {
        if (c < G2) {
          const v8i b = lds_frag(&s_q[j][c * kGroup], kq);
          const v4f p = mfma_f8_16x16x128(wb[jj][rt][c], b, v4f{0.f, 0.f, 0.f, 0.f});
          const float csc = s_s[j][c] * wsc[jj][c];
#pragma unroll
          for (int v = 0; v < 4; v++) acc[v] = __builtin_fmaf(p[v], csc, acc[v]);
        }
      }
      // every column holds the same sums (B is the same route in all 16)
      if (col == 0) {
#pragma unroll
        for (int v = 0; v < 4; v++) s_y[j][rt * 16 + 4 * kq + v] = bf16_to_f32(f32_to_bf16(acc[v]));
      }
    }
  }
  __syncthreads();

  // 4. weighted reduction over the routes, j ascending
  if (tid < kDownRows) {
    float a = 0.0f;
    for (int j = 0; j < k; j++)
      if (s_e[j] >= 0) a = __builtin_fmaf(s_w[j], s_y[j][tid], a);
    out[(size_t)t * H + n0 + tid] = (uint16_t)f32_to_bf16(a);
  }
}


}  // namespace

bool decode_path_fits(int64_t M, int H, int k, int I) {
  return M >= 1 && M <= kMaxTok && M * k <= kMaxR && k <= kMaxK && H <= kMaxCpw * 4 * kGroup &&
         I <= kMaxG2 * kGroup && I % 8 == 0;
}

int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

// LDS of the gate/up kernel: the M quantised hidden rows, their scales, and
// the 4 waves' partial sums for up to tile_cap route tiles.
size_t decode_gate_up_lds(int H, int M, int tile_cap) {
  const int G = H / kGroup;
  return (size_t)M * H + sizeof(float) * M * G + sizeof(float) * 4 * tile_cap * 64 * 4;
}

hipError_t launch_decode_layer(const uint16_t* hidden, int64_t M, int H, const int32_t* ids, const float* topk_w,
                               int k, const ExpertSel& sel, const uint8_t* w13, const float* w13_s,
                               const uint8_t* w2, const float* w2_s, int I, int fmt, float limit, uint16_t* act,
                               uint16_t* out, hipStream_t stream, const LaunchHook* hook) {
  const int R = (int)M * k;
  const int slots = R < sel.L ? R : sel.L;
  const int clamp = __builtin_isfinite(limit) ? 1 : 0;
  // an expert serves at most R routes
  const int tile_cap = (R + 15) / 16;
  const size_t lds = decode_gate_up_lds(H, (int)M, tile_cap);
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute((const void*)decode_gate_up_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)decode_gate_up_lds(kMaxCpw * 4 * kGroup, kMaxTok, kMaxR / 16));
    (void)hipGetLastError();
  });
  if (hook) hook->before(0, stream);
  if (!hook || hook->run(0))
    hipLaunchKernelGGL(decode_gate_up_kernel, dim3(I / 8, slots), dim3(kThreads), lds, stream, hidden, (int)M, H,
                       ids, k, sel, w13, w13_s, I, fmt, limit, clamp, tile_cap, act);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (hook) hook->before(1, stream);
  if (!hook || hook->run(1))
    hipLaunchKernelGGL(decode_down_reduce_kernel, dim3(H / kDownRows, (unsigned)M), dim3(kThreads), 0, stream,
                       act, ids, topk_w, k, sel, w2, w2_s, H, I, fmt, out);
  e = hipGetLastError();
  if (hook) hook->before(2, stream);
  return e;
}

}  // namespace bfp8
