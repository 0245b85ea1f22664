// router.hip -- top-k routers for gfx950: router logits [M, E] fp32 -> the k
// chosen experts per token (largest first) and their weights; single-group,
// and group-limited noaux-TC.
//
// [P2 Changes: a fused single-group top-k router; renormalize option]
// [P2 Reviewed changes: route_noaux_tc.py, a noaux-TC routing kernel]
//   [P2] lmdeploy PR "perf(pytorch): optimize compact blocked FP8 MoE and route
//        preparation"
//
// Work mapping: one wave per token (the wave-level steps are in router.h),
// four tokens per 256-thread workgroup.  Lane j keeps the j-th winner; the
// weights are formed in fp64 and rounded once to fp32.
#include "device.h"
#include "internal.h"
#include "router.h"

namespace bfp8 {

namespace {

constexpr int kRouterThreads = 256;
constexpr int kTokensPerWG = kRouterThreads / 64;
// From this many tokens the router takes 16 lanes per token (below: a wave).
// Measured at E = 256, k = 8: 8.8 against 12.6 us (softmax) and 15.8 against
// 17.9 (sigmoid) at 16,384 tokens, but slower at 256 to 4,096 tokens, where
// there are few waves and each lane's 16 loads and fp64 sigmoids make a wave
// four times longer.
constexpr int64_t kRowsMinM = 8192;

template <int NPL, bool kGrouped>
__global__ __launch_bounds__(kRouterThreads) void router_topk_kernel(const float* __restrict__ logits, int64_t M,
                                                                     int E, int k, int score_fn,
                                                                     const float* __restrict__ bias, int renorm,
                                                                     double scale, int32_t* __restrict__ ids,
                                                                     float* __restrict__ w, int n_group,
                                                                     int topk_group) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kTokensPerWG + (threadIdx.x >> 6);
  if (t >= M) return;  // whole waves only: the reductions need all 64 lanes
  router::WaveRoute<NPL> r;
  if constexpr (kGrouped) {
    __shared__ float s_key[kTokensPerWG][64 + 64 * NPL];  // each wave's group scores and choice keys
    r.load(logits + t * (int64_t)E, E, score_fn, bias, lane, n_group, topk_group, s_key[threadIdx.x >> 6]);
  } else {
    r.load(logits + t * (int64_t)E, E, score_fn, bias, lane);
  }
  // k rounds; lane j keeps winner j
  int my_id = 0;
  float my_logit = 0.0f;
  for (int j = 0; j < k; j++) {
    float lv;
    const int e = r.take(lane, lv);
    if (lane == j) {
      my_id = e;
      my_logit = lv;
    }
  }
  const float wt = r.weight(my_logit, lane, E, k, score_fn, renorm, scale);
  if (lane < k) {
    ids[t * k + lane] = my_id;
    w[t * k + lane] = wt;
  }
}

// Many tokens: the kernel above is bound by instruction issue, one wave per
// token.  Here 16 lanes (one DPP row) route one token, four tokens per wave,
// with row-local steps only.  Lane l of a row holds experts l, l + 16, ...,
// l + 240 (E <= 256).  A round: the row's largest key (DPP maxima, every lane
// of the row ends with it); each lane's lowest expert id holding it, and the
// row's minimum of those (DPP minima); the owner lane retires it.  Lane j of
// the row keeps winner j (k <= 16); the logits of the k winners are read back
// (cached) for the weights.
constexpr int kRowTokensPerWG = kRouterThreads / 16;

template <int CTRL>
__device__ __forceinline__ uint32_t row_dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ double row_dpp_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  return __builtin_bit_cast(double, (uint64_t)row_dpp<CTRL>((uint32_t)u) |
                                        ((uint64_t)row_dpp<CTRL>((uint32_t)(u >> 32)) << 32));
}

__device__ __forceinline__ uint32_t row_max(uint32_t v) {
  v = max(v, row_dpp<0xB1>(v));   // quad_perm 1,0,3,2
  v = max(v, row_dpp<0x4E>(v));   // quad_perm 2,3,0,1
  v = max(v, row_dpp<0x141>(v));  // row_half_mirror
  return max(v, row_dpp<0x140>(v));  // row_mirror
}

__device__ __forceinline__ uint32_t row_min(uint32_t v) {
  v = min(v, row_dpp<0xB1>(v));
  v = min(v, row_dpp<0x4E>(v));
  v = min(v, row_dpp<0x141>(v));
  return min(v, row_dpp<0x140>(v));
}

__device__ __forceinline__ double row_sum_f64(double v) {
  v += row_dpp_f64<0xB1>(v);
  v += row_dpp_f64<0x4E>(v);
  v += row_dpp_f64<0x141>(v);
  return v + row_dpp_f64<0x140>(v);
}

__global__ __launch_bounds__(kRouterThreads) void router_topk_rows_kernel(const float* __restrict__ logits, int64_t M,
                                                                          int E, int k, int score_fn,
                                                                          const float* __restrict__ bias, int renorm,
                                                                          double scale, int32_t* __restrict__ ids,
                                                                          float* __restrict__ w) {
  constexpr int S = 16;  // experts per lane
  const int l = threadIdx.x & 15;
  // a row past the last token routes the last token again and stores nothing,
  // so every lane takes part in the row steps
  const int64_t t0 = (int64_t)blockIdx.x * kRowTokensPerWG + (threadIdx.x >> 4);
  const bool live = t0 < M;
  const int64_t t = live ? t0 : M - 1;
  const float* lg = logits + t * (int64_t)E;
  float v[S];
  uint32_t key[S];
#pragma unroll
  for (int i = 0; i < S; i++) v[i] = lg[min(l + 16 * i, E - 1)];
#pragma unroll
  for (int i = 0; i < S; i++) {
    float s = v[i];
    if (score_fn == kScoreSigmoid) {
      s = router::sigmoid_rn(v[i]);
      if (bias) s = s + bias[min(l + 16 * i, E - 1)];
    }
    key[i] = l + 16 * i < E ? router::order_bits(s) : 0u;
  }
  int my_id = 0;
  for (int j = 0; j < k; j++) {
    uint32_t best = key[0];
#pragma unroll
    for (int i = 1; i < S; i++) best = max(best, key[i]);
    const uint32_t top = row_max(best);
    uint32_t cand = 0xFFFFFFFFu;  // this lane's lowest expert id holding the top key
#pragma unroll
    for (int i = S - 1; i >= 0; i--)
      if (key[i] == top) cand = (uint32_t)(l + 16 * i);
    const uint32_t win = row_min(cand);
#pragma unroll
    for (int i = 0; i < S; i++)
      if ((uint32_t)(l + 16 * i) == win) key[i] = 0u;  // retired
    if (l == j) my_id = (int)win;
  }
  const bool chosen = l < k;
  const float my_logit = lg[chosen ? my_id : 0];
  double num = 0.0, z = 1.0;
  if (score_fn == kScoreSoftmax) {
    // the largest logit is the first winner's (lane 0 of the row)
    const float top_logit = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                                          (int)((threadIdx.x & ~15u) & 63u) * 4,
                                                          __builtin_bit_cast(int, my_logit)));
    const double m = (double)top_logit;
    num = chosen ? exp((double)my_logit - m) : 0.0;
    if (renorm) {
      z = row_sum_f64(num);
    } else {
      double part = 0.0;
#pragma unroll
      for (int i = 0; i < S; i++)
        if (l + 16 * i < E) part += exp((double)v[i] - m);
      z = row_sum_f64(part);
    }
  } else {
    num = chosen ? 1.0 / (1.0 + exp(-(double)my_logit)) : 0.0;
    z = renorm ? row_sum_f64(num) : 1.0;
  }
  if (live && chosen) {
    ids[t * k + l] = my_id;
    w[t * k + l] = (float)(num / z * scale);
  }
}

template <int NPL>
hipError_t launch_npl(const float* logits, int64_t M, int E, int k, int score_fn, const float* bias, int renorm,
                      double scale, int32_t* ids, float* w, hipStream_t stream, int n_group = 1,
                      int topk_group = 1) {
  const int64_t grid = (M + kTokensPerWG - 1) / kTokensPerWG;
  if (n_group > 1)
    hipLaunchKernelGGL((router_topk_kernel<NPL, true>), dim3((unsigned)grid), dim3(kRouterThreads), 0, stream, logits,
                       M, E, k, score_fn, bias, renorm, scale, ids, w, n_group, topk_group);
  else
    hipLaunchKernelGGL((router_topk_kernel<NPL, false>), dim3((unsigned)grid), dim3(kRouterThreads), 0, stream,
                       logits, M, E, k, score_fn, bias, renorm, scale, ids, w, 1, 1);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router_topk(const float* logits, int64_t M, int E, int k, int score_fn, const float* bias,
                              int renorm, double scale, int32_t* ids, float* w, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (M >= kRowsMinM && E <= 256 && k <= 16) {
    const int64_t grid = (M + kRowTokensPerWG - 1) / kRowTokensPerWG;
    hipLaunchKernelGGL(router_topk_rows_kernel, dim3((unsigned)grid), dim3(kRouterThreads), 0, stream, logits, M, E,
                       k, score_fn, bias, renorm, scale, ids, w);
    return hipGetLastError();
  }
  if (E <= 64) return launch_npl<1>(logits, M, E, k, score_fn, bias, renorm, scale, ids, w, stream);
  if (E <= 128) return launch_npl<2>(logits, M, E, k, score_fn, bias, renorm, scale, ids, w, stream);
  if (E <= 256) return launch_npl<4>(logits, M, E, k, score_fn, bias, renorm, scale, ids, w, stream);
  if (E <= 512) return launch_npl<8>(logits, M, E, k, score_fn, bias, renorm, scale, ids, w, stream);
  return launch_npl<16>(logits, M, E, k, score_fn, bias, renorm, scale, ids, w, stream);
}

hipError_t launch_router_noaux_tc(const float* logits, int64_t M, int E, int k, int n_group, int topk_group,
                                  const float* bias, int renorm, double scale, int32_t* ids, float* w,
                                  hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (n_group <= 1)
    return launch_router_topk(logits, M, E, k, kScoreSigmoid, bias, renorm, scale, ids, w, stream);
  const int s = kScoreSigmoid;
  if (E <= 64) return launch_npl<1>(logits, M, E, k, s, bias, renorm, scale, ids, w, stream, n_group, topk_group);
  if (E <= 128) return launch_npl<2>(logits, M, E, k, s, bias, renorm, scale, ids, w, stream, n_group, topk_group);
  if (E <= 256) return launch_npl<4>(logits, M, E, k, s, bias, renorm, scale, ids, w, stream, n_group, topk_group);
  if (E <= 512) return launch_npl<8>(logits, M, E, k, s, bias, renorm, scale, ids, w, stream, n_group, topk_group);
  return launch_npl<16>(logits, M, E, k, s, bias, renorm, scale, ids, w, stream, n_group, topk_group);
}

}  // namespace bfp8
