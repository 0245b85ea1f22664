// router.hip -- single-group top-k router for gfx950: router logits [M, E]
// fp32 -> the k chosen experts per token (largest first) and their weights.
//
// [P2 Changes: a fused single-group top-k router; renormalize option]
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

template <int NPL>
__global__ __launch_bounds__(kRouterThreads) void router_topk_kernel(const float* __restrict__ logits, int64_t M,
                                                                     int E, int k, int score_fn,
                                                                     const float* __restrict__ bias, int renorm,
                                                                     double scale, int32_t* __restrict__ ids,
                                                                     float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kTokensPerWG + (threadIdx.x >> 6);
  if (t >= M) return;  // whole waves only: the reductions need all 64 lanes
  router::WaveRoute<NPL> r;
  r.load(logits + t * (int64_t)E, E, score_fn, bias, lane);
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

template <int NPL>
hipError_t launch_npl(const float* logits, int64_t M, int E, int k, int score_fn, const float* bias, int renorm,
                      double scale, int32_t* ids, float* w, hipStream_t stream) {
  const int64_t grid = (M + kTokensPerWG - 1) / kTokensPerWG;
  hipLaunchKernelGGL(router_topk_kernel<NPL>, dim3((unsigned)grid), dim3(kRouterThreads), 0, stream, logits, M, E, k,
                     score_fn, bias, renorm, scale, ids, w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router_topk(const float* logits, int64_t M, int E, int k, int score_fn, const float* bias,
                              int renorm, double scale, int32_t* ids, float* w, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (E <= 64) return launch_npl<1>(logits, M, E, k, score_fn, bias, renorm, scale, ids, w, stream);
  if (E <= 128) return launch_npl<2>(logits, M, E, k, score_fn, bias, renorm, scale, ids, w, stream);
  if (E <= 256) return launch_npl<4>(logits, M, E, k, score_fn, bias, renorm, scale, ids, w, stream);
  if (E <= 512) return launch_npl<8>(logits, M, E, k, score_fn, bias, renorm, scale, ids, w, stream);
  return launch_npl<16>(logits, M, E, k, score_fn, bias, renorm, scale, ids, w, stream);
}

}  // namespace bfp8
