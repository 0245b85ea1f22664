// router.hip -- single-group top-k router for gfx950: router logits [M, E]
// fp32 -> the k chosen experts per token (largest first) and their weights.
//
// [P2 Changes: a fused single-group top-k router; renormalize option]
//   [P2] lmdeploy PR "perf(pytorch): optimize compact blocked FP8 MoE and route
//        preparation"
//
// Work mapping: one wave per token, four tokens per 256-thread workgroup.
// Lane l holds experts l, l + 64, ... (NPL of them, loads contiguous across
// lanes).  Each expert becomes one 64-bit rank key: the high word is the
// score's fp32 bits mapped to an order-preserving unsigned integer (-0 taken
// as +0), the low word the complement of the expert id, so the largest key is
// the largest score and, among equal scores, the lowest id.  k rounds each
// take the wave's largest key (DPP within 16-lane rows, then four readlanes),
// and the owning lane retires it.  Lane j keeps the j-th winner; the weights
// are formed in fp64 and rounded once to fp32.
#include "device.h"
#include "internal.h"

namespace bfp8 {

namespace {

constexpr int kRouterThreads = 256;
constexpr int kTokensPerWG = kRouterThreads / 64;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return (uint64_t)dpp_u32<CTRL>((uint32_t)v) | ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  return __builtin_bit_cast(double, dpp_u64<CTRL>(__builtin_bit_cast(uint64_t, v)));
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
  uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return (uint64_t)lo | ((uint64_t)hi << 32);
}

// Largest key of the wave, wave-uniform.  Every lane must be active.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint64_t o;
  o = dpp_u64<0xB1>(v);  v = o > v ? o : v;   // quad_perm 1,0,3,2
  o = dpp_u64<0x4E>(v);  v = o > v ? o : v;   // quad_perm 2,3,0,1
  o = dpp_u64<0x141>(v); v = o > v ? o : v;   // row_half_mirror
  o = dpp_u64<0x140>(v); v = o > v ? o : v;   // row_mirror: row maximum in every lane
  uint64_t a = readlane_u64(v, 0), b = readlane_u64(v, 16);
  uint64_t c = readlane_u64(v, 32), d = readlane_u64(v, 48);
  a = b > a ? b : a;
  c = d > c ? d : c;
  return c > a ? c : a;
}

// Sum of the wave's fp64 values, wave-uniform (fixed tree: deterministic).
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  v += dpp_f64<0x141>(v);
  v += dpp_f64<0x140>(v);
  double r0 = __builtin_bit_cast(double, readlane_u64(__builtin_bit_cast(uint64_t, v), 0));
  double r1 = __builtin_bit_cast(double, readlane_u64(__builtin_bit_cast(uint64_t, v), 16));
  double r2 = __builtin_bit_cast(double, readlane_u64(__builtin_bit_cast(uint64_t, v), 32));
  double r3 = __builtin_bit_cast(double, readlane_u64(__builtin_bit_cast(uint64_t, v), 48));
  return (r0 + r1) + (r2 + r3);
}

// fp32 bits -> unsigned integer with the same order as the floats (NaN aside);
// -0 is mapped like +0 so that the two compare equal, as floats do.
__device__ __forceinline__ uint32_t order_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float sigmoid_rn(float x) { return (float)(1.0 / (1.0 + exp(-(double)x))); }

template <int NPL>
__global__ __launch_bounds__(kRouterThreads) void router_topk_kernel(const float* __restrict__ logits, int64_t M,
                                                                     int E, int k, int score_fn,
                                                                     const float* __restrict__ bias, int renorm,
                                                                     double scale, int32_t* __restrict__ ids,
                                                                     float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kTokensPerWG + (threadIdx.x >> 6);
  if (t >= M) return;  // whole waves only: the reductions below need all 64 lanes
  const float* lg = logits + t * (int64_t)E;

  float v[NPL];
  uint64_t key[NPL];
#pragma unroll
  for (int i = 0; i < NPL; i++) {
    const int e = lane + 64 * i;
    v[i] = e < E ? lg[e] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < NPL; i++) {
    const int e = lane + 64 * i;
    float s = v[i];
    if (score_fn == kScoreSigmoid) {
      s = sigmoid_rn(v[i]);
      if (bias) s = s + (e < E ? bias[e] : 0.0f);
    }
    key[i] = e < E ? ((uint64_t)order_bits(s) << 32) | (uint64_t)(~(uint32_t)e) : 0ull;
  }

  // k rounds of "take the largest remaining key"; lane j keeps winner j
  int my_id = 0;
  float my_logit = 0.0f;
  for (int j = 0; j < k; j++) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < NPL; i++) best = key[i] > best ? key[i] : best;
    const uint64_t win = wave_max_u64(best);
    const int e = (int)(~(uint32_t)win);
    float lv = v[0];
#pragma unroll
    for (int i = 0; i < NPL; i++) {
      if (key[i] == win) key[i] = 0ull;  // retired: below every live key
      if (i == (e >> 6)) lv = v[i];
    }
    lv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lv), e & 63));
    if (lane == j) {
      my_id = e;
      my_logit = lv;
    }
  }

  // weights in fp64
  const bool chosen = lane < k;
  double num = 0.0, z = 1.0;
  if (score_fn == kScoreSoftmax) {
    double m = (double)__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_logit), 0));
    num = chosen ? exp((double)my_logit - m) : 0.0;
    if (renorm) {
      z = wave_sum_f64(num);
    } else {
      double part = 0.0;
#pragma unroll
      for (int i = 0; i < NPL; i++)
        if (lane + 64 * i < E) part += exp((double)v[i] - m);
      z = wave_sum_f64(part);
    }
  } else {
    num = chosen ? 1.0 / (1.0 + exp(-(double)my_logit)) : 0.0;
    z = renorm ? wave_sum_f64(num) : 1.0;
  }
  if (chosen) {
    ids[t * k + lane] = my_id;
    w[t * k + lane] = (float)(num / z * scale);
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
