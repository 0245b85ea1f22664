// router.h -- wave-level pieces of the top-k routers, shared by the router
// kernel and the few-token layer kernel that routes for itself.
//
// [P2 Changes: a fused single-group top-k router; renormalize option]
// [P2 Reviewed changes: route_noaux_tc.py, group-limited noaux-TC routing]
//   [P2] lmdeploy PR "perf(pytorch): optimize compact blocked FP8 MoE and route
//        preparation"
//
// One wave routes one token.  Lane l holds experts l, l + 64, ... (NPL of
// them).  With groups (noaux-TC), the keys of experts outside the chosen
// groups are retired before the sort: each lane g < n_group scores group g
// (the fp32 sum of its two largest keys, read from LDS), and topk_group
// rounds of wave maxima pick the groups (the lowest index among equal scores).
// Each expert's score becomes an order-preserving unsigned integer (-0 taken
// as +0); each lane sorts its keys once.  Each round takes the
// largest of the lanes' heads (DPP-fused maxima within 16-lane rows, row
// broadcasts across them, one readlane); a ballot finds the lane holding it
// (a minimum over expert ids settles equal heads), and that lane pops it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace bfp8 {
namespace router {

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROWS, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint64_t r = (uint64_t)dpp_u32<CTRL>(0u, (uint32_t)u) | ((uint64_t)dpp_u32<CTRL>(0u, (uint32_t)(u >> 32)) << 32);
  return __builtin_bit_cast(double, r);
}

// Largest value of the wave, wave-uniform.  Every lane must be active.  The
// row maximum by DPP (quad swaps, half-row and row mirrors: every lane of a
// row ends with it), then the row broadcasts carry rows 0-2 into row 3, whose
// lane 63 is read.  Rows a broadcast does not write keep their own value.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(0u, v));   // quad_perm 1,0,3,2
  v = max(v, dpp_u32<0x4E>(0u, v));   // quad_perm 2,3,0,1
  v = max(v, dpp_u32<0x141>(0u, v));  // row_half_mirror
  v = max(v, dpp_u32<0x140>(0u, v));  // row_mirror
  v = max(v, dpp_u32<0x142, 0xA>(v, v));  // row_bcast15: row 0 -> 1, row 2 -> 3
  v = max(v, dpp_u32<0x143, 0xC>(v, v));  // row_bcast31: row 1 -> 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Smallest value of the wave, wave-uniform; as wave_max_u32.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<0xB1>(0u, v));
  v = min(v, dpp_u32<0x4E>(0u, v));
  v = min(v, dpp_u32<0x141>(0u, v));
  v = min(v, dpp_u32<0x140>(0u, v));
  v = min(v, dpp_u32<0x142, 0xA>(v, v));
  v = min(v, dpp_u32<0x143, 0xC>(v, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Sum of the wave's fp64 values, wave-uniform (fixed tree: deterministic).
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  v += dpp_f64<0x141>(v);
  v += dpp_f64<0x140>(v);
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  double r[4];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 16 * q);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 16 * q);
    r[q] = __builtin_bit_cast(double, (uint64_t)lo | ((uint64_t)hi << 32));
  }
  return (r[0] + r[1]) + (r[2] + r[3]);
}

// fp32 bits -> unsigned integer with the same order as the floats; -0 is
// mapped like +0 so that the two compare equal, as floats do.  Live keys are
// at least 1 (only a NaN could map lower), so 0 marks a retired or absent
// expert.
__device__ __forceinline__ uint32_t order_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return max((u & 0x80000000u) ? ~u : (u | 0x80000000u), 1u);
}

__device__ __forceinline__ float sigmoid_rn(float x) { return (float)(1.0 / (1.0 + exp(-(double)x))); }

// (a1, a2), a1 >= a2, becomes the two largest of {a1, a2, b1, b2} (b1 >= b2);
// equal values count twice, as two experts with equal keys do.
__device__ __forceinline__ void top2_merge(float& a1, float& a2, float b1, float b2) {
  const float n2 = fmaxf(fminf(a1, b1), fmaxf(a2, b2));
  a1 = fmaxf(a1, b1);
  a2 = n2;
}

// A token's logits and keys, loaded by one wave.  Loads are unconditional
// (indexes clamped into the row); absent experts get key 0.
template <int NPL>
struct WaveRoute {
  float v[NPL];       // logits in expert order (lane + 64 i)
  uint32_t key[NPL];  // the lane's keys, sorted largest first; key[0] is its head
  int id[NPL];        // expert id of each sorted key
  float sv[NPL];      // logit of each sorted key

  // n_group > 1: keep only the experts of the topk_group best groups of
  // E / n_group consecutive experts (n_group <= 64); s_key: n_group + E floats
  // of LDS private to this wave.
  __device__ __forceinline__ void load(const float* lg, int E, int score_fn, const float* bias, int lane,
                                       int n_group = 1, int topk_group = 1, float* s_key = nullptr) {
    float b[NPL], sc[NPL];
#pragma unroll
    for (int i = 0; i < NPL; i++) v[i] = lg[min(lane + 64 * i, E - 1)];
    if (score_fn == kScoreSigmoid && bias) {
#pragma unroll
      for (int i = 0; i < NPL; i++) b[i] = bias[min(lane + 64 * i, E - 1)];
    }
#pragma unroll
    for (int i = 0; i < NPL; i++) {
      float s = v[i];
      if (score_fn == kScoreSigmoid) {
        s = sigmoid_rn(v[i]);
        if (bias) s = s + b[i];
      }
      sc[i] = s;
      key[i] = lane + 64 * i < E ? order_bits(s) : 0u;
      id[i] = lane + 64 * i;
      sv[i] = v[i];
    }
    if (n_group > 1) {
      const int gs = E / n_group;
      uint32_t gkey = 0u;
      if ((gs & (gs - 1)) == 0 && gs < 64) {
        // groups within 64 lanes: a top-2 butterfly over each aligned run of
        // gs lanes, slot by slot; the run's first lane stores the score
#pragma unroll
        for (int i = 0; i < NPL; i++) {
          float a1 = lane + 64 * i < E ? sc[i] : -__builtin_inff(), a2 = -__builtin_inff();
          for (int d = 1; d < gs; d <<= 1) top2_merge(a1, a2, __shfl_xor(a1, d), __shfl_xor(a2, d));
          if ((lane & (gs - 1)) == 0 && lane + 64 * i < E) s_key[(lane + 64 * i) / gs] = gs > 1 ? a1 + a2 : a1;
        }
      } else if (gs % 64 == 0) {
        // groups of whole slots: each lane's top-2 over the group's slots,
        // then a butterfly over the wave
        for (int g = 0; g < n_group; g++) {
          float a1 = -__builtin_inff(), a2 = -__builtin_inff();
#pragma unroll
          for (int i = 0; i < NPL; i++)
            if (64 * i >= g * gs && 64 * i < (g + 1) * gs) top2_merge(a1, a2, sc[i], -__builtin_inff());
          for (int d = 1; d < 64; d <<= 1) top2_merge(a1, a2, __shfl_xor(a1, d), __shfl_xor(a2, d));
          if (lane == 0) s_key[g] = a1 + a2;
        }
      } else {
        // other group widths: lane g scans group g's keys
#pragma unroll
        for (int i = 0; i < NPL; i++)
          if (lane + 64 * i < E) s_key[n_group + lane + 64 * i] = sc[i];
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's LDS writes are done
        if (lane < n_group) {
          float a1 = -__builtin_inff(), a2 = -__builtin_inff();
          for (int e = lane * gs; e < (lane + 1) * gs; e++) top2_merge(a1, a2, s_key[n_group + e], -__builtin_inff());
          s_key[lane] = gs > 1 ? a1 + a2 : a1;
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the group scores are in LDS
      if (lane < n_group) gkey = order_bits(s_key[lane]);
      uint64_t chosen = 0;
      for (int j = 0; j < topk_group; j++) {
        const uint32_t top = wave_max_u32(gkey);
        const int wl = (int)__builtin_ctzll(__ballot(gkey == top));  // lowest group among equal scores
        chosen |= 1ull << wl;
        if (lane == wl) gkey = 0u;
      }
#pragma unroll
      for (int i = 0; i < NPL; i++)
        if (lane + 64 * i < E && !((chosen >> ((lane + 64 * i) / gs)) & 1ull)) key[i] = 0u;
    }
    // odd-even transposition sort, largest first; a swap only on a strictly
    // smaller key keeps equal keys in ascending id order
#pragma unroll
    for (int r = 0; r < NPL; r++) {
#pragma unroll
      for (int i = r & 1; i + 1 < NPL; i += 2) {
        if (key[i] < key[i + 1]) {
          const uint32_t tk = key[i];
          key[i] = key[i + 1];
          key[i + 1] = tk;
          const int ti = id[i];
          id[i] = id[i + 1];
          id[i + 1] = ti;
          const float tv = sv[i];
          sv[i] = sv[i + 1];
          sv[i + 1] = tv;
        }
      }
    }
  }

  // One round: the largest remaining key (lowest expert id among equals) is
  // retired; returns its expert id and logit, wave-uniform.  Needs a live key.
  // Each lane's head is its largest key and, among its equal keys, the lowest
  // id, so the winner is the head equal to the wave maximum with the lowest
  // id: one lane in the usual case, a second reduction when heads tie.
  __device__ __forceinline__ int take(int lane, float& logit) {
    const uint32_t top = wave_max_u32(key[0]);
    const uint64_t hit = __ballot(key[0] == top);
    int wl;
    if (__popcll(hit) == 1) {
      wl = (int)__builtin_ctzll(hit);
    } else {
      const uint32_t lowest = wave_min_u32(key[0] == top ? (uint32_t)id[0] : 0xFFFFFFFFu);
      wl = (int)(lowest & 63u);  // expert l + 64 i lives in lane l
    }
    const int e = __builtin_amdgcn_readlane(id[0], wl);
    logit = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sv[0]), wl));
    if (lane == wl) {  // pop the head
#pragma unroll
      for (int i = 0; i + 1 < NPL; i++) {
        key[i] = key[i + 1];
        id[i] = id[i + 1];
        sv[i] = sv[i + 1];
      }
      key[NPL - 1] = 0u;
    }
    return e;
  }

  // Weight of the expert lane j < k chose (my_logit), fp64 rounded once to
  // fp32; lanes j >= k get 0.  All 64 lanes must call it.
  __device__ __forceinline__ float weight(float my_logit, int lane, int E, int k, int score_fn, int renorm,
                                          double scale) const {
    const bool chosen = lane < k;
    double num = 0.0, z = 1.0;
    if (score_fn == kScoreSoftmax) {
      const double m =
          (double)__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_logit), 0));
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
    return (float)(num / z * scale);
  }
};

}  // namespace router
}  // namespace bfp8
