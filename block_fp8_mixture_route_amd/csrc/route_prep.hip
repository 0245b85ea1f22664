// route_prep.hip -- route preparation for gfx950: top-k routes sorted by local
// expert (stable) plus compact per-expert blocks of block_m routes, emitted
// only for experts that receive routes.
//
// [P2 Changes] one workgroup handles small problems end to end; larger ones
// run a count pass over many workgroups, then a scan + scatter pass.
// [P2 Suppressed comments] the slice [expert_offset, expert_offset + L) is
// validated on the host before anything runs.
// [P3 Purpose] the local experts can also be given by an expert map from
// global to local ids (remote experts marked negative).
// [P1 Modification, Active-expert block scheduling] blocks exist only for
// experts with routes.
// [P2 Changes: the fused single-group top-k router feeds the layer] for a few
// tokens the single workgroup can rank the tokens itself first (one wave per
// token, the router kernel's wave code), so that the router and route
// preparation are one launch; the counting sort then reads the ids from LDS.
//
// Determinism and stability without atomics on positions: every segment of
// routes is split into 16 contiguous wave sub-segments; each wave counts its
// sub-segment into its own LDS histogram; an exclusive scan over
// (expert, segment, wave) gives every wave a private cursor per expert; each
// wave then walks its sub-segment 64 routes at a time in route order, ranks
// equal experts inside the chunk with ballots, and advances its cursors.  The
// result equals a stable counting sort.
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
#include "router.h"

namespace bfp8 {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxL = 2048;
constexpr int64_t kSingleMaxRoutes = 4096;
// Largest expert count whose single-workgroup launch also carries the input
// quantisation: its quantisation workgroups get the same dynamic LDS as the
// route-prep workgroup, (16 + 3) L + 64 ints, 38 KB at 512.
constexpr int32_t kQuantMaxL = 512;

// Exclusive scan of v[0..n) in LDS by the whole 1024-thread workgroup.
// Returns the total.  tmp: 32 ints of LDS.  Ends with a barrier.
__device__ int block_exclusive_scan(int* v, int n, int* tmp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (n + kThreads - 1) / kThreads;  // consecutive items per thread
  const int b = tid * per;
  int local = 0;
  for (int i = 0; i < per; i++)
    if (b + i < n) local += v[b + i];
  // inclusive scan of `local` across the wave
  int x = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int s = lane < kWaves ? tmp[lane] : 0;
    int t = s;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      int y = __shfl_up(t, d);
      if (lane >= d) t += y;
    }
    if (lane < kWaves) tmp[lane] = t - s;  // exclusive wave offsets
    if (lane == kWaves - 1) tmp[kWaves] = t;
  }
  __syncthreads();
  int run = tmp[wave] + x - local;  // exclusive prefix of this thread
  for (int i = 0; i < per; i++) {
    if (b + i < n) {
      int c = v[b + i];
      v[b + i] = run;
      run += c;
    }
  }
  int total = tmp[kWaves];
  __syncthreads();
  return total;
}

// The optional input quantisation carried by the first launch of route
// preparation (one launch fewer in the layer): workgroups n_main and up each
// quantise 64 groups of 128 of x (same arithmetic as quant_fp8).
struct QuantJob {
  const uint16_t* x = nullptr;  // nullptr: no quantisation workgroups
  int64_t n_groups = 0;
  int fmt = 0;
  uint8_t* q = nullptr;
  float* s = nullptr;
};
constexpr int kQuantGroupsPerWG = kThreads / 16;

__device__ __forceinline__ bool quant_job(const QuantJob& qj, int n_main) {
  if (qj.x == nullptr || (int)blockIdx.x < n_main) return false;
  const int64_t gid = (int64_t)(blockIdx.x - n_main) * kQuantGroupsPerWG + (threadIdx.x >> 4);
  if (gid < qj.n_groups) quant_group8(qj.x, gid, threadIdx.x & 15, qj.fmt, qj.q, qj.s);
  return true;
}

inline unsigned quant_wgs(const QuantJob& qj) {
  return qj.x ? (unsigned)((qj.n_groups + kQuantGroupsPerWG - 1) / kQuantGroupsPerWG) : 0u;
}

// Count pass of the multi-workgroup path: hist[seg][e] for each segment.
__global__ __launch_bounds__(kThreads) void route_count_kernel(const int32_t* __restrict__ ids, int64_t R,
                                                               ExpertSel sel, int64_t seg_len,
                                                               int32_t* __restrict__ hist, int n_main, QuantJob qj) {
  if (quant_job(qj, n_main)) return;
  const int32_t L = sel.L;
  extern __shared__ int lds[];
  int* h = lds;
  for (int e = threadIdx.x; e < L; e += kThreads) h[e] = 0;
  __syncthreads();
  const int64_t s0 = (int64_t)blockIdx.x * seg_len;
  const int64_t s1 = s0 + seg_len < R ? s0 + seg_len : R;
  for (int64_t r = s0 + threadIdx.x; r < s1; r += kThreads) {
    const int e = local_of(sel, ids[r]);
    if (e >= 0) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < L; e += kThreads) hist[(size_t)blockIdx.x * L + e] = h[e];
}

// Scan + scatter.  With n_seg == 1 and hist == nullptr this is the whole
// single-workgroup route preparation.  Workgroup 0 also writes the offsets,
// the blocks and the -1 fills.  kRoute (single workgroup only): the routes'
// expert ids are not read from `ids` but made here first from the router
// logits of the R / k tokens (ra), written to ra.ids / ra.w for the kernels
// after this one and kept in LDS for the sort.
template <bool kRoute>
__global__ __launch_bounds__(kThreads) void route_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t R, ExpertSel sel, int32_t block_m, int64_t seg_len,
    const int32_t* __restrict__ hist, int n_seg, int32_t* __restrict__ sorted_routes,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ block_expert, int32_t* __restrict__ block_start,
    int64_t max_blocks, int32_t* __restrict__ num_blocks, QuantJob qj, RouterArgs ra, int k) {
  if (quant_job(qj, n_seg)) return;
  const int32_t L = sel.L;
  extern __shared__ int lds[];
  int* wh = lds;                       // [kWaves][L] wave histograms -> cursors
  int* offs = wh + kWaves * L;         // [L] expert totals -> exclusive offsets
  int* base = offs + L;                // [L] routes of this expert in earlier segments
  int* cnt = base + L;                 // [L] expert totals (kept)
  int* tmp = cnt + L;                  // [64] scan scratch
  int* s_ids = tmp + 64;               // kRoute: [R] the routes' expert ids
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seg = blockIdx.x;

  if constexpr (kRoute) {
    // 0. the router: wave w ranks tokens w, w + 16, ... (all 64 lanes of a
    //    wave take part in every round), lane j < k keeping winner j
    float* s_key = reinterpret_cast<float*>(s_ids + R) + (size_t)wave * (64 + ra.E);  // grouped selection only
    const int64_t M = R / k;
    for (int64_t t = wave; t < M; t += kWaves) {
      router::WaveRoute<kFoldedRouterMaxE / 64> rt;
      rt.load(ra.logits + t * ra.E, ra.E, ra.score_fn, ra.bias, lane, ra.n_group, ra.topk_group, s_key);
      int my_id = 0;
      float my_logit = 0.0f;
      for (int j = 0; j < k; j++) {
        float lv;
        const int e = rt.take(lane, lv);
        if (lane == j) {
          my_id = e;
          my_logit = lv;
        }
      }
      const float wt = rt.weight(my_logit, lane, ra.E, k, ra.score_fn, ra.renorm, ra.scale);
      if (lane < k) {
        ra.ids[t * k + lane] = my_id;
        ra.w[t * k + lane] = wt;
        s_ids[t * k + lane] = my_id;
      }
    }
  }
  // a route's expert id: made above (kRoute) or given
  auto id_of = [&](int64_t r) -> int32_t {
    if constexpr (kRoute)
      return s_ids[r];
    else
      return ids[r];
  };

  for (int i = tid; i < kWaves * L; i += kThreads) wh[i] = 0;
  __syncthreads();

  const int64_t s0 = (int64_t)seg * seg_len;
  const int64_t s1 = s0 + seg_len < R ? s0 + seg_len : R;
  const int64_t n = s1 > s0 ? s1 - s0 : 0;
  const int64_t sub = ((n + kWaves - 1) / kWaves + 63) / 64 * 64;  // wave sub-segment, whole chunks
  const int64_t w0 = s0 + wave * sub;
  const int64_t w1 = w0 + sub < s1 ? w0 + sub : s1;

  // 1. wave histograms
  for (int64_t r = w0 + lane; r < w1; r += 64) {
    const int e = local_of(sel, id_of(r));
    if (e >= 0) atomicAdd(&wh[wave * L + e], 1);
  }
  __syncthreads();

  // 2. per expert: exclusive over waves; totals over all segments (the
  //    segment counts are read 8 at a time, every load of a batch issued
  //    before the first is used)
  for (int e = tid; e < L; e += kThreads) {
    int cw[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; w++) cw[w] = wh[w * L + e];
    int run = 0;
#pragma unroll
    for (int w = 0; w < kWaves; w++) {
      wh[w * L + e] = run;
      run += cw[w];
    }
    int before = 0, total = run;
    if (hist) {
      total = 0;
      for (int b0 = 0; b0 < n_seg; b0 += 8) {
        int c[8];
#pragma unroll
        for (int u = 0; u < 8; u++) c[u] = hist[(size_t)min(b0 + u, n_seg - 1) * L + e];
#pragma unroll
        for (int u = 0; u < 8; u++) {
          const int cu = b0 + u < n_seg ? c[u] : 0;
          if (b0 + u < seg) before += cu;
          total += cu;
        }
      }
    }
    base[e] = before;
    cnt[e] = total;
    offs[e] = total;
  }
  __syncthreads();
  const int n_kept = block_exclusive_scan(offs, L, tmp);

  for (int i = tid; i < kWaves * L; i += kThreads) {
    int e = i % L;
    wh[i] += offs[e] + base[e];
  }
  __syncthreads();

  // 3. in-order scatter, 64 routes per step per wave
  int nbits = 0;
  while ((1 << nbits) < L) nbits++;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t c0 = w0; c0 < w1; c0 += 64) {
    const int64_t r = c0 + lane;
    int e = r < w1 ? local_of(sel, id_of(r)) : -1;
    uint64_t same = __ballot(e >= 0);
    for (int bit = 0; bit < nbits; bit++) {
      uint64_t m = __ballot(e >= 0 && ((e >> bit) & 1));
      same &= ((e >> bit) & 1) ? m : ~m;
    }
    if (e >= 0) {
      int rank = __popcll(same & below);
      int p = wh[wave * L + e];
      sorted_routes[p + rank] = (int32_t)r;
      if (rank == 0) wh[wave * L + e] = p + __popcll(same);
    }
  }

  if (seg != 0) return;

  // 4. offsets, blocks and fills (workgroup 0 only)
  for (int e = tid; e < L; e += kThreads) expert_offsets[e] = offs[e];
  if (tid == 0) expert_offsets[L] = n_kept;
  for (int64_t i = n_kept + tid; i < R; i += kThreads) sorted_routes[i] = -1;
  __syncthreads();
  for (int e = tid; e < L; e += kThreads) base[e] = (cnt[e] + block_m - 1) / block_m;
  __syncthreads();
  const int nb = block_exclusive_scan(base, L, tmp);
  if (block_expert) {
    for (int e = tid; e < L; e += kThreads) {
      const int nbe = (cnt[e] + block_m - 1) / block_m;
      for (int i = 0; i < nbe; i++) {
        block_expert[base[e] + i] = e;
        block_start[base[e] + i] = offs[e] + i * block_m;
      }
    }
    for (int64_t i = nb + tid; i < max_blocks; i += kThreads) {
      block_expert[i] = -1;
      block_start[i] = -1;
    }
  }
  if (tid == 0) *num_blocks = nb;
}

size_t scatter_lds_bytes(int32_t L) { return sizeof(int) * ((size_t)(kWaves + 3) * L + 64); }

// With the router folded in: the routes' ids, and each wave's group scores
// and keys when the selection is grouped.
size_t routed_lds_bytes(int32_t L, int64_t R, int E, bool grouped) {
  return scatter_lds_bytes(L) + sizeof(int) * (size_t)R + (grouped ? sizeof(float) * (size_t)kWaves * (64 + E) : 0);
}

}  // namespace

bool route_prep_single_fits(int64_t R, int32_t L) { return R <= kSingleMaxRoutes && L <= kMaxL; }

int route_prep_num_segments(int64_t R) {
  int64_t seg = 1024;
  while ((R + seg - 1) / seg > 64) seg *= 2;
  int64_t n = (R + seg - 1) / seg;
  return n < 1 ? 1 : (int)n;
}

static int64_t segment_length(int64_t R) {
  int n = route_prep_num_segments(R);
  return R == 0 ? 1 : (R + n - 1) / n;
}

size_t route_prep_ws_bytes(int64_t R, int32_t L) {
  return sizeof(int32_t) * (size_t)route_prep_num_segments(R) * (size_t)L;
}

bool route_prep_can_quant(bool single, int32_t L) { return !single || L <= kQuantMaxL; }

bool route_prep_can_route(int64_t M, int32_t E, int32_t L, int64_t R) {
  return M >= 1 && M <= kRoutePrepRouterMaxM && E >= 1 && E <= kFoldedRouterMaxE && L <= kRoutePrepRouterMaxL &&
         route_prep_single_fits(R, L);
}

hipError_t launch_route_prepare(const int32_t* ids, int64_t R, const ExpertSel& sel, int32_t block_m,
                                int32_t* sorted_routes, int32_t* expert_offsets, int32_t* block_expert,
                                int32_t* block_start, int64_t max_blocks, int32_t* num_blocks, bool single,
                                void* ws, hipStream_t stream, const QuantArgs* quant, const RouterArgs* route,
                                int k) {
  const int32_t L = sel.L;
  if (route && (!single || k < 1 || R % k != 0 || !route_prep_can_route(R / k, route->E, L, R)))
    return hipErrorInvalidValue;  // the caller checks
  QuantJob qj;
  if (quant && quant->rows > 0) {
    if (!route_prep_can_quant(single, L)) return hipErrorInvalidValue;  // the caller checks
    qj.x = quant->x;
    qj.n_groups = quant->rows * (quant->K / kGroup);
    qj.fmt = quant->fmt;
    qj.q = quant->q;
    qj.s = quant->s;
  }
  const unsigned nq = quant_wgs(qj);
  // Large expert counts need more than 64 KB of LDS in one workgroup
  // (gfx950 allows up to 160 KB); raise the function's limit once.
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute((const void*)route_scatter_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)scatter_lds_bytes(kMaxL));
    (void)hipFuncSetAttribute((const void*)route_scatter_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)routed_lds_bytes(kRoutePrepRouterMaxL, kSingleMaxRoutes, kFoldedRouterMaxE, true));
    (void)hipGetLastError();
  });
  if (route) {
    const size_t lds = routed_lds_bytes(L, R, route->E, route->n_group > 1);
    hipLaunchKernelGGL(route_scatter_kernel<true>, dim3(1 + nq), dim3(kThreads), lds, stream, ids, R, sel, block_m,
                       R > 0 ? R : (int64_t)1, (const int32_t*)nullptr, 1, sorted_routes, expert_offsets,
                       block_expert, block_start, max_blocks, num_blocks, qj, *route, k);
    return hipGetLastError();
  }
  const size_t lds = scatter_lds_bytes(L);
  if (single) {
    hipLaunchKernelGGL(route_scatter_kernel<false>, dim3(1 + nq), dim3(kThreads), lds, stream, ids, R, sel, block_m,
                       R > 0 ? R : (int64_t)1, (const int32_t*)nullptr, 1, sorted_routes, expert_offsets,
                       block_expert, block_start, max_blocks, num_blocks, qj, RouterArgs{}, 0);
    return hipGetLastError();
  }
  const int n_seg = route_prep_num_segments(R);
  const int64_t seg_len = segment_length(R);
  int32_t* hist = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(route_count_kernel, dim3(n_seg + nq), dim3(kThreads), sizeof(int) * (size_t)L, stream, ids, R,
                     sel, seg_len, hist, n_seg, qj);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_scatter_kernel<false>, dim3(n_seg), dim3(kThreads), lds, stream, ids, R, sel, block_m,
                     seg_len, (const int32_t*)hist, n_seg, sorted_routes, expert_offsets, block_expert,
                     block_start, max_blocks, num_blocks, QuantJob(), RouterArgs{}, 0);
  return hipGetLastError();
}

}  // namespace bfp8
