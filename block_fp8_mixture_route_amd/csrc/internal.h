// internal.h -- launchers shared by the C-ABI layer (api.hip) and the kernel
// files.  Every launcher enqueues on `stream` and returns the launch status;
// argument checking is done by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bfp8 {

// The experts of this device, as the layer and route preparation see them:
// either the contiguous slice [offset, offset + L) of the global ids, or an
// expert map from global id to local expert (map[id] for id in [0, E); a
// value outside [0, L) marks a remote expert).
struct ExpertSel {
  const int32_t* map = nullptr;  // device, [E]; null: the slice
  int32_t E = 0;                 // global expert count (map form)
  int32_t offset = 0;            // first global id of the slice (slice form)
  int32_t L = 0;                 // local experts
};

// The local expert global id `id` selects, or -1 when it is not local.
__device__ __forceinline__ int local_of(const ExpertSel& s, int32_t id) {
  if (s.map) {
    if (id < 0 || id >= s.E) return -1;
    const int32_t m = s.map[id];
    return (m >= 0 && m < s.L) ? m : -1;
  }
  const int64_t e = (int64_t)id - s.offset;
  return (e >= 0 && e < s.L) ? (int)e : -1;
}

// Which rows of an act+quant call are processed.
enum RowFilterMode : int {
  kRowsAll = 0,    // every row
  kRowsIds = 1,    // ids[r] in [0, E)
  kRowsIdsMap = 2, // ids[r] in [0, E) and map[ids[r]] >= 0
  kRowsLocal = 3   // local_of(sel, ids[r]) >= 0
};

// Optional profiling hook: records caller-owned HIP events on the stream
// before stage i (and, with i == number of stages, after the last one), and
// can restrict a call to one stage.
struct LaunchHook {
  void* const* events = nullptr;
  int n = 0;      // number of events in the array
  int only = -1;  // >= 0: launch stage `only` alone
  void before(int i, hipStream_t stream) const {
    if (events && i < n && events[i]) (void)hipEventRecord(static_cast<hipEvent_t>(events[i]), stream);
  }
  bool run(int i) const { return only < 0 || only == i; }
};

struct RowFilter {
  const int32_t* ids = nullptr;
  const int32_t* map = nullptr;  // kRowsIdsMap
  int32_t E = 0;                 // kRowsIds, kRowsIdsMap
  ExpertSel sel;                 // kRowsLocal
  int mode = kRowsAll;
};

__device__ __forceinline__ bool row_live(const RowFilter& f, int64_t r) {
  if (f.mode == kRowsAll) return true;
  const int32_t id = f.ids[r];
  if (f.mode == kRowsLocal) return local_of(f.sel, id) >= 0;
  if (id < 0 || id >= f.E) return false;
  return f.mode != kRowsIdsMap || f.map[id] >= 0;
}

hipError_t launch_quant_fp8(const uint16_t* x, int64_t rows, int K, int fmt, uint8_t* q, float* s,
                            hipStream_t stream);
hipError_t launch_silu_and_mul(const uint16_t* gu, int64_t rows, int I, float limit, uint16_t* out,
                               hipStream_t stream);
hipError_t launch_silu_and_mul_quant(const uint16_t* gu, int64_t rows, int I, const RowFilter& f, float limit,
                                     int fmt, uint8_t* q, float* s, hipStream_t stream);
// The same over a row list: rows list[i] for i < *count (count on the device,
// at most n_list), e.g. route preparation's sorted routes and kept count.
hipError_t launch_silu_and_mul_quant_list(const uint16_t* gu, const int32_t* list, const int32_t* count,
                                          int64_t n_list, int I, float limit, int fmt, uint8_t* q, float* s,
                                          hipStream_t stream);
// Router scoring functions (values of the C ABI's score_fn).
enum RouterScore : int { kScoreSoftmax = 0, kScoreSigmoid = 1 };

// A router folded into the first kernel of a layer path: the kernel ranks the
// token's logits itself and writes the routing to ids / w for the kernels
// after it.
struct RouterArgs {
  const float* logits;  // [M, E] fp32
  const float* bias;    // [E] fp32 selection bias or null (sigmoid scoring)
  int32_t* ids;         // [M, k] out
  float* w;             // [M, k] out
  double scale;
  int E;
  int score_fn;
  int renorm;
  int n_group;     // > 1: group-limited (noaux-TC) selection, sigmoid scoring
  int topk_group;
};
// Largest expert count the folded router handles (four experts per lane).
constexpr int kFoldedRouterMaxE = 256;
// Most tokens for which the layer folds the router in: one wave of every
// gate/up workgroup ranks its token before the weight loads, and that delay
// grows with the ranks to walk (measured at the 7168 x 256 decode shape:
// folded against the router's launch then the layer, 15.3 against 17.7 us at
// 1 token, 42.4 against 44.0 at 4, 74.4 against 73.9 at 8, 104.2 against
// 100.9 at 12).
constexpr int64_t kFoldedRouterMaxM = 4;

hipError_t launch_router_topk(const float* logits, int64_t M, int E, int k, int score_fn, const float* bias,
                              int renorm, double scale, int32_t* ids, float* w, hipStream_t stream);
// Group-limited noaux-TC routing (sigmoid scores; n_group <= 1 is the
// single-group sigmoid router).
hipError_t launch_router_noaux_tc(const float* logits, int64_t M, int E, int k, int n_group, int topk_group,
                                  const float* bias, int renorm, double scale, int32_t* ids, float* w,
                                  hipStream_t stream);

// ids null: every route counts; otherwise only routes local under sel.
hipError_t launch_moe_reduce(const uint16_t* y, const float* w, const int32_t* ids, const ExpertSel& sel, int64_t M,
                             int k, int H, uint16_t* out, hipStream_t stream);

// Route preparation.  Picks the single-workgroup kernel when `single` is true,
// otherwise count -> scan+scatter over `route_prep_num_segments(R)` workgroups
// with a workspace of route_prep_ws_bytes(R, L) bytes.
bool route_prep_single_fits(int64_t R, int32_t L);
// Input quantisation that the first launch of route preparation can carry
// (quant_fp8 of x [rows, K] into q, s), so that the layer makes one launch
// fewer.  Possible unless the single-workgroup path serves more than 512
// experts.
struct QuantArgs {
  const uint16_t* x;
  int64_t rows;
  int K;
  int fmt;
  uint8_t* q;
  float* s;
};
bool route_prep_can_quant(bool single, int32_t L);
int route_prep_num_segments(int64_t R);
size_t route_prep_ws_bytes(int64_t R, int32_t L);
// Route preparation can also make the routing itself: with `route`, the
// single workgroup first ranks the R / k tokens' router logits (one wave per
// token, as the router kernel), writes route->ids / route->w and sorts those
// ids (`ids` is then not read).  Up to kRoutePrepRouterMaxM tokens,
// kFoldedRouterMaxE experts and kRoutePrepRouterMaxL local experts, on the
// single-workgroup path.
constexpr int64_t kRoutePrepRouterMaxM = 64;
constexpr int32_t kRoutePrepRouterMaxL = 512;
bool route_prep_can_route(int64_t M, int32_t E, int32_t L, int64_t R);
hipError_t launch_route_prepare(const int32_t* ids, int64_t R, const ExpertSel& sel, int32_t block_m,
                                int32_t* sorted_routes, int32_t* expert_offsets, int32_t* block_expert,
                                int32_t* block_start, int64_t max_blocks, int32_t* num_blocks, bool single,
                                void* ws, hipStream_t stream, const QuantArgs* quant = nullptr,
                                const RouterArgs* route = nullptr, int k = 0);

// Grouped block-FP8 GEMM over compact blocks (general path).
hipError_t launch_grouped_gemm(const uint8_t* A, const float* As, int a_row_div, const uint8_t* B,
                               const float* Bs, int N, int K, const int32_t* sorted_routes,
                               const int32_t* expert_offsets, const int32_t* block_expert,
                               const int32_t* block_start, const int32_t* num_blocks, int64_t max_blocks,
                               int block_m, uint16_t* C, hipStream_t stream, bool channel = false);

// MXFP4-weight grouped GEMM: B [L, N, K/2] packed E2M1 with E8M0 scale bytes
// Bs [L, N, K/32]; A and As as launch_grouped_gemm.  K a multiple of 256.
hipError_t launch_grouped_gemm_mxfp4(const uint8_t* A, const float* As, int a_row_div, const uint8_t* B,
                                     const uint8_t* Bs, int N, int K, const int32_t* sorted_routes,
                                     const int32_t* expert_offsets, const int32_t* block_expert,
                                     const int32_t* block_start, const int32_t* num_blocks, int64_t max_blocks,
                                     int block_m, uint16_t* C, hipStream_t stream);

// W8A8 variant: one scale per activation row (dynamic: amax / 448 of the row
// in fmt; static_scale > 0: that scale for every row).  Rows of up to 8192.
bool rows_quant_fits(int K);
hipError_t launch_quant_fp8_rows(const uint16_t* x, int64_t rows, int K, int fmt, float static_scale, uint8_t* q,
                                 float* s, hipStream_t stream);
hipError_t launch_silu_and_mul_quant_rows(const uint16_t* gu, int64_t rows, int I, const RowFilter& f, float limit,
                                          int fmt, float static_scale, uint8_t* q, float* s, hipStream_t stream);

// Small-batch path of the fused layer: gate/up + SwiGLU kernel, then down +
// moe_reduce kernel.  act: [M*k, I] BF16 scratch.
bool decode_path_fits(int64_t M, int H, int k, int I);
// Few-token path: gate/up + SwiGLU kernel per route, then down + moe_reduce
// kernel per token, both matrix-vector streaming kernels (each route reads its
// expert's rows).  act: [M*k, I] BF16 scratch.
// wfmt: the weight format, as the C ABI's weight_scale_mode (block-FP8 and
// W8A8: I 128, 256 or 512; MXFP4: H % 256 == 0 and I 256 or 512).
bool token_path_fits(int64_t M, int H, int k, int I, int wfmt = 0);
int device_cu_count();  // of the current device; 0 when there is none
// Fault bits of the bounded in-kernel waits on the current device (bit 0: the
// few-token gate/up kernel's wait for its hidden row ran out); optionally
// cleared.  Synchronous.
hipError_t read_wait_faults(unsigned* flags, bool clear);
// w13_s / w2_s as wfmt says: fp32 block scales; fp32 scales per row [L, 2I]
// and [L, H] (W8A8, with a1_static / a2_static > 0 the static activation
// scales of the hidden and SwiGLU rows, else per-row dynamic ones); or E8M0
// bytes [L, 2I, H/32] and [L, H, I/32] (MXFP4: w13 / w2 packed E2M1, [L, 2I,
// H/2] and [L, H, I/2]).
hipError_t launch_token_layer(const uint16_t* hidden, int64_t M, int H, const int32_t* ids, const float* topk_w,
                              int k, const ExpertSel& sel, const uint8_t* w13, const void* w13_s,
                              const uint8_t* w2, const void* w2_s, int I, int fmt, float limit, uint16_t* act,
                              uint16_t* out, hipStream_t stream, const LaunchHook* hook,
                              const RouterArgs* route = nullptr, int wfmt = 0, float a1_static = 0.0f,
                              float a2_static = 0.0f);
hipError_t launch_decode_layer(const uint16_t* hidden, int64_t M, int H, const int32_t* ids, const float* topk_w,
                               int k, const ExpertSel& sel, const uint8_t* w13, const float* w13_s,
                               const uint8_t* w2, const float* w2_s, int I, int fmt, float limit, uint16_t* act,
                               uint16_t* out, hipStream_t stream, const LaunchHook* hook);

// The read-bandwidth probe (stream_probe.hip): pattern 0 contiguous 512 KiB
// slabs, 1 GEMM-shaped 128-row tiles of row_bytes with `piece` bytes per row
// per load, 2 the same with each workgroup's walk along K rotated; lds_bytes
// of unused dynamic LDS per workgroup.  Workgroups of a
// launch: stream_probe_grid.
int64_t stream_probe_grid(size_t bytes, int pattern, int row_bytes);
hipError_t launch_stream_probe(const uint8_t* buf, size_t bytes, int pattern, int row_bytes, int piece,
                               int lds_bytes, uint32_t* sink, hipStream_t stream);

}  // namespace bfp8
