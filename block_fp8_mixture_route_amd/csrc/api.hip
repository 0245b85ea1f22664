// api.hip -- the C ABI declared in include/bfp8moe.h.  Host code: validates
// arguments before anything is enqueued, lays out workspaces, picks kernels
// by shape and launches them on the caller's stream.  Never allocates device
// memory, never synchronises, never reads device data (except the debugging
// query bfp8moe_wait_faults).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "../../include/bfp8moe.h"
#include "internal.h"

namespace {

thread_local std::string g_last_error;

bfp8moe_status_t fail(bfp8moe_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bfp8moe_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return BFP8MOE_OK;
  return fail(BFP8MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define REQUIRE(cond, ...)                                        \
  do {                                                            \
    if (!(cond)) return fail(BFP8MOE_ERR_INVALID_ARG, __VA_ARGS__); \
  } while (0)

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Workspace carving for the fused layer.
struct LayerPlan {
  int64_t M, R;
  int32_t H, I, k, E, L, offset, block_m, fmt;
  const int32_t* map;  // expert map (device, [E]) or null: the slice [offset, offset + L)
  float clamp;
  int64_t max_blocks;
  bool route_single;
  bool rq_fused;  // general path: route preparation carries the input quantisation
  bool channel;   // the W8A8 variant: per-row activation and per-channel weight scales
  bool mxfp4;     // MXFP4 weights (E2M1 with E8M0 scales per 32 along K)
  float a1_static, a2_static;
  int mode;  // kModeGeneral, kModeDecode, kModeToken
  size_t off_aq, off_as, off_sorted, off_eoff, off_bexp, off_bstart, off_nb, off_rws, off_h13, off_q, off_s,
      off_y, off_act, total;
};

const char* const kGeneralStages[] = {"route_prepare", "quant_fp8", "gate_up_gemm",
                                      "silu_and_mul_quant", "down_gemm", "moe_reduce"};
// General path whose route preparation also quantises the input (one launch
// fewer): stage 0 covers both.
const char* const kGeneralFusedStages[] = {"route_prepare_quant", "gate_up_gemm", "silu_and_mul_quant", "down_gemm",
                                           "moe_reduce"};
const char* const kMxfp4Stages[] = {"route_prepare", "quant_fp8", "gate_up_gemm_mxfp4", "silu_and_mul_quant",
                                    "down_gemm_mxfp4", "moe_reduce"};
const char* const kMxfp4FusedStages[] = {"route_prepare_quant", "gate_up_gemm_mxfp4", "silu_and_mul_quant",
                                         "down_gemm_mxfp4", "moe_reduce"};
const char* const kChannelStages[] = {"route_prepare", "quant_fp8_rows", "gate_up_gemm_channel",
                                      "silu_and_mul_quant_rows", "down_gemm_channel", "moe_reduce"};
const char* const kDecodeStages[] = {"decode_gate_up_swiglu", "decode_down_reduce"};
const char* const kTokenStages[] = {"token_gate_up_swiglu", "token_down_reduce"};
const char* const kTokenMxfp4Stages[] = {"token_gate_up_swiglu_mxfp4", "token_down_reduce_mxfp4"};
const char* const kTokenChannelStages[] = {"token_gate_up_swiglu_channel", "token_down_reduce_channel"};
enum { kModeGeneral = 0, kModeDecode = 1, kModeToken = 2 };

// The few-token path is the default up to this many tokens: it reads one
// expert's weights once per route, the general path once per expert.  At the
// decode shape (256 experts, top-8, H 7168, I 256, uniform routing) with
// block scales, the few-token path leads at 15 tokens (120.8 against 122.9 µs)
// and the general path at 16 (125.3 against 127.1).  With per-channel (W8A8)
// weights the bound stays where it was measured before the general path's
// GEMM staged its scales: 12.  The small-batch path is the default up to
// kDecodeAutoMaxM tokens where the few-token path does not fit.
constexpr int64_t kTokenAutoMaxM = 15;
constexpr int64_t kTokenAutoMaxMChannel = 12;
constexpr int64_t kDecodeAutoMaxM = 4;
// With MXFP4 weights the few-token kernels do as much vector work per
// element as with E4M3 rows while the general path's FP4 MFMA halves its
// weight bytes: measured at the decode shape, the two paths are even at 8
// tokens (66.1 against 65.2 µs) and the general path leads from 12.
constexpr int64_t kTokenAutoMaxMMxfp4 = 8;

// Routes per compact block of the general path, from the routes per local
// expert on average: 16 below 8; then 32, and 64 from 32 routes per expert
// (MXFP4 weights: above 48).  Measured: 16 beat 32 at 0.5, 1 and 4 routes
// per expert (16 and 32 decode-shape tokens, 128 small-shape tokens), 32 beat
// 16 at 16 and 32 (512 small-shape tokens, 2048 large-shape tokens); with the
// GEMM's scales staged in LDS, 64 beat 32 at 32 routes per expert for block
// FP8 and W8A8 weights (2048 large-shape tokens: 1,443 against 1,478 us) and
// lost at 16 (512 small-shape tokens), and the MXFP4 GEMM lost at 64 in all.
int auto_block_m(int64_t R, int32_t L, int32_t weight_scale_mode) {
  const int64_t per_expert = R / (L > 0 ? L : 1);
  const int64_t to64 = weight_scale_mode == BFP8MOE_WEIGHT_MXFP4 ? 49 : 32;
  return per_expert < 8 ? 16 : per_expert < to64 ? 32 : 64;
}

void plan_layer(LayerPlan& p, int64_t M, int32_t H, int32_t k, int32_t E, int32_t I, const bfp8moe_opts_t& o) {
  p.M = M;
  p.H = H;
  p.I = I;
  p.k = k;
  p.E = E;
  p.R = M * k;
  p.L = o.local_num_experts > 0 ? o.local_num_experts : E;
  p.offset = o.expert_offset;
  p.map = o.expert_map;
  p.fmt = o.scale_fmt;
  p.clamp = o.clamp_limit;
  p.block_m = o.block_m > 0 ? o.block_m : auto_block_m(p.R, p.L, o.weight_scale_mode);
  p.max_blocks = bfp8moe_max_blocks(p.R, p.L, p.block_m);
  p.channel = o.weight_scale_mode == BFP8MOE_WEIGHT_SCALE_CHANNEL;
  p.mxfp4 = o.weight_scale_mode == BFP8MOE_WEIGHT_MXFP4;
  p.a1_static = o.act_static_scale;
  p.a2_static = o.inter_static_scale;
  const bool block = !p.channel && !p.mxfp4;  // the small-batch path takes block scales only
  const bool fits = block && bfp8::decode_path_fits(M, H, k, I);
  const bool token_fits = bfp8::token_path_fits(M, H, k, I, o.weight_scale_mode);
  if (o.flags & BFP8MOE_FLAG_LAYER_GENERAL)
    p.mode = kModeGeneral;
  else if (o.flags & BFP8MOE_FLAG_LAYER_DECODE)
    p.mode = fits ? kModeDecode : kModeGeneral;
  else if (o.flags & BFP8MOE_FLAG_LAYER_TOKEN)
    p.mode = token_fits ? kModeToken : kModeGeneral;
  else if (token_fits && M <= (p.mxfp4 ? kTokenAutoMaxMMxfp4 : p.channel ? kTokenAutoMaxMChannel : kTokenAutoMaxM))
    p.mode = kModeToken;
  else
    p.mode = (fits && M <= kDecodeAutoMaxM) ? kModeDecode : kModeGeneral;
  if (o.flags & BFP8MOE_FLAG_ROUTE_SINGLE_WG)
    p.route_single = true;
  else if (o.flags & BFP8MOE_FLAG_ROUTE_MULTI_WG)
    p.route_single = false;
  else
    p.route_single = bfp8::route_prep_single_fits(p.R, p.L);
  p.rq_fused = !p.channel && bfp8::route_prep_can_quant(p.route_single, p.L);
  size_t o_ = 0;
  auto take = [&](size_t bytes) {
    size_t at = o_;
    o_ = align_up(o_ + bytes);
    return at;
  };
  if (p.mode == kModeToken || p.mode == kModeDecode) {
    p.off_act = take(sizeof(uint16_t) * (size_t)p.R * I);
    p.total = o_;
    return;
  }
  p.off_act = 0;
  p.off_aq = take((size_t)M * H);
  p.off_as = take(sizeof(float) * (size_t)M * (p.channel ? 1 : H / 128));
  p.off_sorted = take(sizeof(int32_t) * (size_t)p.R);
  p.off_eoff = take(sizeof(int32_t) * ((size_t)p.L + 1));
  p.off_bexp = take(sizeof(int32_t) * (size_t)p.max_blocks);
  p.off_bstart = take(sizeof(int32_t) * (size_t)p.max_blocks);
  p.off_nb = take(sizeof(int32_t));
  p.off_rws = take(p.route_single ? 0 : bfp8::route_prep_ws_bytes(p.R, p.L));
  p.off_h13 = take(sizeof(uint16_t) * (size_t)p.R * 2 * I);
  p.off_q = take((size_t)p.R * I);
  p.off_s = take(sizeof(float) * (size_t)p.R * (p.channel ? 1 : I / 128));
  p.off_y = take(sizeof(uint16_t) * (size_t)p.R * H);
  p.total = o_;
}

bfp8::ExpertSel layer_sel(const LayerPlan& p) {
  bfp8::ExpertSel sel;
  sel.map = p.map;
  sel.E = p.E;
  sel.offset = p.offset;
  sel.L = p.L;
  return sel;
}

int plan_stages(const LayerPlan& p) { return p.mode == kModeGeneral ? (p.rq_fused ? 5 : 6) : 2; }

bool valid_fmt(int32_t f) { return f == BFP8MOE_SCALE_FP32 || f == BFP8MOE_SCALE_UE8M0; }

// Route preparation under either form of the local expert set (checks, then
// the launch).
bfp8moe_status_t route_prepare_sel(const int32_t* topk_ids, int64_t R, const bfp8::ExpertSel& sel, int32_t block_m,
                                   int32_t* sorted_routes, int32_t* expert_offsets, int32_t* block_expert,
                                   int32_t* block_start, int64_t max_blocks, int32_t* num_blocks, void* ws,
                                   size_t ws_bytes, uint32_t flags, void* stream) {
  REQUIRE(R >= 0 && R <= 0x7FFFFFFF, "R=%lld out of range [0, 2^31)", (long long)R);
  const int32_t L = sel.L;
  REQUIRE(L >= 1, "local_num_experts=%d must be >= 1", L);
  REQUIRE(block_m >= 1, "block_m=%d must be >= 1", block_m);
  REQUIRE(R == 0 || (topk_ids && sorted_routes), "topk_ids and sorted_routes must be non-null");
  REQUIRE(expert_offsets && num_blocks, "expert_offsets and num_blocks must be non-null");
  REQUIRE((block_expert == nullptr) == (block_start == nullptr),
          "block_expert and block_start must both be given or both be null");
  const int64_t need_blocks = bfp8moe_max_blocks(R, L, block_m);
  REQUIRE(block_expert == nullptr || max_blocks >= need_blocks, "max_blocks=%lld < required %lld",
          (long long)max_blocks, (long long)need_blocks);
  if (L > 2048) return fail(BFP8MOE_ERR_UNSUPPORTED, "local_num_experts=%d above 2048", L);
  const bool single = (flags & BFP8MOE_FLAG_ROUTE_SINGLE_WG)  ? true
                      : (flags & BFP8MOE_FLAG_ROUTE_MULTI_WG) ? false
                                                               : bfp8::route_prep_single_fits(R, L);
  const size_t need = single ? 0 : bfp8::route_prep_ws_bytes(R, L);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(BFP8MOE_ERR_WORKSPACE, "route workspace %zu bytes < required %zu", ws_bytes, need);
  return hip_status(bfp8::launch_route_prepare(topk_ids, R, sel, block_m, sorted_routes, expert_offsets,
                                               block_expert, block_start, block_expert ? max_blocks : 0, num_blocks,
                                               single, ws, (hipStream_t)stream),
                    "moe_route_prepare");
}

// moe_reduce under either form of the local expert set.
bfp8moe_status_t reduce_sel(const uint16_t* y, const float* topk_w, const int32_t* topk_ids,
                            const bfp8::ExpertSel& sel, int64_t M, int32_t k, int32_t H, uint16_t* out,
                            void* stream) {
  REQUIRE(M >= 0 && k >= 1, "M=%lld k=%d invalid", (long long)M, k);
  REQUIRE(H > 0 && H % 8 == 0, "H=%d must be a positive multiple of 8", H);
  REQUIRE(M == 0 || (y && topk_w && out), "y, topk_w and out must be non-null");
  REQUIRE(aligned16(y) && aligned16(out), "y and out must be 16-byte aligned");
  return hip_status(bfp8::launch_moe_reduce(y, topk_w, topk_ids, sel, M, k, H, out, (hipStream_t)stream),
                    "moe_reduce");
}

}  // namespace

extern "C" {

void bfp8moe_opts_init(bfp8moe_opts_t* opts) {
  if (!opts) return;
  opts->block_m = 0;
  opts->scale_fmt = BFP8MOE_SCALE_FP32;
  opts->clamp_limit = INFINITY;
  opts->expert_offset = 0;
  opts->local_num_experts = 0;
  opts->expert_map = nullptr;
  opts->flags = 0;
  opts->stage_events = nullptr;
  opts->weight_scale_mode = BFP8MOE_WEIGHT_SCALE_BLOCK;
  opts->act_static_scale = 0.0f;
  opts->inter_static_scale = 0.0f;
}

const char* bfp8moe_status_string(int status) {
  switch (status) {
    case BFP8MOE_OK: return "ok";
    case BFP8MOE_ERR_INVALID_ARG: return "invalid argument";
    case BFP8MOE_ERR_UNSUPPORTED: return "unsupported shape";
    case BFP8MOE_ERR_WORKSPACE: return "workspace too small";
    case BFP8MOE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

const char* bfp8moe_last_error(void) { return g_last_error.c_str(); }

bfp8moe_status_t bfp8moe_wait_faults(uint32_t* flags, int clear) {
  REQUIRE(flags != nullptr, "flags must be non-null");
  unsigned f = 0;
  const hipError_t e = bfp8::read_wait_faults(&f, clear != 0);
  if (e != hipSuccess) return hip_status(e, "bfp8moe_wait_faults");
  *flags = f;
  return BFP8MOE_OK;
}

bfp8moe_status_t bfp8moe_stream_probe(const uint8_t* buf, size_t bytes, int32_t pattern, int32_t row_bytes,
                                      int32_t piece, int32_t lds_bytes, uint32_t* sink, int64_t sink_len,
                                      void* stream) {
  REQUIRE(buf != nullptr && sink != nullptr, "buf and sink must be non-null");
  REQUIRE(aligned16(buf), "buf must be 16-byte aligned");
  REQUIRE(pattern >= 0 && pattern <= 2, "pattern=%d must be 0 (contiguous), 1 (tile) or 2 (tile, rotated)",
          pattern);
  if (pattern != 0) {
    REQUIRE(piece == 128 || piece == 256 || piece == 1024, "piece=%d must be 128, 256 or 1024", piece);
    REQUIRE(row_bytes >= 1024 && row_bytes % 1024 == 0 && row_bytes % piece == 0,
            "row_bytes=%d must be a positive multiple of 1024 and of piece", row_bytes);
  }
  REQUIRE(lds_bytes >= 0 && lds_bytes <= 163840, "lds_bytes=%d out of [0, 163840]", lds_bytes);
  const int64_t grid = bfp8::stream_probe_grid(bytes, pattern, row_bytes);
  REQUIRE(grid >= 1 && grid <= 0x7FFFFFFF, "%zu bytes give %lld workgroups", bytes, (long long)grid);
  REQUIRE(sink_len >= grid, "sink holds %lld words for %lld workgroups", (long long)sink_len, (long long)grid);
  return hip_status(bfp8::launch_stream_probe(buf, bytes, pattern, row_bytes, piece, lds_bytes, sink,
                                              (hipStream_t)stream),
                    "bfp8moe_stream_probe");
}

int64_t bfp8moe_max_blocks(int64_t R, int32_t L, int32_t block_m) {
  if (R <= 0 || L <= 0 || block_m <= 0) return 0;
  const int64_t d = R < L ? R : L;
  return (R + d * (block_m - 1)) / block_m;
}

size_t moe_route_prepare_workspace_size(int64_t R, int32_t L, uint32_t flags) {
  if (R < 0 || L <= 0) return 0;
  bool single = (flags & BFP8MOE_FLAG_ROUTE_SINGLE_WG)  ? true
                : (flags & BFP8MOE_FLAG_ROUTE_MULTI_WG) ? false
                                                         : bfp8::route_prep_single_fits(R, L);
  return single ? 0 : bfp8::route_prep_ws_bytes(R, L);
}

bfp8moe_status_t moe_route_prepare(const int32_t* topk_ids, int64_t R, int32_t expert_offset, int32_t L,
                                   int32_t block_m, int32_t* sorted_routes, int32_t* expert_offsets,
                                   int32_t* block_expert, int32_t* block_start, int64_t max_blocks,
                                   int32_t* num_blocks, void* ws, size_t ws_bytes, uint32_t flags,
                                   void* stream) {
  REQUIRE(expert_offset >= 0, "expert_offset=%d must be >= 0", expert_offset);
  bfp8::ExpertSel sel;
  sel.offset = expert_offset;
  sel.L = L;
  return route_prepare_sel(topk_ids, R, sel, block_m, sorted_routes, expert_offsets, block_expert, block_start,
                           max_blocks, num_blocks, ws, ws_bytes, flags, stream);
}

bfp8moe_status_t moe_route_prepare_map(const int32_t* topk_ids, int64_t R, const int32_t* expert_map,
                                       int32_t num_experts, int32_t L, int32_t block_m, int32_t* sorted_routes,
                                       int32_t* expert_offsets, int32_t* block_expert, int32_t* block_start,
                                       int64_t max_blocks, int32_t* num_blocks, void* ws, size_t ws_bytes,
                                       uint32_t flags, void* stream) {
  REQUIRE(expert_map != nullptr, "expert_map must be non-null");
  REQUIRE(num_experts >= 1, "num_experts=%d must be >= 1", num_experts);
  bfp8::ExpertSel sel;
  sel.map = expert_map;
  sel.E = num_experts;
  sel.L = L;
  return route_prepare_sel(topk_ids, R, sel, block_m, sorted_routes, expert_offsets, block_expert, block_start,
                           max_blocks, num_blocks, ws, ws_bytes, flags, stream);
}

bfp8moe_status_t quant_fp8(const uint16_t* x, int64_t rows, int32_t K, int32_t scale_fmt, uint8_t* q,
                           float* scales, void* stream) {
  REQUIRE(rows >= 0, "rows=%lld must be >= 0", (long long)rows);
  REQUIRE(K > 0 && K % 128 == 0, "K=%d must be a positive multiple of 128", K);
  REQUIRE(valid_fmt(scale_fmt), "scale_fmt=%d is not 0 (fp32) or 1 (ue8m0)", scale_fmt);
  REQUIRE(rows == 0 || (x && q && scales), "x, q and scales must be non-null");
  REQUIRE(aligned16(x) && aligned16(q), "x and q must be 16-byte aligned");
  return hip_status(bfp8::launch_quant_fp8(x, rows, K, scale_fmt, q, scales, (hipStream_t)stream), "quant_fp8");
}

bfp8moe_status_t silu_and_mul(const uint16_t* gate_up, int64_t rows, int32_t I, float clamp_limit, uint16_t* out,
                              void* stream) {
  REQUIRE(rows >= 0, "rows=%lld must be >= 0", (long long)rows);
  REQUIRE(I > 0 && I % 128 == 0, "I=%d must be a positive multiple of 128", I);
  REQUIRE(!isnan(clamp_limit) && clamp_limit > 0, "clamp_limit must be positive (+inf = unclamped)");
  REQUIRE(rows == 0 || (gate_up && out), "gate_up and out must be non-null");
  REQUIRE(aligned16(gate_up) && aligned16(out), "gate_up and out must be 16-byte aligned");
  return hip_status(bfp8::launch_silu_and_mul(gate_up, rows, I, clamp_limit, out, (hipStream_t)stream),
                    "silu_and_mul");
}

bfp8moe_status_t silu_and_mul_quant_fp8(const uint16_t* gate_up, int64_t rows, int32_t I,
                                        const int32_t* row_expert_ids, const int32_t* expert_map, int32_t E,
                                        float clamp_limit, int32_t scale_fmt, uint8_t* q, float* scales,
                                        void* stream) {
  REQUIRE(rows >= 0, "rows=%lld must be >= 0", (long long)rows);
  REQUIRE(I > 0 && I % 128 == 0, "I=%d must be a positive multiple of 128", I);
  REQUIRE(valid_fmt(scale_fmt), "scale_fmt=%d is not 0 (fp32) or 1 (ue8m0)", scale_fmt);
  REQUIRE(!isnan(clamp_limit) && clamp_limit > 0, "clamp_limit must be positive (+inf = unclamped)");
  REQUIRE(rows == 0 || (gate_up && q && scales), "gate_up, q and scales must be non-null");
  REQUIRE(expert_map == nullptr || row_expert_ids != nullptr, "expert_map requires row_expert_ids");
  REQUIRE(row_expert_ids == nullptr || E >= 1, "E=%d must be >= 1 when row_expert_ids is given", E);
  REQUIRE(aligned16(gate_up) && aligned16(q), "gate_up and q must be 16-byte aligned");
  bfp8::RowFilter f;
  f.ids = row_expert_ids;
  f.map = expert_map;
  f.E = E;
  f.mode = row_expert_ids == nullptr ? bfp8::kRowsAll : (expert_map ? bfp8::kRowsIdsMap : bfp8::kRowsIds);
  return hip_status(bfp8::launch_silu_and_mul_quant(gate_up, rows, I, f, clamp_limit, scale_fmt, q, scales,
                                                    (hipStream_t)stream),
                    "silu_and_mul_quant_fp8");
}

bfp8moe_status_t moe_fp8_grouped_gemm(const uint8_t* A, const float* A_scale, int32_t a_row_div,
                                      const uint8_t* B, const float* B_scale, int32_t L, int32_t N, int32_t K,
                                      const int32_t* sorted_routes, const int32_t* expert_offsets,
                                      const int32_t* block_expert, const int32_t* block_start,
                                      const int32_t* num_blocks, int64_t max_blocks, int32_t block_m,
                                      int64_t R, uint16_t* C, void* stream) {
  REQUIRE(N > 0 && N % 128 == 0, "N=%d must be a positive multiple of 128", N);
  REQUIRE(K > 0 && K % 128 == 0, "K=%d must be a positive multiple of 128", K);
  REQUIRE(L >= 1, "L=%d must be >= 1", L);
  REQUIRE(a_row_div >= 1, "a_row_div=%d must be >= 1", a_row_div);
  REQUIRE(block_m == 16 || block_m == 32 || block_m == 64, "block_m=%d must be 16, 32 or 64", block_m);
  REQUIRE(R >= 0 && R <= 0x7FFFFFFF, "R=%lld out of range", (long long)R);
  REQUIRE(max_blocks >= 0, "max_blocks must be >= 0");
  REQUIRE(max_blocks == 0 || (A && A_scale && B && B_scale && sorted_routes && expert_offsets && block_expert &&
                              block_start && num_blocks && C),
          "all pointers must be non-null");
  REQUIRE(aligned16(A) && aligned16(B) && aligned16(C), "A, B and C must be 16-byte aligned");
  return hip_status(bfp8::launch_grouped_gemm(A, A_scale, a_row_div, B, B_scale, N, K, sorted_routes,
                                              expert_offsets, block_expert, block_start, num_blocks, max_blocks,
                                              block_m, C, (hipStream_t)stream),
                    "moe_fp8_grouped_gemm");
}

bfp8moe_status_t quant_fp8_rows(const uint16_t* x, int64_t rows, int32_t K, int32_t scale_fmt, float static_scale,
                                uint8_t* q, float* scales, void* stream) {
  REQUIRE(rows >= 0 && rows <= 0x7FFFFFFF, "rows=%lld out of range", (long long)rows);
  REQUIRE(bfp8::rows_quant_fits(K), "K=%d must be a positive multiple of 128 up to 8192", K);
  REQUIRE(valid_fmt(scale_fmt), "scale_fmt=%d is not 0 (fp32) or 1 (ue8m0)", scale_fmt);
  REQUIRE(isfinite(static_scale) && static_scale >= 0, "static_scale must be finite and >= 0 (0 = dynamic)");
  REQUIRE(rows == 0 || (x && q && scales), "x, q and scales must be non-null");
  REQUIRE(aligned16(x) && aligned16(q), "x and q must be 16-byte aligned");
  return hip_status(bfp8::launch_quant_fp8_rows(x, rows, K, scale_fmt, static_scale, q, scales, (hipStream_t)stream),
                    "quant_fp8_rows");
}

bfp8moe_status_t silu_and_mul_quant_fp8_rows(const uint16_t* gate_up, int64_t rows, int32_t I,
                                             const int32_t* row_expert_ids, const int32_t* expert_map, int32_t E,
                                             float clamp_limit, int32_t scale_fmt, float static_scale, uint8_t* q,
                                             float* scales, void* stream) {
  REQUIRE(rows >= 0 && rows <= 0x7FFFFFFF, "rows=%lld out of range", (long long)rows);
  REQUIRE(bfp8::rows_quant_fits(I), "I=%d must be a positive multiple of 128 up to 8192", I);
  REQUIRE(valid_fmt(scale_fmt), "scale_fmt=%d is not 0 (fp32) or 1 (ue8m0)", scale_fmt);
  REQUIRE(!isnan(clamp_limit) && clamp_limit > 0, "clamp_limit must be positive (+inf = unclamped)");
  REQUIRE(isfinite(static_scale) && static_scale >= 0, "static_scale must be finite and >= 0 (0 = dynamic)");
  REQUIRE(rows == 0 || (gate_up && q && scales), "gate_up, q and scales must be non-null");
  REQUIRE(expert_map == nullptr || row_expert_ids != nullptr, "expert_map requires row_expert_ids");
  REQUIRE(row_expert_ids == nullptr || E >= 1, "E=%d must be >= 1 when row_expert_ids is given", E);
  REQUIRE(aligned16(gate_up) && aligned16(q), "gate_up and q must be 16-byte aligned");
  bfp8::RowFilter f;
  f.ids = row_expert_ids;
  f.map = expert_map;
  f.E = E;
  f.mode = row_expert_ids == nullptr ? bfp8::kRowsAll : (expert_map ? bfp8::kRowsIdsMap : bfp8::kRowsIds);
  return hip_status(bfp8::launch_silu_and_mul_quant_rows(gate_up, rows, I, f, clamp_limit, scale_fmt, static_scale, q,
                                                         scales, (hipStream_t)stream),
                    "silu_and_mul_quant_fp8_rows");
}

bfp8moe_status_t moe_fp8_grouped_gemm_channel(const uint8_t* A, const float* A_scale, int32_t a_row_div,
                                              const uint8_t* B, const float* B_scale, int32_t L, int32_t N,
                                              int32_t K, const int32_t* sorted_routes,
                                              const int32_t* expert_offsets, const int32_t* block_expert,
                                              const int32_t* block_start, const int32_t* num_blocks,
                                              int64_t max_blocks, int32_t block_m, int64_t R, uint16_t* C,
                                              void* stream) {
  REQUIRE(N > 0 && N % 128 == 0, "N=%d must be a positive multiple of 128", N);
  REQUIRE(K > 0 && K % 128 == 0, "K=%d must be a positive multiple of 128", K);
  REQUIRE(L >= 1, "L=%d must be >= 1", L);
  REQUIRE(a_row_div >= 1, "a_row_div=%d must be >= 1", a_row_div);
  REQUIRE(block_m == 16 || block_m == 32 || block_m == 64, "block_m=%d must be 16, 32 or 64", block_m);
  REQUIRE(R >= 0 && R <= 0x7FFFFFFF, "R=%lld out of range", (long long)R);
  REQUIRE(max_blocks >= 0, "max_blocks must be >= 0");
  REQUIRE(max_blocks == 0 || (A && A_scale && B && B_scale && sorted_routes && expert_offsets && block_expert &&
                              block_start && num_blocks && C),
          "all pointers must be non-null");
  REQUIRE(aligned16(A) && aligned16(B) && aligned16(C) && aligned16(B_scale),
          "A, B, B_scale and C must be 16-byte aligned");
  return hip_status(bfp8::launch_grouped_gemm(A, A_scale, a_row_div, B, B_scale, N, K, sorted_routes,
                                              expert_offsets, block_expert, block_start, num_blocks, max_blocks,
                                              block_m, C, (hipStream_t)stream, true),
                    "moe_fp8_grouped_gemm_channel");
}

bfp8moe_status_t moe_reduce(const uint16_t* y, const float* topk_w, const int32_t* topk_ids, int32_t expert_offset,
                            int32_t L, int64_t M, int32_t k, int32_t H, uint16_t* out, void* stream) {
  REQUIRE(topk_ids == nullptr || (L >= 1 && expert_offset >= 0), "invalid expert slice");
  bfp8::ExpertSel sel;
  sel.offset = expert_offset;
  sel.L = L;
  return reduce_sel(y, topk_w, topk_ids, sel, M, k, H, out, stream);
}

bfp8moe_status_t moe_reduce_map(const uint16_t* y, const float* topk_w, const int32_t* topk_ids,
                                const int32_t* expert_map, int32_t num_experts, int32_t L, int64_t M, int32_t k,
                                int32_t H, uint16_t* out, void* stream) {
  REQUIRE(topk_ids && expert_map, "topk_ids and expert_map must be non-null");
  REQUIRE(num_experts >= 1 && L >= 1, "num_experts=%d and L=%d must be >= 1", num_experts, L);
  bfp8::ExpertSel sel;
  sel.map = expert_map;
  sel.E = num_experts;
  sel.L = L;
  return reduce_sel(y, topk_w, topk_ids, sel, M, k, H, out, stream);
}

bfp8moe_status_t moe_router_topk(const float* logits, int64_t M, int32_t E, int32_t k, int32_t score_fn,
                                 const float* bias, int32_t renormalize, double scale, int32_t* topk_ids,
                                 float* topk_w, void* stream) {
  // four tokens per workgroup and a 32-bit grid
  REQUIRE(M >= 0 && M <= 4 * (int64_t)0x7FFFFFFF, "M=%lld out of range", (long long)M);
  REQUIRE(E >= 1 && E <= 1024, "E=%d must be in [1, 1024]", E);
  REQUIRE(k >= 1 && k <= 64 && k <= E, "k=%d must be in [1, min(E, 64)]", k);
  REQUIRE(score_fn == BFP8MOE_SCORE_SOFTMAX || score_fn == BFP8MOE_SCORE_SIGMOID, "score_fn=%d invalid", score_fn);
  REQUIRE(bias == nullptr || score_fn == BFP8MOE_SCORE_SIGMOID, "a selection bias needs sigmoid scoring");
  REQUIRE(isfinite(scale), "scale must be finite");
  REQUIRE(M == 0 || (logits && topk_ids && topk_w), "logits, topk_ids and topk_w must be non-null");
  return hip_status(bfp8::launch_router_topk(logits, M, E, k, score_fn, bias, renormalize != 0, scale, topk_ids,
                                             topk_w, (hipStream_t)stream),
                    "moe_router_topk");
}

bfp8moe_status_t moe_router_noaux_tc(const float* logits, int64_t M, int32_t E, int32_t k, int32_t n_group,
                                     int32_t topk_group, const float* bias, int32_t renormalize, double scale,
                                     int32_t* topk_ids, float* topk_w, void* stream) {
  REQUIRE(M >= 0 && M <= 4 * (int64_t)0x7FFFFFFF, "M=%lld out of range", (long long)M);
  REQUIRE(E >= 1 && E <= 1024, "E=%d must be in [1, 1024]", E);
  REQUIRE(n_group >= 1 && n_group <= 64 && E % n_group == 0, "n_group=%d must divide E=%d and be in [1, 64]",
          n_group, E);
  REQUIRE(topk_group >= 1 && topk_group <= n_group, "topk_group=%d must be in [1, n_group=%d]", topk_group, n_group);
  REQUIRE(k >= 1 && k <= 64 && (int64_t)k <= (int64_t)topk_group * (E / n_group),
          "k=%d must be in [1, min(64, topk_group * E / n_group)]", k);
  REQUIRE(isfinite(scale), "scale must be finite");
  REQUIRE(M == 0 || (logits && topk_ids && topk_w), "logits, topk_ids and topk_w must be non-null");
  return hip_status(bfp8::launch_router_noaux_tc(logits, M, E, k, n_group, topk_group, bias, renormalize != 0, scale,
                                                 topk_ids, topk_w, (hipStream_t)stream),
                    "moe_router_noaux_tc");
}

}  // extern "C"

namespace {

bfp8moe_status_t check_layer_shape(int64_t M, int32_t H, int32_t k, int32_t E, int32_t I, const bfp8moe_opts_t& o) {
  REQUIRE(M >= 0 && M * (int64_t)(k > 0 ? k : 1) <= 0x7FFFFFFF, "M=%lld out of range", (long long)M);
  REQUIRE(k >= 1, "k=%d must be >= 1", k);
  REQUIRE(E >= 1, "E=%d must be >= 1", E);
  REQUIRE(H > 0 && H % 128 == 0, "H=%d must be a positive multiple of 128", H);
  REQUIRE(I > 0 && I % 128 == 0, "I=%d must be a positive multiple of 128", I);
  REQUIRE(valid_fmt(o.scale_fmt), "scale_fmt=%d is not 0 (fp32) or 1 (ue8m0)", o.scale_fmt);
  REQUIRE(!isnan(o.clamp_limit) && o.clamp_limit > 0, "clamp_limit must be positive (+inf = unclamped)");
  const int32_t L = o.local_num_experts > 0 ? o.local_num_experts : E;
  REQUIRE(o.local_num_experts >= 0 && o.expert_offset >= 0 && (int64_t)o.expert_offset + L <= E,
          "expert slice [%d, %d + %d) is not inside [0, %d)", o.expert_offset, o.expert_offset, L, E);
  REQUIRE(o.expert_map == nullptr || o.expert_offset == 0, "expert_map and expert_offset are exclusive");
  REQUIRE(o.block_m == 0 || o.block_m == 16 || o.block_m == 32 || o.block_m == 64,
          "block_m=%d must be 0, 16, 32 or 64", o.block_m);
  REQUIRE((o.flags & (BFP8MOE_FLAG_ROUTE_SINGLE_WG | BFP8MOE_FLAG_ROUTE_MULTI_WG)) !=
              (BFP8MOE_FLAG_ROUTE_SINGLE_WG | BFP8MOE_FLAG_ROUTE_MULTI_WG),
          "route flags are exclusive");
  if (L > 2048) return fail(BFP8MOE_ERR_UNSUPPORTED, "local_num_experts=%d above 2048", L);
  REQUIRE(o.weight_scale_mode == BFP8MOE_WEIGHT_SCALE_BLOCK || o.weight_scale_mode == BFP8MOE_WEIGHT_SCALE_CHANNEL ||
              o.weight_scale_mode == BFP8MOE_WEIGHT_MXFP4,
          "weight_scale_mode=%d is not 0 (block), 1 (channel) or 2 (MXFP4)", o.weight_scale_mode);
  REQUIRE(isfinite(o.act_static_scale) && o.act_static_scale >= 0 && isfinite(o.inter_static_scale) &&
              o.inter_static_scale >= 0,
          "static scales must be finite and >= 0 (0 = dynamic)");
  if (o.weight_scale_mode == BFP8MOE_WEIGHT_SCALE_CHANNEL) {
    if (!bfp8::rows_quant_fits(H) || !bfp8::rows_quant_fits(I))
      return fail(BFP8MOE_ERR_UNSUPPORTED, "the W8A8 (channel) variant takes H and I up to 8192 (H=%d I=%d)", H, I);
    if (o.flags & BFP8MOE_FLAG_LAYER_DECODE)
      return fail(BFP8MOE_ERR_UNSUPPORTED, "the W8A8 (channel) variant runs on the general and few-token paths");
  }
  if (o.weight_scale_mode == BFP8MOE_WEIGHT_MXFP4) {
    if (H % 256 != 0 || I % 256 != 0)
      return fail(BFP8MOE_ERR_UNSUPPORTED, "MXFP4 weights take H and I in multiples of 256 (H=%d I=%d)", H, I);
    if (o.flags & BFP8MOE_FLAG_LAYER_DECODE)
      return fail(BFP8MOE_ERR_UNSUPPORTED, "MXFP4 weights run on the general and few-token paths");
    REQUIRE(o.act_static_scale == 0 && o.inter_static_scale == 0, "static scales belong to the W8A8 variant");
  }
  if ((o.flags & BFP8MOE_FLAG_LAYER_DECODE) && M > 0 && !bfp8::decode_path_fits(M, H, k, I))
    return fail(BFP8MOE_ERR_UNSUPPORTED,
                "small-batch path forced but M=%lld k=%d H=%d I=%d exceed its limits (M<=8, k<=8, H<=8192, "
                "I<=512)",
                (long long)M, k, H, I);
  if ((o.flags & BFP8MOE_FLAG_LAYER_TOKEN) && M > 0 &&
      !bfp8::token_path_fits(M, H, k, I, o.weight_scale_mode))
    return fail(BFP8MOE_ERR_UNSUPPORTED,
                "few-token path forced but M=%lld k=%d H=%d I=%d do not fit it (M<=32, k<=16, H<=8192, "
                "I in {128, 256, 512}; MXFP4: I in {256, 512})",
                (long long)M, k, H, I);
  {
    const uint32_t paths = o.flags & (BFP8MOE_FLAG_LAYER_GENERAL | BFP8MOE_FLAG_LAYER_DECODE | BFP8MOE_FLAG_LAYER_TOKEN);
    REQUIRE((paths & (paths - 1)) == 0, "layer path flags are exclusive");
  }
  return BFP8MOE_OK;
}

}  // namespace

extern "C" {

int32_t fused_moe_block_fp8_stages(int64_t M, int32_t H, int32_t k, int32_t E, int32_t I,
                                   const bfp8moe_opts_t* opts, const char** names, int32_t cap) {
  bfp8moe_opts_t o;
  bfp8moe_opts_init(&o);
  if (opts) o = *opts;
  if (check_layer_shape(M, H, k, E, I, o) != BFP8MOE_OK) return -1;
  LayerPlan p;
  plan_layer(p, M, H, k, E, I, o);
  const char* const* list = p.mode == kModeToken    ? (p.mxfp4     ? kTokenMxfp4Stages
                                                       : p.channel ? kTokenChannelStages
                                                                   : kTokenStages)
                            : p.mode == kModeDecode ? kDecodeStages
                            : p.channel             ? kChannelStages
                            : p.mxfp4               ? (p.rq_fused ? kMxfp4FusedStages : kMxfp4Stages)
                            : p.rq_fused            ? kGeneralFusedStages
                                                    : kGeneralStages;
  const int32_t n = plan_stages(p);
  for (int32_t i = 0; names && i < n && i < cap; i++) names[i] = list[i];
  return n;
}

size_t fused_moe_block_fp8_workspace_size(int64_t M, int32_t H, int32_t k, int32_t E, int32_t I,
                                          const bfp8moe_opts_t* opts) {
  bfp8moe_opts_t o;
  bfp8moe_opts_init(&o);
  if (opts) o = *opts;
  if (check_layer_shape(M, H, k, E, I, o) != BFP8MOE_OK) return 0;
  LayerPlan p;
  plan_layer(p, M, H, k, E, I, o);
  return p.total;
}

}  // extern "C"

namespace {

// The layer for either scale type: w13_scale / w2_scale are fp32 (block and
// channel scales) or E8M0 bytes (MXFP4), as o.weight_scale_mode says.  With
// `route` (general path, single-workgroup route preparation, the caller has
// checked bfp8::route_prep_can_route), route preparation makes the routing
// itself and writes it to topk_ids / topk_w, which the later stages read.
bfp8moe_status_t layer_impl(const uint16_t* hidden, int64_t M, int32_t H, const int32_t* topk_ids,
                            const float* topk_w, int32_t k, const uint8_t* w13, const void* w13_scale_v,
                            const uint8_t* w2, const void* w2_scale_v, int32_t E, int32_t I, const bfp8moe_opts_t& o,
                            uint16_t* out, void* ws, size_t ws_bytes, void* stream,
                            const bfp8::RouterArgs* route = nullptr) {
  const float* w13_scale = static_cast<const float*>(w13_scale_v);
  const float* w2_scale = static_cast<const float*>(w2_scale_v);
  {
    const bfp8moe_status_t st = check_layer_shape(M, H, k, E, I, o);
    if (st != BFP8MOE_OK) return st;
  }
  REQUIRE(M == 0 || (hidden && topk_ids && topk_w && w13 && w13_scale && w2 && w2_scale && out),
          "all pointers must be non-null");
  REQUIRE(aligned16(hidden) && aligned16(w13) && aligned16(w2) && aligned16(out),
          "hidden, w13, w2 and out must be 16-byte aligned");
  REQUIRE(o.weight_scale_mode != BFP8MOE_WEIGHT_SCALE_CHANNEL || (aligned16(w13_scale) && aligned16(w2_scale)),
          "channel weight scales must be 16-byte aligned");
  REQUIRE(o.weight_scale_mode != BFP8MOE_WEIGHT_MXFP4 ||
              ((reinterpret_cast<uintptr_t>(w13_scale_v) & 7u) == 0 && (reinterpret_cast<uintptr_t>(w2_scale_v) & 7u) == 0),
          "MXFP4 scale bytes must be 8-byte aligned");
  if (M == 0) return BFP8MOE_OK;
  LayerPlan p;
  plan_layer(p, M, H, k, E, I, o);
  const int only = (int)((o.flags >> BFP8MOE_FLAG_STAGE_SHIFT) & 15u) - 1;
  const int n_stages = plan_stages(p);
  if (only >= n_stages) return fail(BFP8MOE_ERR_INVALID_ARG, "stage %d selected, the path has %d", only, n_stages);
  if (ws == nullptr || ws_bytes < p.total)
    return fail(BFP8MOE_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, p.total);
  REQUIRE((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) == 0, "workspace must be 256-byte aligned");

  hipStream_t st = (hipStream_t)stream;
  char* base = static_cast<char*>(ws);
  bfp8::LaunchHook hook;
  hook.events = o.stage_events;
  hook.n = o.stage_events ? n_stages + 1 : 0;
  hook.only = only;
  if (p.mode == kModeToken) {
    uint16_t* act = reinterpret_cast<uint16_t*>(base + p.off_act);
    return hip_status(bfp8::launch_token_layer(hidden, M, H, topk_ids, topk_w, k, layer_sel(p), w13, w13_scale_v,
                                               w2, w2_scale_v, I, p.fmt, p.clamp, act, out, st, &hook, nullptr,
                                               o.weight_scale_mode, p.a1_static, p.a2_static),
                      "fused_moe_block_fp8 (few tokens)");
  }
  if (p.mode == kModeDecode) {
    uint16_t* act = reinterpret_cast<uint16_t*>(base + p.off_act);
    return hip_status(bfp8::launch_decode_layer(hidden, M, H, topk_ids, topk_w, k, layer_sel(p), w13, w13_scale, w2,
                                                w2_scale, I, p.fmt, p.clamp, act, out, st, &hook),
                      "fused_moe_block_fp8 (small batch)");
  }
  uint8_t* aq = reinterpret_cast<uint8_t*>(base + p.off_aq);
  float* as = reinterpret_cast<float*>(base + p.off_as);
  int32_t* sorted = reinterpret_cast<int32_t*>(base + p.off_sorted);
  int32_t* eoff = reinterpret_cast<int32_t*>(base + p.off_eoff);
  int32_t* bexp = reinterpret_cast<int32_t*>(base + p.off_bexp);
  int32_t* bstart = reinterpret_cast<int32_t*>(base + p.off_bstart);
  int32_t* nb = reinterpret_cast<int32_t*>(base + p.off_nb);
  void* rws = base + p.off_rws;
  uint16_t* h13 = reinterpret_cast<uint16_t*>(base + p.off_h13);
  uint8_t* q = reinterpret_cast<uint8_t*>(base + p.off_q);
  float* s = reinterpret_cast<float*>(base + p.off_s);
  uint16_t* y = reinterpret_cast<uint16_t*>(base + p.off_y);

  hipError_t e = hipSuccess;
  // stage numbers: with the input quantisation carried by route preparation
  // (rq_fused) the stages after it move down by one
  const int sq = p.rq_fused ? 0 : 1;  // the stage that quantises the input
  int st_i = 0;
  hook.before(st_i, st);
  if (hook.run(st_i)) {
    const bfp8::QuantArgs qa{hidden, M, H, p.fmt, aq, as};
    e = bfp8::launch_route_prepare(topk_ids, p.R, layer_sel(p), p.block_m, sorted, eoff, bexp, bstart, p.max_blocks,
                                   nb, p.route_single, rws, st, p.rq_fused ? &qa : nullptr, route, k);
  }
  if (e != hipSuccess) return hip_status(e, "fused_moe_block_fp8: route prep");
  if (sq == 1) {
    hook.before(++st_i, st);
    if (hook.run(st_i))
      e = p.channel ? bfp8::launch_quant_fp8_rows(hidden, M, H, p.fmt, p.a1_static, aq, as, st)
                    : bfp8::launch_quant_fp8(hidden, M, H, p.fmt, aq, as, st);
    if (e != hipSuccess) return hip_status(e, "fused_moe_block_fp8: input quant");
  }
  hook.before(++st_i, st);
  if (hook.run(st_i))
    e = p.mxfp4 ? bfp8::launch_grouped_gemm_mxfp4(aq, as, k, w13, static_cast<const uint8_t*>(w13_scale_v), 2 * I, H,
                                                  sorted, eoff, bexp, bstart, nb, p.max_blocks, p.block_m, h13, st)
                : bfp8::launch_grouped_gemm(aq, as, k, w13, w13_scale, 2 * I, H, sorted, eoff, bexp, bstart, nb,
                                            p.max_blocks, p.block_m, h13, st, p.channel);
  if (e != hipSuccess) return hip_status(e, "fused_moe_block_fp8: gate/up GEMM");
  // act+quant over the local routes only: route preparation's sorted list
  // and its kept count (per-row scales: every row, filtered)
  bfp8::RowFilter f;
  f.ids = topk_ids;
  f.sel = layer_sel(p);
  f.mode = bfp8::kRowsLocal;
  hook.before(++st_i, st);
  if (hook.run(st_i))
    e = p.channel ? bfp8::launch_silu_and_mul_quant_rows(h13, p.R, I, f, p.clamp, p.fmt, p.a2_static, q, s, st)
                  : bfp8::launch_silu_and_mul_quant_list(h13, sorted, eoff + p.L, p.R, I, p.clamp, p.fmt, q, s, st);
  if (e != hipSuccess) return hip_status(e, "fused_moe_block_fp8: act+quant");
  hook.before(++st_i, st);
  if (hook.run(st_i))
    e = p.mxfp4 ? bfp8::launch_grouped_gemm_mxfp4(q, s, 1, w2, static_cast<const uint8_t*>(w2_scale_v), H, I, sorted,
                                                  eoff, bexp, bstart, nb, p.max_blocks, p.block_m, y, st)
                : bfp8::launch_grouped_gemm(q, s, 1, w2, w2_scale, H, I, sorted, eoff, bexp, bstart, nb,
                                            p.max_blocks, p.block_m, y, st, p.channel);
  if (e != hipSuccess) return hip_status(e, "fused_moe_block_fp8: down GEMM");
  hook.before(++st_i, st);
  if (hook.run(st_i)) e = bfp8::launch_moe_reduce(y, topk_w, topk_ids, layer_sel(p), M, k, H, out, st);
  hook.before(++st_i, st);
  return hip_status(e, "fused_moe_block_fp8: moe_reduce");
}

}  // namespace

extern "C" {

bfp8moe_status_t fused_moe_block_fp8(const uint16_t* hidden, int64_t M, int32_t H, const int32_t* topk_ids,
                                     const float* topk_w, int32_t k, const uint8_t* w13, const float* w13_scale,
                                     const uint8_t* w2, const float* w2_scale, int32_t E, int32_t I,
                                     const bfp8moe_opts_t* opts, uint16_t* out, void* ws, size_t ws_bytes,
                                     void* stream) {
  bfp8moe_opts_t o;
  bfp8moe_opts_init(&o);
  if (opts) o = *opts;
  REQUIRE(o.weight_scale_mode != BFP8MOE_WEIGHT_MXFP4, "MXFP4 weights (E8M0 scale bytes) take fused_moe_mxfp4");
  return layer_impl(hidden, M, H, topk_ids, topk_w, k, w13, w13_scale, w2, w2_scale, E, I, o, out, ws, ws_bytes,
                    stream);
}

bfp8moe_status_t fused_moe_mxfp4(const uint16_t* hidden, int64_t M, int32_t H, const int32_t* topk_ids,
                                 const float* topk_w, int32_t k, const uint8_t* w13, const uint8_t* w13_scale,
                                 const uint8_t* w2, const uint8_t* w2_scale, int32_t E, int32_t I,
                                 const bfp8moe_opts_t* opts, uint16_t* out, void* ws, size_t ws_bytes,
                                 void* stream) {
  REQUIRE(opts != nullptr && opts->weight_scale_mode == BFP8MOE_WEIGHT_MXFP4,
          "fused_moe_mxfp4 takes opts with weight_scale_mode BFP8MOE_WEIGHT_MXFP4");
  return layer_impl(hidden, M, H, topk_ids, topk_w, k, w13, w13_scale, w2, w2_scale, E, I, *opts, out, ws, ws_bytes,
                    stream);
}

bfp8moe_status_t moe_mxfp4_grouped_gemm(const uint8_t* A, const float* A_scale, int32_t a_row_div, const uint8_t* B,
                                        const uint8_t* B_scale, int32_t L, int32_t N, int32_t K,
                                        const int32_t* sorted_routes, const int32_t* expert_offsets,
                                        const int32_t* block_expert, const int32_t* block_start,
                                        const int32_t* num_blocks, int64_t max_blocks, int32_t block_m, int64_t R,
                                        uint16_t* C, void* stream) {
  REQUIRE(N > 0 && N % 128 == 0, "N=%d must be a positive multiple of 128", N);
  REQUIRE(K > 0 && K % 256 == 0, "K=%d must be a positive multiple of 256", K);
  REQUIRE(L >= 1, "L=%d must be >= 1", L);
  REQUIRE(a_row_div >= 1, "a_row_div=%d must be >= 1", a_row_div);
  REQUIRE(block_m == 16 || block_m == 32 || block_m == 64, "block_m=%d must be 16, 32 or 64", block_m);
  REQUIRE(R >= 0 && R <= 0x7FFFFFFF, "R=%lld out of range", (long long)R);
  REQUIRE(max_blocks >= 0, "max_blocks must be >= 0");
  REQUIRE(max_blocks == 0 || (A && A_scale && B && B_scale && sorted_routes && expert_offsets && block_expert &&
                              block_start && num_blocks && C),
          "all pointers must be non-null");
  REQUIRE(aligned16(A) && aligned16(B) && aligned16(C), "A, B and C must be 16-byte aligned");
  REQUIRE((reinterpret_cast<uintptr_t>(B_scale) & 7u) == 0, "B_scale must be 8-byte aligned");
  return hip_status(bfp8::launch_grouped_gemm_mxfp4(A, A_scale, a_row_div, B, B_scale, N, K, sorted_routes,
                                                    expert_offsets, block_expert, block_start, num_blocks,
                                                    max_blocks, block_m, C, (hipStream_t)stream),
                    "moe_mxfp4_grouped_gemm");
}

bfp8moe_status_t fused_moe_block_fp8_routed(const uint16_t* hidden, int64_t M, int32_t H, const float* router_logits,
                                            const float* router_bias, int32_t score_fn, int32_t renormalize,
                                            double routed_scale, int32_t n_group, int32_t topk_group, int32_t k,
                                            int32_t* topk_ids, float* topk_w,
                                            const uint8_t* w13, const float* w13_scale, const uint8_t* w2,
                                            const float* w2_scale, int32_t E, int32_t I, const bfp8moe_opts_t* opts,
                                            uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  bfp8moe_opts_t o;
  bfp8moe_opts_init(&o);
  if (opts) o = *opts;
  REQUIRE(E >= 1 && E <= 1024, "E=%d must be in [1, 1024]", E);
  REQUIRE(k >= 1 && k <= 64 && k <= E, "k=%d must be in [1, min(E, 64)]", k);
  REQUIRE(score_fn == BFP8MOE_SCORE_SOFTMAX || score_fn == BFP8MOE_SCORE_SIGMOID, "score_fn=%d invalid", score_fn);
  REQUIRE(router_bias == nullptr || score_fn == BFP8MOE_SCORE_SIGMOID, "a selection bias needs sigmoid scoring");
  REQUIRE(isfinite(routed_scale), "routed_scale must be finite");
  REQUIRE(n_group >= 1 && n_group <= 64 && E % n_group == 0, "n_group=%d must divide E=%d and be in [1, 64]",
          n_group, E);
  REQUIRE(n_group == 1 || score_fn == BFP8MOE_SCORE_SIGMOID, "grouped (noaux-TC) selection uses sigmoid scoring");
  REQUIRE(topk_group >= 1 && topk_group <= n_group, "topk_group=%d must be in [1, n_group=%d]", topk_group, n_group);
  REQUIRE((int64_t)k <= (int64_t)topk_group * (E / n_group), "k=%d exceeds the experts of %d groups", k,
          topk_group);
  REQUIRE(o.stage_events == nullptr && ((o.flags >> BFP8MOE_FLAG_STAGE_SHIFT) & 15u) == 0,
          "the routed layer takes no stage events or stage selection");
  {
    const bfp8moe_status_t st = check_layer_shape(M, H, k, E, I, o);
    if (st != BFP8MOE_OK) return st;
  }
  REQUIRE(M == 0 || (router_logits && topk_ids && topk_w), "router_logits, topk_ids and topk_w must be non-null");
  if (M == 0) return BFP8MOE_OK;
  // every check of both steps before anything is enqueued
  REQUIRE(hidden && w13 && w13_scale && w2 && w2_scale && out, "all pointers must be non-null");
  REQUIRE(aligned16(hidden) && aligned16(w13) && aligned16(w2) && aligned16(out),
          "hidden, w13, w2 and out must be 16-byte aligned");
  LayerPlan p;
  plan_layer(p, M, H, k, E, I, o);
  if (ws == nullptr || ws_bytes < p.total)
    return fail(BFP8MOE_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, p.total);
  REQUIRE((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) == 0, "workspace must be 256-byte aligned");
  REQUIRE(o.weight_scale_mode != BFP8MOE_WEIGHT_MXFP4, "MXFP4 weights (E8M0 scale bytes) take fused_moe_mxfp4");
  if (o.flags & BFP8MOE_FLAG_ROUTER_IN_ROUTE_PREP) {
    // the router inside route preparation's workgroup, one launch for both
    if (p.mode != kModeGeneral || !p.route_single || !bfp8::route_prep_can_route(M, E, p.L, p.R))
      return fail(BFP8MOE_ERR_UNSUPPORTED,
                  "the router in route preparation needs the general path, one route-prep workgroup, M <= %lld, "
                  "E <= %d and L <= %d (M=%lld E=%d L=%d)",
                  (long long)bfp8::kRoutePrepRouterMaxM, bfp8::kFoldedRouterMaxE, bfp8::kRoutePrepRouterMaxL,
                  (long long)M, E, p.L);
    const bfp8::RouterArgs ra{router_logits, router_bias, topk_ids, topk_w, routed_scale, E, score_fn,
                              renormalize != 0, n_group, topk_group};
    return layer_impl(hidden, M, H, topk_ids, topk_w, k, w13, w13_scale, w2, w2_scale, E, I, o, out, ws, ws_bytes,
                      stream, &ra);
  }
  if (p.mode == kModeToken && E <= bfp8::kFoldedRouterMaxE && M <= bfp8::kFoldedRouterMaxM) {
    uint16_t* act = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + p.off_act);
    const bfp8::RouterArgs ra{router_logits, router_bias, topk_ids, topk_w, routed_scale, E, score_fn,
                              renormalize != 0, n_group, topk_group};
    return hip_status(bfp8::launch_token_layer(hidden, M, H, topk_ids, topk_w, k, layer_sel(p), w13, w13_scale, w2,
                                               w2_scale, I, p.fmt, p.clamp, act, out, (hipStream_t)stream, nullptr,
                                               &ra),
                      "fused_moe_block_fp8_routed (few tokens)");
  }
  // other paths: the router's own launch, then the layer
  const bfp8moe_status_t rs =
      n_group > 1 ? moe_router_noaux_tc(router_logits, M, E, k, n_group, topk_group, router_bias, renormalize,
                                        routed_scale, topk_ids, topk_w, stream)
                  : moe_router_topk(router_logits, M, E, k, score_fn, router_bias, renormalize, routed_scale,
                                    topk_ids, topk_w, stream);
  if (rs != BFP8MOE_OK) return rs;
  return fused_moe_block_fp8(hidden, M, H, topk_ids, topk_w, k, w13, w13_scale, w2, w2_scale, E, I, &o, out, ws,
                             ws_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The layer without a workspace argument, for callers that cannot allocate.
// Its workspace is `scratch`, a file-scope device array: each GPU the library
// runs on holds its own copy for the life of the process.  In host code the
// array's name is a host-side stand-in, so its device address is looked up
// once per device (hipGetSymbolAddress, with that device current) and only
// that address is handed to kernels.

static __device__ __align__(256) uint8_t scratch[BFP8MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the
// first call on each device).
bfp8moe_status_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "fused_moe_block_fp8_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(BFP8MOE_ERR_UNSUPPORTED, "fused_moe_block_fp8_noalloc: device %d beyond the %d the library tracks",
                dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "fused_moe_block_fp8_noalloc: hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(BFP8MOE_ERR_HIP, "fused_moe_block_fp8_noalloc: null scratch address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BFP8MOE_OK;
}

}  // namespace

extern "C" bfp8moe_status_t fused_moe_block_fp8_noalloc(const uint16_t* hidden, int64_t M, int32_t H,
                                                        const int32_t* topk_ids, const float* topk_w, int32_t k,
                                                        const uint8_t* w13, const float* w13_scale, const uint8_t* w2,
                                                        const float* w2_scale, int32_t E, int32_t I,
                                                        const bfp8moe_opts_t* opts, uint16_t* out, void* stream) {
  bfp8moe_opts_t o;
  bfp8moe_opts_init(&o);
  if (opts) o = *opts;
  {
    const bfp8moe_status_t st = check_layer_shape(M, H, k, E, I, o);
    if (st != BFP8MOE_OK) return st;
  }
  LayerPlan p;
  plan_layer(p, M, H, k, E, I, o);
  if (p.total > (size_t)BFP8MOE_NOALLOC_SCRATCH_BYTES)
    return fail(BFP8MOE_ERR_WORKSPACE,
                "fused_moe_block_fp8_noalloc: this call needs %zu bytes of scratch, the limit is %zu; "
                "use fused_moe_block_fp8 with a workspace",
                p.total, (size_t)BFP8MOE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const bfp8moe_status_t st = scratch_address(&ws);
  if (st != BFP8MOE_OK) return st;
  return fused_moe_block_fp8(hidden, M, H, topk_ids, topk_w, k, w13, w13_scale, w2, w2_scale, E, I, &o, out, ws,
                             (size_t)BFP8MOE_NOALLOC_SCRATCH_BYTES, stream);
}
