/*
 * bfp8moe.h -- C ABI of the block-FP8 fused MoE library for AMD Instinct
 * MI355X (gfx950).
 *
 * The library computes one mixture-of-experts FFN layer whose expert weights
 * are OCP E4M3FN bytes with one fp32 scale per 128x128 block, and whose
 * activations are quantised on the fly to E4M3FN with one scale per 1x128
 * group.  The layer is a pipeline of five steps, each also exported alone:
 *
 *   moe_route_prepare       top-k routes sorted by expert into compact blocks
 *   quant_fp8               group-128 dynamic activation quantisation
 *   moe_fp8_grouped_gemm    block-FP8 grouped GEMM over active experts only
 *   silu_and_mul_quant_fp8  SwiGLU (optionally clamped) fused with quant_fp8
 *   moe_reduce              top-k weighted sum back to token order
 *
 * and fused_moe_block_fp8 runs the whole layer in one call.  The step before
 * it, the single-group top-k router (moe_router_topk), turns router logits
 * into the top-k ids and weights; fused_moe_block_fp8_routed runs the router
 * and the layer in one call.
 *
 * Sources, cited by page title and section:
 *   [P1] lmdeploy PR "Perf/pytorch block fp8 moe decode"
 *   [P2] lmdeploy PR "perf(pytorch): optimize compact blocked FP8 MoE and route
 *        preparation"
 *   [P3] vLLM PR "[Kernel][Perf] Fuse clamped MoE activation and UE8M0 FP8 block
 *        quantization"
 *   [P4] lmdeploy PR "Moe Reduce kernel"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.  Every pointer argument is a DEVICE pointer unless it is marked
 *   "host".  The caller owns all memory (inputs, outputs, workspace); the
 *   library never allocates, frees, synchronises the host or reads device data
 *   on the host, so every call is legal inside HIP stream capture (the one
 *   exception is the debugging query bfp8moe_wait_faults).
 * Layout.  Row-major and contiguous.  BF16 is passed as uint16_t bit patterns,
 *   E4M3FN as uint8_t codes.  Device pointers must be 16-byte aligned.
 * Streams.  `stream` is a hipStream_t passed as void*; NULL is the default
 *   stream.  Work is enqueued asynchronously on it.
 * Errors.  Arguments are validated on the host before anything is enqueued; a
 *   non-zero status means nothing was launched (except BFP8MOE_ERR_HIP, which
 *   reports a failed launch).  bfp8moe_last_error() returns a message for the
 *   most recent failure on the calling thread.
 * Masked routes.  A route whose expert id, minus expert_offset, falls outside
 *   [0, local_num_experts) -- for example -1 -- is not an error: it is skipped
 *   by every step, and rows that belong to it are left untouched
 *   [P3 Purpose: optional filtering of invalid or non-local expert rows].
 * Expert maps.  Instead of a contiguous slice, the local experts can be given
 *   by an expert map: a device int32 array of E entries, entry i the local
 *   expert of global expert i, or a value outside [0, local_num_experts) --
 *   for example -1 -- for an expert held elsewhere [P3 Purpose: the
 *   expert_map of expert parallelism].  Routes whose ids fall outside [0, E)
 *   or whose entry is outside [0, local_num_experts) are masked.
 * Determinism.  Repeated calls with the same inputs give bit-identical outputs.
 */
#ifndef BFP8MOE_H
#define BFP8MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BFP8MOE_OK = 0,
    BFP8MOE_ERR_INVALID_ARG = 1,   /* null pointer, bad size, slice outside [0, E), ... */
    BFP8MOE_ERR_UNSUPPORTED = 2,   /* a shape the kernels do not handle (no silent fallback) */
    BFP8MOE_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required */
    BFP8MOE_ERR_HIP = 4            /* a HIP launch failed */
} bfp8moe_status_t;

/* Format of the per-group activation scales.  Both are stored as fp32.
 * FP32:  scale = max(amax, 1e-10) / 448, one IEEE fp32 division.
 * UE8M0: that value rounded up to a power of two (its fp32 exponent field,
 *        plus one when the mantissa is non-zero)
 *        [P4 Pull request overview: scale_fmt 'ue8m0'; P3 Purpose: UE8M0 scales]. */
typedef enum { BFP8MOE_SCALE_FP32 = 0, BFP8MOE_SCALE_UE8M0 = 1 } bfp8moe_scale_fmt_t;

/* Test-only switches that force one implementation where several exist. */
enum {
    BFP8MOE_FLAG_ROUTE_SINGLE_WG = 1u << 0,  /* route prep: one workgroup */
    BFP8MOE_FLAG_ROUTE_MULTI_WG = 1u << 1,   /* route prep: count -> scan+scatter over many workgroups */
    BFP8MOE_FLAG_LAYER_GENERAL = 1u << 2,    /* fused layer: staged general path */
    BFP8MOE_FLAG_LAYER_DECODE = 1u << 3,     /* fused layer: small-batch two-kernel path */
    BFP8MOE_FLAG_LAYER_TOKEN = 1u << 4,      /* fused layer: few-token two-kernel path */
    /* fused_moe_block_fp8_routed on the general path: the router runs inside
     * route preparation's single workgroup, one wave per token, so router and
     * route preparation are one launch [P2 Changes: the fused top-k router
     * feeds the layer].  Up to 64 tokens, 256 experts, 512 local experts;
     * otherwise the call fails with BFP8MOE_ERR_UNSUPPORTED.  Off by default:
     * measured slower than the router's own launch at 16 to 64 tokens. */
    BFP8MOE_FLAG_ROUTER_IN_ROUTE_PREP = 1u << 5,
    BFP8MOE_FLAG_STAGE_SHIFT = 8             /* flags bits 8..11, see BFP8MOE_FLAG_ONLY_STAGE */
};
/* Test and profiling switch of the fused layer: launch only stage s (0-based,
 * in the order fused_moe_block_fp8_stages lists them) of the path the call
 * takes, reading and writing the workspace exactly as a whole call does.  A
 * stage past the first reads what the earlier stages of a whole call with
 * the same arguments and workspace left there; stage 0 needs nothing.  Lets
 * a profiler time one kernel on its own.  s past the last stage is rejected. */
#define BFP8MOE_FLAG_ONLY_STAGE(s) ((uint32_t)((s) + 1) << BFP8MOE_FLAG_STAGE_SHIFT)

/* Options of the fused layer.  Initialise with bfp8moe_opts_init(). */
typedef struct {
    int32_t block_m;            /* routes per compact block for the general path (16, 32 or 64);
                                   0 = auto: 16 below 8 routes per local expert, then 32,
                                   and 64 from 32 (MXFP4 weights: above 48) */
    int32_t scale_fmt;          /* bfp8moe_scale_fmt_t for both activation quantisations */
    float clamp_limit;          /* SwiGLU clamp; +INFINITY = unclamped [P3 Purpose: finite SwiGLU clamping] */
    int32_t expert_offset;      /* first global expert held locally [P2 Suppressed comments] */
    int32_t local_num_experts;  /* experts held locally (weights' leading dimension); 0 = all E */
    uint32_t flags;             /* BFP8MOE_FLAG_* (tests only); 0 = choose by shape */
    void* const* stage_events;  /* profiling, NULL = off: host array of n+1 hipEvent_t (as void*) for a call
                                   of n stages (fused_moe_block_fp8_stages); event i is recorded on the
                                   stream before stage i, event n after the last.  Events are caller-owned.
                                   For eager calls; not for use under stream capture. */
    int32_t weight_scale_mode;  /* bfp8moe_weight_scale_t: BLOCK (default) or CHANNEL (the W8A8 variant) */
    float act_static_scale;     /* CHANNEL only: > 0 a static per-tensor scale of the hidden states;
                                   0 = one dynamic scale per token (its amax / 448, in scale_fmt) */
    float inter_static_scale;   /* CHANNEL only: the same for the SwiGLU output (per route row) */
    const int32_t* expert_map;  /* NULL = the slice above; else the expert map (device, [E] int32; see
                                   "Expert maps"), with expert_offset 0 and local_num_experts the weights'
                                   leading dimension.  Read by the kernels, not by the host. */
} bfp8moe_opts_t;

/* How the layer's weights and activations are scaled.
 * BLOCK:   [128, 128] weight blocks (w13_scale [L, 2I/128, H/128], w2_scale
 *          [L, H/128, I/128]) and 1x128 activation groups -- the block-FP8
 *          layer [P3 Purpose: FP8 W8A8 block shape [128, 128]].
 * CHANNEL: one fp32 scale per weight row (w13_scale [L, 2I], w2_scale [L, H])
 *          and one per activation row, dynamic or static -- the W8A8 variant
 *          [P2 Reviewed changes: w8a8.py, the static FP8 MoE backend].  Runs
 *          the few-token path (two launches; stages
 *          "token_gate_up_swiglu_channel", "token_down_reduce_channel") or the
 *          general path (six launches); H and I at most 8192.
 * MXFP4:   weights in OCP MX FP4 -- E2M1 elements two to a byte (the even
 *          element of a pair in the low nibble) with one E8M0 scale byte per 32
 *          along K (w13 [L, 2I, H/2] with w13_scale [L, 2I, H/32] bytes, w2
 *          [L, H, I/2] with w2_scale [L, H, I/32]); activations as BLOCK
 *          [P2 Reviewed changes: v4_fp4_grouped_gemm.py, v4_swiglu_quant.py;
 *          P3 Matched GLM serving A/B: MXFP4 the DeepSeek-V4 checkpoint's
 *          weight format].  Called through fused_moe_mxfp4 (byte scales); runs
 *          the few-token path (up to 8 tokens by default, I 256 or 512; stages
 *          "token_gate_up_swiglu_mxfp4", "token_down_reduce_mxfp4") or the
 *          general path; H and I multiples of 256.  Neither variant takes the
 *          small-batch path. */
typedef enum {
    BFP8MOE_WEIGHT_SCALE_BLOCK = 0,
    BFP8MOE_WEIGHT_SCALE_CHANNEL = 1,
    BFP8MOE_WEIGHT_MXFP4 = 2
} bfp8moe_weight_scale_t;

/* Fill *opts with the defaults: block_m 0, FP32 scales, no clamp, the full
 * expert range, no flags, no stage events, block scaling.  opts: host
 * pointer. */
void bfp8moe_opts_init(bfp8moe_opts_t* opts);

const char* bfp8moe_status_string(int status);
/* Message of the last failure on this thread ("" if none).  Host string owned
 * by the library, valid until the next call on the same thread. */
const char* bfp8moe_last_error(void);

/* Fault bits of the kernels' bounded waits on the current device, accumulated
 * since the last clear: bit 0 is set when a column wave of the few-token
 * gate/up kernel ran out of its bounded wait for the quantised hidden row (the
 * kernel then ends normally, but that column of that call is unspecified);
 * bit 1 when, in that kernel's W8A8 form, a hidden-row wave ran out of its
 * wait for the other hidden-row waves' maxima (the row's scale of that call is
 * then unspecified).
 * flags: host pointer.  clear != 0 resets them afterwards.  A debugging and
 * testing query: it synchronises with the device (it copies one word), so it
 * is not for use inside stream capture or a latency-critical loop. */
bfp8moe_status_t bfp8moe_wait_faults(uint32_t* flags, int clear);

/* Measurement only (no part of the layer): one launch that reads the device
 * buffer buf [bytes] and keeps nothing, to time what this memory system gives
 * a read shape.  pattern 0: contiguous 512 KiB slabs, one per workgroup
 * (bytes / 512 KiB workgroups).  pattern 1: the buffer as rows of row_bytes
 * (a multiple of 1024 and of piece), one workgroup per 128 rows read the way
 * the grouped GEMM reads a weight tile, piece bytes of each row per load
 * (128, 256 or 1024; 128 is the GEMM's; bytes / (128 row_bytes)
 * workgroups).  pattern 2: as 1, workgroup b starting along the row at piece
 * b mod (row_bytes / piece) and wrapping around.  lds_bytes (0 .. 163840) of unused dynamic LDS per workgroup
 * bound how many share a compute unit.  sink [sink_len] device uint32, at
 * least one word per workgroup (never written in practice).  buf 16-byte
 * aligned.  Returns BFP8MOE_ERR_INVALID_ARG for any other shape. */
bfp8moe_status_t bfp8moe_stream_probe(const uint8_t* buf, size_t bytes, int32_t pattern, int32_t row_bytes,
                                      int32_t piece, int32_t lds_bytes, uint32_t* sink, int64_t sink_len,
                                      void* stream);

/* ------------------------------------------------------------------------- */
/* Route preparation                                                         */
/* [P2 Changes: shared route preparation, one workgroup for small problems,   */
/*  a scalable parallel path for large ones, sorted-indices and compact-block */
/*  contracts; P1 Modification, Active-expert block scheduling: blocks only   */
/*  for experts that receive tokens]                                          */
/* ------------------------------------------------------------------------- */

/* Upper bound on the number of compact blocks for R routes over L local
 * experts: floor((R + min(L, R) * (block_m - 1)) / block_m).  Host function. */
int64_t bfp8moe_max_blocks(int64_t R, int32_t L, int32_t block_m);

/* Device workspace (bytes) moe_route_prepare needs for R routes and L experts
 * (0 when the single-workgroup path will be used). */
size_t moe_route_prepare_workspace_size(int64_t R, int32_t L, uint32_t flags);

/* topk_ids [R] int32: the flattened [M, k] router choice, route r = t*k + j.
 * A route is kept when topk_ids[r] - expert_offset lies in [0, L).
 * Outputs:
 *   sorted_routes  [R]   kept routes ordered by local expert, ties by route
 *                        index (stable); entries past the kept routes are -1.
 *   expert_offsets [L+1] start of each local expert's segment in sorted_routes;
 *                        expert_offsets[L] = number of kept routes.
 *   block_expert, block_start [max_blocks] (both NULL = sorted-indices contract
 *                        only): for each expert with c > 0 routes, in expert
 *                        order, ceil(c / block_m) blocks naming the local
 *                        expert and the block's first position in
 *                        sorted_routes; a block holds min(block_m, segment end
 *                        - start) routes.  Unused slots hold -1.
 *   num_blocks     [1]   number of blocks (device int32).
 * max_blocks must be >= bfp8moe_max_blocks(R, L, block_m).  Requires
 * 0 <= expert_offset, 1 <= L, block_m >= 1, R <= 2^31 - 1.  ws may be NULL when
 * the size function returns 0. */
bfp8moe_status_t moe_route_prepare(const int32_t* topk_ids, int64_t R, int32_t expert_offset, int32_t L,
                                   int32_t block_m, int32_t* sorted_routes, int32_t* expert_offsets,
                                   int32_t* block_expert, int32_t* block_start, int64_t max_blocks,
                                   int32_t* num_blocks, void* ws, size_t ws_bytes, uint32_t flags,
                                   void* stream);

/* moe_route_prepare with the local experts given by an expert map
 * [P3 Purpose: expert_map]: route r is kept when topk_ids[r] lies in
 * [0, num_experts) and e = expert_map[topk_ids[r]] lies in [0, L); it joins
 * local expert e's segment.  expert_map: device int32 [num_experts], read by
 * the kernels (its values are not checked on the host: any value outside
 * [0, L) masks).  Outputs, ordering, workspace and the other requirements as
 * moe_route_prepare; num_experts >= 1. */
bfp8moe_status_t moe_route_prepare_map(const int32_t* topk_ids, int64_t R, const int32_t* expert_map,
                                       int32_t num_experts, int32_t L, int32_t block_m, int32_t* sorted_routes,
                                       int32_t* expert_offsets, int32_t* block_expert, int32_t* block_start,
                                       int64_t max_blocks, int32_t* num_blocks, void* ws, size_t ws_bytes,
                                       uint32_t flags, void* stream);

/* ------------------------------------------------------------------------- */
/* Group-128 activation quantisation                                         */
/* [P1 Motivation: quant_fp8 feeding the FP8 projection; P4 Pull request      */
/*  overview: scale_fmt; P3 Purpose: dynamic E4M3 block quantisation]         */
/* ------------------------------------------------------------------------- */

/* x [rows, K] BF16 -> q [rows, K] E4M3FN and scales [rows, K/128] fp32.
 * Per group of 128 columns: s from the group's amax (see bfp8moe_scale_fmt_t),
 * q_i = E4M3FN(x_i / s) by IEEE fp32 division and round-to-nearest-even,
 * saturating at +-448.  K must be a positive multiple of 128. */
bfp8moe_status_t quant_fp8(const uint16_t* x, int64_t rows, int32_t K, int32_t scale_fmt, uint8_t* q,
                           float* scales, void* stream);

/* ------------------------------------------------------------------------- */
/* SwiGLU and fused SwiGLU + quantisation                                    */
/* [P1 Modification, Fused SwiGLU and FP8 quantization; P3 Purpose]           */
/* ------------------------------------------------------------------------- */

/* gate_up [rows, 2I] BF16, gate in columns [0, I), up in [I, 2I).
 * out [rows, I] BF16 = bf16(silu(g) * u) with g = min(gate, clamp_limit),
 * u = clamp(up, -clamp_limit, clamp_limit) when clamp_limit is finite, and
 * silu(g) = g / (1 + exp(-g)) evaluated in fp32 (exp correctly rounded), one
 * rounding to BF16.  I must be a positive multiple of 128.  This is the
 * unfused half of the two-kernel path. */
bfp8moe_status_t silu_and_mul(const uint16_t* gate_up, int64_t rows, int32_t I, float clamp_limit,
                              uint16_t* out, void* stream);

/* Fused SwiGLU + group-128 quantisation: for every live row, q and scales are
 * bit-identical to quant_fp8(silu_and_mul(gate_up)); the BF16 SwiGLU value
 * never leaves registers.  A row r is live unless row_expert_ids is given and
 * row_expert_ids[r] is outside [0, E), or expert_map [E] is given and
 * expert_map[row_expert_ids[r]] < 0.  Rows that are not live are not written.
 * q [rows, I] E4M3FN, scales [rows, I/128] fp32.  expert_map requires
 * row_expert_ids. */
bfp8moe_status_t silu_and_mul_quant_fp8(const uint16_t* gate_up, int64_t rows, int32_t I,
                                        const int32_t* row_expert_ids, const int32_t* expert_map, int32_t E,
                                        float clamp_limit, int32_t scale_fmt, uint8_t* q, float* scales,
                                        void* stream);

/* The W8A8 variant's quantisation [P2 Reviewed changes: w8a8.py, the static
 * FP8 MoE backend]: one scale per row.  x [rows, K] BF16 -> q [rows, K]
 * E4M3FN and scales [rows] fp32; the scale is static_scale when > 0 (codes
 * saturate at +-448), else the row's amax / 448 over all K (in scale_fmt, as
 * quant_fp8's group scale).  K a positive multiple of 128, at most 8192. */
bfp8moe_status_t quant_fp8_rows(const uint16_t* x, int64_t rows, int32_t K, int32_t scale_fmt, float static_scale,
                                uint8_t* q, float* scales, void* stream);

/* Fused SwiGLU + per-row quantisation (the W8A8 variant): for every live row
 * (filtering as silu_and_mul_quant_fp8), q [rows, I] and scales [rows] equal
 * quant_fp8_rows(silu_and_mul(gate_up)).  I at most 8192. */
bfp8moe_status_t silu_and_mul_quant_fp8_rows(const uint16_t* gate_up, int64_t rows, int32_t I,
                                             const int32_t* row_expert_ids, const int32_t* expert_map, int32_t E,
                                             float clamp_limit, int32_t scale_fmt, float static_scale, uint8_t* q,
                                             float* scales, void* stream);

/* ------------------------------------------------------------------------- */
/* Block-FP8 grouped GEMM over compact blocks                                */
/* [P3 Purpose: FP8 W8A8 block shape [128, 128]; P1 Modification:            */
/*  GEMM programs only for blocks that receive tokens; P2 Changes: transposed */
/*  MMA for small-M gate/up tiles]                                           */
/* ------------------------------------------------------------------------- */

/* For every block b < *num_blocks (device value) with local expert
 * e = block_expert[b] and routes r = sorted_routes[p] for p in
 * [block_start[b], min(block_start[b] + block_m, expert_offsets[e+1])):
 *   C[r, n] = bf16( sum_g (A_scale[r/a_row_div, g] * B_scale[e, n/128, g])
 *                        * sum_{i in group g} A[r/a_row_div, i] * B[e, n, i] ),  n < N,
 * accumulated in fp32.  A [R/a_row_div rows, K] E4M3FN with A_scale [.., K/128];
 * B [L, N, K] E4M3FN with B_scale [L, N/128, K/128]; C [R, N] BF16 indexed by
 * route id (rows of routes not in any block are untouched).  a_row_div is the
 * top-k for the gate/up projection (token rows feed k routes) and 1 for the
 * down projection.  N and K must be positive multiples of 128; block_m one of
 * 16, 32, 64; max_blocks the size of the block arrays; R the number of routes
 * (rows of C).  The block arrays must be laid out as moe_route_prepare writes
 * them for the same block_m: an expert's blocks consecutive, its i-th block
 * starting at expert_offsets[e] + i * block_m (the kernel derives a block's
 * start from its expert's segment instead of reading it). */
bfp8moe_status_t moe_fp8_grouped_gemm(const uint8_t* A, const float* A_scale, int32_t a_row_div,
                                      const uint8_t* B, const float* B_scale, int32_t L, int32_t N, int32_t K,
                                      const int32_t* sorted_routes, const int32_t* expert_offsets,
                                      const int32_t* block_expert, const int32_t* block_start,
                                      const int32_t* num_blocks, int64_t max_blocks, int32_t block_m,
                                      int64_t R, uint16_t* C, void* stream);

/* The grouped GEMM with MXFP4 weights: as moe_fp8_grouped_gemm with
 * B [L, N, K/2] packed E2M1 and B_scale [L, N, K/32] E8M0 bytes (8-byte
 * aligned):
 *   C[r, n] = bf16( sum_g A_scale[r/a_row_div, g] * sum_{b in group g} 2^(B_scale[e, n, b] - 127)
 *                        * sum_{i in block b} A[r/a_row_div, i] * B[e, n, i] ),
 * blocks b of 32 along K, accumulated in fp32.  K a positive multiple of 256
 * [P2 Reviewed changes: v4_fp4_grouped_gemm.py]. */
bfp8moe_status_t moe_mxfp4_grouped_gemm(const uint8_t* A, const float* A_scale, int32_t a_row_div, const uint8_t* B,
                                        const uint8_t* B_scale, int32_t L, int32_t N, int32_t K,
                                        const int32_t* sorted_routes, const int32_t* expert_offsets,
                                        const int32_t* block_expert, const int32_t* block_start,
                                        const int32_t* num_blocks, int64_t max_blocks, int32_t block_m, int64_t R,
                                        uint16_t* C, void* stream);

/* The grouped GEMM of the W8A8 variant: as moe_fp8_grouped_gemm with one
 * activation scale per row, A_scale [R/a_row_div rows], and one weight scale
 * per output channel, B_scale [L, N] (16-byte aligned):
 *   C[r, n] = bf16( A_scale[r/a_row_div] * B_scale[e, n] * sum_i A[r/a_row_div, i] * B[e, n, i] ). */
bfp8moe_status_t moe_fp8_grouped_gemm_channel(const uint8_t* A, const float* A_scale, int32_t a_row_div,
                                              const uint8_t* B, const float* B_scale, int32_t L, int32_t N,
                                              int32_t K, const int32_t* sorted_routes,
                                              const int32_t* expert_offsets, const int32_t* block_expert,
                                              const int32_t* block_start, const int32_t* num_blocks,
                                              int64_t max_blocks, int32_t block_m, int64_t R, uint16_t* C,
                                              void* stream);

/* ------------------------------------------------------------------------- */
/* Single-group top-k router                                                 */
/* [P2 Changes: a fused single-group top-k router, with a renormalize        */
/*  option, produces the top-k ids and weights the layer consumes]           */
/* ------------------------------------------------------------------------- */

typedef enum { BFP8MOE_SCORE_SOFTMAX = 0, BFP8MOE_SCORE_SIGMOID = 1 } bfp8moe_score_fn_t;

/* logits [M, E] fp32 -> topk_ids [M, k] int32 and topk_w [M, k] fp32, each
 * token's k experts in order of decreasing score.  All experts form one group.
 * Ranking: softmax scoring ranks the logits themselves (softmax is increasing);
 * sigmoid scoring ranks s_e + bias[e] in fp32, s_e the sigmoid of the logit
 * computed in fp64 and rounded to fp32, bias [E] fp32 optional (NULL: none;
 * it steers the choice only, never a weight).  Equal ranks go to the lower
 * expert id; -0 and +0 rank equal.  Weights, fp64 rounded once to fp32, times
 * scale:
 *   softmax:  exp(l_j - max_e l_e) / Z, Z summed over the k chosen experts when
 *             renormalize != 0, else over all E (plain softmax probabilities);
 *   sigmoid:  1 / (1 + exp(-l_j)), divided by the sum over the k chosen when
 *             renormalize != 0.
 * 1 <= E <= 1024, 1 <= k <= min(E, 64); a bias needs sigmoid scoring; NaN
 * logits are outside the contract (the ids stay k distinct values in [0, E)).
 * The output is fed to the layer as its topk_ids / topk_w. */
bfp8moe_status_t moe_router_topk(const float* logits, int64_t M, int32_t E, int32_t k, int32_t score_fn,
                                 const float* bias, int32_t renormalize, double scale, int32_t* topk_ids,
                                 float* topk_w, void* stream);

/* Group-limited noaux-TC router [P2 Reviewed changes: route_noaux_tc.py, a
 * noaux-TC routing kernel the MoE router switches to].  Reading of the method
 * the pages name: sigmoid scores s_e computed as above; choice keys
 * s_e + bias[e] in fp32 (s_e alone when bias is NULL); the E experts form
 * n_group groups of E / n_group consecutive ids, each scored by the fp32 sum of
 * its two largest keys (its one key when a group has one expert); the
 * topk_group best groups are kept (equal scores: the lower group index); the
 * k largest keys among their experts are chosen, largest first (equal keys:
 * the lower expert id).  Weights as moe_router_topk's sigmoid scoring: from
 * the unbiased scores, divided by their sum over the k chosen when
 * renormalize != 0, times scale.  1 <= E <= 1024, n_group in [1, 64] dividing
 * E, 1 <= topk_group <= n_group, 1 <= k <= min(64, topk_group * E / n_group);
 * n_group = 1 is moe_router_topk with sigmoid scoring. */
bfp8moe_status_t moe_router_noaux_tc(const float* logits, int64_t M, int32_t E, int32_t k, int32_t n_group,
                                     int32_t topk_group, const float* bias, int32_t renormalize, double scale,
                                     int32_t* topk_ids, float* topk_w, void* stream);

/* ------------------------------------------------------------------------- */
/* moe_reduce                                                                */
/* [P4 Pull request overview: a dedicated reduction applies the router        */
/*  weights, which the expert GEMMs no longer apply]                          */
/* ------------------------------------------------------------------------- */

/* out[t, n] = bf16(acc) where acc starts at +0 and, for j = 0..k-1 in order,
 * acc = fmaf(topk_w[t, j], y[t*k + j, n], acc) over live routes (all routes
 * when topk_ids is NULL; otherwise topk_ids[t, j] - expert_offset in [0, L)).
 * y [M*k, H] BF16, topk_w [M, k] fp32, out [M, H] BF16.  H must be a positive
 * multiple of 8. */
bfp8moe_status_t moe_reduce(const uint16_t* y, const float* topk_w, const int32_t* topk_ids,
                            int32_t expert_offset, int32_t L, int64_t M, int32_t k, int32_t H, uint16_t* out,
                            void* stream);

/* moe_reduce with live routes given by an expert map: topk_ids[t, j] in
 * [0, num_experts) and expert_map[topk_ids[t, j]] in [0, L).  topk_ids and
 * expert_map (device int32 [num_experts]) non-null; num_experts, L >= 1. */
bfp8moe_status_t moe_reduce_map(const uint16_t* y, const float* topk_w, const int32_t* topk_ids,
                                const int32_t* expert_map, int32_t num_experts, int32_t L, int64_t M, int32_t k,
                                int32_t H, uint16_t* out, void* stream);

/* ------------------------------------------------------------------------- */
/* The whole layer                                                           */
/* [P1 Modification: gate/up GEMM -> fused SwiGLU + FP8 quant -> down GEMM;   */
/*  P4: moe_reduce; P2 Changes: route preparation]                            */
/* ------------------------------------------------------------------------- */

/* Number of stages (kernel launches, route preparation counted as one) a
 * fused_moe_block_fp8 call with these sizes and options makes on the current
 * device, and, when names is non-NULL, up to cap stage names (static strings)
 * in order.  The few-token path has two stages ("token_gate_up_swiglu",
 * "token_down_reduce"); the small-batch path two ("decode_gate_up_swiglu", "decode_down_reduce"); the
 * general path five ("route_prepare_quant", "gate_up_gemm",
 * "silu_and_mul_quant", "down_gemm", "moe_reduce"): route preparation's first
 * launch also quantises the input, except where one workgroup sorts for more
 * than 512 local experts, where it is six ("route_prepare", "quant_fp8", ...).
 * Returns -1 for arguments fused_moe_block_fp8 would reject. */
int32_t fused_moe_block_fp8_stages(int64_t M, int32_t H, int32_t k, int32_t E, int32_t I,
                                   const bfp8moe_opts_t* opts, const char** names, int32_t cap);

/* Workspace (bytes) fused_moe_block_fp8 needs for these sizes and options. */
size_t fused_moe_block_fp8_workspace_size(int64_t M, int32_t H, int32_t k, int32_t E, int32_t I,
                                          const bfp8moe_opts_t* opts);

/* hidden [M, H] BF16; topk_ids [M, k] int32 global expert ids (masked as
 * described above); topk_w [M, k] fp32 router weights;
 * w13 [L, 2I, H] E4M3FN (rows [0, I) gate, [I, 2I) up) with
 * w13_scale [L, 2I/128, H/128]; w2 [L, H, I] E4M3FN with w2_scale
 * [L, H/128, I/128]; L = opts->local_num_experts (or E).
 * out [M, H] BF16 = moe_reduce over routes of
 *   down( silu_and_mul_quant( gate_up( quant_fp8(hidden) ) ) ).
 * The hidden states and the SwiGLU output are both quantised with
 * opts->scale_fmt.  H and I must be positive multiples of 128.  A shared
 * expert can ride along as routes: split its width into experts of width I
 * (stored after the routed ones) and give every token those ids with weight 1
 * [P3: the shared expert runs beside the routed layer]; the few-token path
 * takes up to 16 routes per token.  ws: device
 * workspace of at least fused_moe_block_fp8_workspace_size() bytes, 256-byte
 * aligned; its contents need no initialisation and are not kept between
 * calls.  Calls that share a workspace must not run concurrently.  opts: host
 * pointer (NULL = defaults).
 * Three implementations, chosen by shape unless a test flag forces one:
 *   few tokens (M <= 32, k <= 16, H <= 8192, I in {128, 256, 512}; the
 *     default up to 15 tokens, 12 with per-channel weight scales, 8 with
 *     MXFP4 weights): two matrix-vector kernels -- input
 *     quantisation, gate/up GEMM and SwiGLU per route (M x k x I/8
 *     workgroups; each route reads its expert's rows), then the SwiGLU
 *     output's quantisation, down GEMM and moe_reduce per token and block of
 *     output rows (about 256 workgroups per token), each issuing its down
 *     weight loads as soon as it has read the routing;
 *   small batch (M <= 8, k <= 8, H <= 8192, I <= 512): two kernels -- gate/up
 *     GEMM with route grouping, input quantisation and SwiGLU fused; then the
 *     SwiGLU output's quantisation, down GEMM and moe_reduce fused;
 *   general: route prep (its first launch also quant_fp8 of the hidden
 *     states) -> grouped GEMM -> silu_and_mul_quant_fp8 -> grouped GEMM ->
 *     moe_reduce.
 * Forcing a path on a shape outside its limits returns
 * BFP8MOE_ERR_UNSUPPORTED. */
bfp8moe_status_t fused_moe_block_fp8(const uint16_t* hidden, int64_t M, int32_t H, const int32_t* topk_ids,
                                     const float* topk_w, int32_t k, const uint8_t* w13, const float* w13_scale,
                                     const uint8_t* w2, const float* w2_scale, int32_t E, int32_t I,
                                     const bfp8moe_opts_t* opts, uint16_t* out, void* ws, size_t ws_bytes,
                                     void* stream);

/* The layer with MXFP4 weights (see bfp8moe_weight_scale_t): arguments as
 * fused_moe_block_fp8 with w13 [L, 2I, H/2], w13_scale [L, 2I, H/32], w2
 * [L, H, I/2], w2_scale [L, H, I/32] (E8M0 bytes, 8-byte aligned).  opts is
 * required and must have weight_scale_mode BFP8MOE_WEIGHT_MXFP4; the
 * workspace is fused_moe_block_fp8_workspace_size with the same opts.  Stages:
 * "route_prepare_quant", "gate_up_gemm_mxfp4", "silu_and_mul_quant",
 * "down_gemm_mxfp4", "moe_reduce" (a separate "quant_fp8" where route
 * preparation cannot carry it). */
bfp8moe_status_t fused_moe_mxfp4(const uint16_t* hidden, int64_t M, int32_t H, const int32_t* topk_ids,
                                 const float* topk_w, int32_t k, const uint8_t* w13, const uint8_t* w13_scale,
                                 const uint8_t* w2, const uint8_t* w2_scale, int32_t E, int32_t I,
                                 const bfp8moe_opts_t* opts, uint16_t* out, void* ws, size_t ws_bytes,
                                 void* stream);

/* The layer with its router: moe_router_topk on router_logits [M, E] fp32
 * (score_fn, router_bias, renormalize, routed_scale as there) -- or, with
 * n_group > 1, moe_router_noaux_tc (n_group groups keeping topk_group; sigmoid
 * scoring) -- writing the routing to topk_ids [M, k] / topk_w [M, k]
 * (caller-owned outputs), then fused_moe_block_fp8 on it; same results as
 * the two calls in a row.
 * [P2 Changes: the fused single-group top-k router feeds the MoE layer;
 *  Reviewed changes: route_noaux_tc.py]
 * On the few-token path with E <= 256 and at most 4 tokens the router is
 * folded into the layer's first kernel (one launch fewer): each gate/up
 * workgroup ranks its token's logits itself.  With
 * BFP8MOE_FLAG_ROUTER_IN_ROUTE_PREP in opts->flags the general path does the
 * same inside route preparation's launch (up to 64 tokens).  Elsewhere the
 * router runs as its own launch first.  Takes
 * the workspace of fused_moe_block_fp8_workspace_size for the same sizes and
 * options; opts must not set stage events or a stage selection. */
bfp8moe_status_t fused_moe_block_fp8_routed(const uint16_t* hidden, int64_t M, int32_t H, const float* router_logits,
                                            const float* router_bias, int32_t score_fn, int32_t renormalize,
                                            double routed_scale, int32_t n_group, int32_t topk_group, int32_t k,
                                            int32_t* topk_ids, float* topk_w,
                                            const uint8_t* w13, const float* w13_scale, const uint8_t* w2,
                                            const float* w2_scale, int32_t E, int32_t I, const bfp8moe_opts_t* opts,
                                            uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * fused_moe_block_fp8 with the same arguments and results, whose workspace is
 * a device array the library holds, BFP8MOE_NOALLOC_SCRATCH_BYTES per GPU for
 * the life of the process (its address is looked up on the first call on each
 * device).  The call allocates nothing; the caller still passes inputs and
 * the output.  A call whose workspace (fused_moe_block_fp8_workspace_size)
 * exceeds the limit returns BFP8MOE_ERR_WORKSPACE, having launched nothing.
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (different streams, different host threads) race and must be
 * serialised by the caller.  The array needs no initialisation and keeps the
 * last call's intermediates. */
#define BFP8MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
bfp8moe_status_t fused_moe_block_fp8_noalloc(const uint16_t* hidden, int64_t M, int32_t H, const int32_t* topk_ids,
                                             const float* topk_w, int32_t k, const uint8_t* w13,
                                             const float* w13_scale, const uint8_t* w2, const float* w2_scale,
                                             int32_t E, int32_t I, const bfp8moe_opts_t* opts, uint16_t* out,
                                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BFP8MOE_H */
