/*
 * bfp8moe_oracle.c -- plain, slow CPU oracle for the block-FP8 fused MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file: only the test-suite, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant with the
 * HIP library; both sides receive the same seeded input bytes and nothing else.
 *
 * Sources (web pages; cited by title and section):
 *   [P1] lmdeploy PR "Perf/pytorch block fp8 moe decode"
 *   [P2] lmdeploy PR "perf(pytorch): optimize compact blocked FP8 MoE and route
 *        preparation"
 *   [P3] vLLM PR "[Kernel][Perf] Fuse clamped MoE activation and UE8M0 FP8 block
 *        quantization"
 *   [P4] lmdeploy PR "Moe Reduce kernel"
 *
 * Precision policy.  Steps whose floating-point result decides an integer (an
 * FP8 code, a scale) or whose output precision the pages fix (BF16 activation
 * after SwiGLU, fp32 moe_reduce accumulation) are computed in IEEE fp32 with the
 * operation order written below, no contraction (build with -ffp-contract=off).
 * The two GEMMs are computed from their definition in fp64: the per-128-group
 * sums of E4M3 products are exact in fp64, scale products and the sum over
 * groups are fp64, and the result is rounded once to BF16.
 *
 * Pins (see tests/test_oracle_*.py): every function here is checked against
 * brute force, closed forms or invariants that do not reuse this code.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <fenv.h>

#define ORACLE_GROUP 128          /* quantisation group / weight block edge [P3 Purpose: block shape 128] */
#define ORACLE_E4M3_MAX 448.0f    /* largest finite OCP E4M3FN value */

/* Floor applied to a group's amax before the scale is formed.  The pages do
 * not state one; this value only changes the scale stored for an all-zero
 * group (reading documented with the oracle). */
#define ORACLE_AMAX_EPS 1e-10f

enum { ORACLE_SCALE_FP32 = 0, ORACLE_SCALE_UE8M0 = 1 };

/* ------------------------------------------------------------------------- */
/* BF16 <-> fp32                                                             */
/* ------------------------------------------------------------------------- */

static float f32_from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

double oracle_bf16_to_f64(uint16_t h) { return (double)f32_from_bits((uint32_t)h << 16); }
static float bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* Round an fp32 value to BF16, nearest-even.  NaN becomes a quiet NaN with
 * the sign kept; overflow rounds to infinity as IEEE rounding does. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t b = bits_from_f32(f);
    if (isnan(f)) return (uint16_t)(((b >> 16) & 0x8000u) | 0x7FC0u);
    uint32_t lsb = (b >> 16) & 1u;
    b += 0x7FFFu + lsb;
    return (uint16_t)(b >> 16);
}

/* Round a double straight to BF16, nearest-even, in one rounding.  Used for
 * the GEMM outputs, whose value is formed in fp64. */
uint16_t oracle_f64_to_bf16(double x)
{
    if (isnan(x)) return 0x7FC0u;
    if (x == 0.0) return signbit(x) ? 0x8000u : 0x0000u;
    uint16_t sign = signbit(x) ? 0x8000u : 0;
    double a = fabs(x);
    int e;
    frexp(a, &e);                 /* a = f * 2^e, f in [0.5, 1) */
    int ue = e - 1;               /* a in [2^ue, 2^(ue+1)) */
    if (ue < -126) ue = -126;     /* subnormal range: fixed quantum 2^-133 */
    /* BF16 has 8 significant bits: quantum is 2^(ue-7). */
    double q = ldexp(a, -(ue - 7));
    double r = nearbyint(q);      /* default mode: nearest, ties to even */
    double v = ldexp(r, ue - 7);
    /* v is exactly representable as fp32 unless it overflowed. */
    if (v > 3.3895313892515355e38) return (uint16_t)(sign | 0x7F80u);
    float vf = (float)v;
    return (uint16_t)(sign | (uint16_t)(bits_from_f32(vf) >> 16));
}

/* ------------------------------------------------------------------------- */
/* OCP E4M3FN codec                                                          */
/* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no infinities, the  */
/* all-ones exponent+mantissa pattern is NaN, largest finite magnitude 448.   */
/* ------------------------------------------------------------------------- */

/* Decode one E4M3FN byte to its exact value. */
double oracle_e4m3_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);              /* subnormal: m * 2^-9 */
    else v = ldexp(1.0 + m / 8.0, e - 7);              /* normal */
    return s ? -v : v;
}

/* Encode an fp32 value as E4M3FN: round to nearest, ties to even mantissa;
 * magnitudes at or above 448 saturate to 448; NaN maps to 0x7F with the sign
 * kept; the sign of zero is kept.  Rounding is done on the exact value in fp64. */
uint8_t oracle_e4m3_encode(float x)
{
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    if (isnan(x)) return (uint8_t)(sign | 0x7F);
    double a = fabs((double)x);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: quantum 2^-9; m == 8 carries into the smallest normal */
        int m = (int)nearbyint(ldexp(a, 9));
        return (uint8_t)(sign | m);
    }
    int e;
    double f = frexp(a, &e);      /* a = f * 2^e, f in [0.5, 1) */
    int ue = e - 1;               /* a = (2f) * 2^ue, 2f in [1, 2) */
    int m = (int)nearbyint((2.0 * f - 1.0) * 8.0);
    if (m == 8) { m = 0; ue += 1; }
    return (uint8_t)(sign | ((ue + 7) << 3) | m);
}

/* ------------------------------------------------------------------------- */
/* Group-128 dynamic activation quantisation ("quant_fp8")                    */
/* [P1 Motivation: quant_fp8 after the BF16 intermediate]                     */
/* [P4 Pull request overview: scale_fmt 'ue8m0' rounds scales]               */
/* [P3 Purpose: dynamic E4M3 block quantisation with UE8M0 scales]            */
/* ------------------------------------------------------------------------- */

/* Scale of one group from its amax.  fp32: amax/448 by one IEEE division.
 * UE8M0: that value rounded UP to a power of two, read off its fp32 bit
 * fields (ceil of log2). */
float oracle_group_scale(float amax, int fmt)
{
    float a = amax > ORACLE_AMAX_EPS ? amax : ORACLE_AMAX_EPS;
    float v = a / ORACLE_E4M3_MAX;
    if (fmt == ORACLE_SCALE_UE8M0) {
        uint32_t b = bits_from_f32(v);
        uint32_t ex = (b >> 23) & 0xFFu;
        uint32_t mant = b & 0x7FFFFFu;
        if (mant != 0) ex += 1;
        return f32_from_bits(ex << 23);
    }
    return v;
}

/* Quantise one row of K values given as fp32 (each exactly a BF16 value). */
static void quant_row_f32(const float* x, int K, int fmt, uint8_t* q, float* s)
{
    for (int g = 0; g < K / ORACLE_GROUP; g++) {
        const float* xg = x + (size_t)g * ORACLE_GROUP;
        float amax = 0.0f;
        for (int i = 0; i < ORACLE_GROUP; i++) {
            float a = fabsf(xg[i]);
            if (a > amax) amax = a;
        }
        float sc = oracle_group_scale(amax, fmt);
        s[g] = sc;
        for (int i = 0; i < ORACLE_GROUP; i++)
            q[(size_t)g * ORACLE_GROUP + i] = oracle_e4m3_encode(xg[i] / sc);
    }
}

/* x: [rows, K] BF16; q: [rows, K] E4M3; s: [rows, K/128] fp32. */
void oracle_quant_fp8(const uint16_t* x, int64_t rows, int K, int fmt, uint8_t* q, float* s)
{
    float* row = (float*)malloc(sizeof(float) * (size_t)K);
    for (int64_t r = 0; r < rows; r++) {
        for (int i = 0; i < K; i++) row[i] = bf16_to_f32(x[(size_t)r * K + i]);
        quant_row_f32(row, K, fmt, q + (size_t)r * K, s + (size_t)r * (K / ORACLE_GROUP));
    }
    free(row);
}

/* ------------------------------------------------------------------------- */
/* SwiGLU with optional finite clamp                                          */
/* [P1 Motivation: gate/up GEMM -> silu_and_mul -> BF16 intermediate]         */
/* [P3 Purpose: finite SwiGLU clamping; BF16 SiLU and gated multiplication]   */
/* ------------------------------------------------------------------------- */

/* exp(x) rounded to fp32, computed as a double then rounded once. */
float oracle_exp_rn(float x) { return (float)exp((double)x); }

/* One BF16 output of SwiGLU.  The gate is clamped from above and the up value
 * to [-limit, limit] when the limit is finite.  silu(g) = g / (1 + exp(-g)),
 * then times up, each step an fp32 operation, and one rounding to BF16. */
uint16_t oracle_swiglu_one(uint16_t gate, uint16_t up, float clamp_limit)
{
    float g = bf16_to_f32(gate);
    float u = bf16_to_f32(up);
    if (isfinite(clamp_limit)) {
        if (g > clamp_limit) g = clamp_limit;
        if (u > clamp_limit) u = clamp_limit;
        if (u < -clamp_limit) u = -clamp_limit;
    }
    float e = oracle_exp_rn(-g);
    float d = 1.0f + e;
    float sg = g / d;
    float h = sg * u;
    return oracle_f32_to_bf16(h);
}

/* gate_up: [rows, 2I] BF16 (gate columns 0..I-1, up columns I..2I-1);
 * out: [rows, I] BF16. */
void oracle_silu_and_mul(const uint16_t* gate_up, int64_t rows, int I, float clamp_limit, uint16_t* out)
{
    for (int64_t r = 0; r < rows; r++) {
        const uint16_t* gu = gate_up + (size_t)r * 2 * I;
        for (int i = 0; i < I; i++)
            out[(size_t)r * I + i] = oracle_swiglu_one(gu[i], gu[I + i], clamp_limit);
    }
}

/* A row is processed unless its expert id is negative or, when an expert map
 * is given, the map sends it to a negative (non-local) entry.
 * [P3 Purpose: optional filtering of invalid or non-local expert rows] */
static int row_is_live(const int32_t* row_expert_ids, const int32_t* expert_map, int E, int64_t r)
{
    if (!row_expert_ids) return 1;
    int32_t id = row_expert_ids[r];
    if (id < 0 || id >= E) return 0;
    if (expert_map && expert_map[id] < 0) return 0;
    return 1;
}

/* Fused SwiGLU(+clamp) then group-128 quantisation of each live row.  Rows that
 * are filtered out are not written at all.  By construction this equals
 * quant_fp8(silu_and_mul(x)) on live rows
 * [P1 Correctness and validation; P3 Correctness and validation]. */
void oracle_silu_and_mul_quant_fp8(const uint16_t* gate_up, int64_t rows, int I,
                                   const int32_t* row_expert_ids, const int32_t* expert_map, int E,
                                   float clamp_limit, int fmt, uint8_t* q, float* s)
{
    uint16_t* act = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)I);
    float* actf = (float*)malloc(sizeof(float) * (size_t)I);
    for (int64_t r = 0; r < rows; r++) {
        if (!row_is_live(row_expert_ids, expert_map, E, r)) continue;
        oracle_silu_and_mul(gate_up + (size_t)r * 2 * I, 1, I, clamp_limit, act);
        for (int i = 0; i < I; i++) actf[i] = bf16_to_f32(act[i]);
        quant_row_f32(actf, I, fmt, q + (size_t)r * I, s + (size_t)r * (I / ORACLE_GROUP));
    }
    free(act);
    free(actf);
}

/* ------------------------------------------------------------------------- */
/* Route preparation: routes sorted by (local) expert, plus compact blocks     */
/* [P2 Changes: shared route preparation; sorted-indices and compact-blocks    */
/*  contracts; Suppressed comments: expert_offset / local_num_experts slice]   */
/* [P1 Modification, Active-expert block scheduling: blocks only for experts   */
/*  that receive tokens]                                                       */
/* ------------------------------------------------------------------------- */

int64_t oracle_max_blocks(int64_t R, int L, int block_m)
{
    int64_t d = R < L ? R : L;
    return (R + d * (block_m - 1)) / block_m;
}

/* Route r = t*k + j.  A route whose expert id minus expert_offset lies outside
 * [0, L) is dropped.  Kept routes are ordered by local expert, ties by route
 * index (a stable counting sort).  Entries of sorted_routes past the kept
 * routes are -1.  For every expert with c > 0 routes, ceil(c / block_m) blocks
 * follow in expert order, each naming its local expert and its first position
 * in sorted_routes; unused block slots up to max_blocks hold -1.
 * Returns the number of blocks (also stored in *num_blocks). */
int64_t oracle_route_prepare(const int32_t* topk_ids, int64_t R, int expert_offset, int L, int block_m,
                             int32_t* sorted_routes, int32_t* expert_offsets,
                             int32_t* block_expert, int32_t* block_start, int64_t max_blocks,
                             int32_t* num_blocks)
{
    int64_t* counts = (int64_t*)calloc((size_t)L, sizeof(int64_t));
    for (int64_t r = 0; r < R; r++) {
        int64_t e = (int64_t)topk_ids[r] - expert_offset;
        if (e >= 0 && e < L) counts[e]++;
    }
    int64_t acc = 0;
    for (int e = 0; e < L; e++) { expert_offsets[e] = (int32_t)acc; acc += counts[e]; }
    expert_offsets[L] = (int32_t)acc;
    for (int64_t i = 0; i < R; i++) sorted_routes[i] = -1;
    int64_t* fill = (int64_t*)calloc((size_t)L, sizeof(int64_t));
    for (int64_t r = 0; r < R; r++) {          /* ascending r: stable */
        int64_t e = (int64_t)topk_ids[r] - expert_offset;
        if (e >= 0 && e < L) {
            sorted_routes[expert_offsets[e] + fill[e]] = (int32_t)r;
            fill[e]++;
        }
    }
    int64_t nb = 0;
    if (block_expert && block_start) {
        for (int64_t b = 0; b < max_blocks; b++) { block_expert[b] = -1; block_start[b] = -1; }
        for (int e = 0; e < L; e++) {
            for (int64_t i = 0; i * block_m < counts[e]; i++) {
                block_expert[nb] = e;
                block_start[nb] = (int32_t)(expert_offsets[e] + i * block_m);
                nb++;
            }
        }
    } else {
        for (int e = 0; e < L; e++) nb += (counts[e] + block_m - 1) / block_m;
    }
    if (num_blocks) *num_blocks = (int32_t)nb;
    free(counts);
    free(fill);
    return nb;
}

/* ------------------------------------------------------------------------- */
/* Block-FP8 W8A8 GEMM of one activation row against one expert's weights      */
/* [P3 Purpose: FP8 W8A8 block shape [128, 128]]                               */
/* [P1 Motivation: gate/up GEMM and down-projection on FP8 inputs]             */
/* ------------------------------------------------------------------------- */

/* One output of the block-FP8 GEMM before its rounding:
 *   sum_g (a_s[g] * w_s[g]) * sum_{i in group g} dec(a[i]) * dec(w[i])
 * ad: [K] decoded activation values; a_s: [K/128]; w: one weight row [K]
 * (E4M3 codes); w_s: that row's [K/128] block scales.  All arithmetic is fp64:
 * each product of two E4M3 values has at most 8 significant bits and a group
 * sum of 128 of them is exact, so only the scale products and the sum over
 * groups round, at 2^-53.  When abs_sum is non-NULL it receives
 * sum_g |a_s[g] * w_s[g]| * sum_i |dec(a[i]) * dec(w[i])|, the magnitude that
 * bounds the rounding error of any fp32 evaluation of the same sum. */
static double gemm_dot(const double* ad, const float* a_s, const uint8_t* w, const float* w_s, int G,
                       double* abs_sum)
{
    double acc = 0.0, mag = 0.0;
    for (int g = 0; g < G; g++) {
        double p = 0.0, pa = 0.0;
        for (int i = g * ORACLE_GROUP; i < (g + 1) * ORACLE_GROUP; i++) {
            double t = ad[i] * oracle_e4m3_decode(w[i]);
            p += t;
            pa += fabs(t);
        }
        double c = (double)a_s[g] * (double)w_s[g];
        acc += c * p;
        mag += fabs(c) * pa;
    }
    if (abs_sum) *abs_sum = mag;
    return acc;
}

/* out[n] = bf16( sum_g  (a_s[g] * w_s[n/128][g]) * sum_{i in group g} dec(a[i]) * dec(W[n][i]) )
 * a: [K] E4M3, a_s: [K/128]; W: [N, K] E4M3 (row n = output n, K contiguous);
 * w_s: [N/128, K/128].  The sum is gemm_dot's, rounded once to BF16.  When
 * acc_out / abs_out are non-NULL they receive the unrounded value and its
 * magnitude bound for each n.  Output rows are independent: OpenMP spreads
 * them over the host's threads. */
static void gemm_row_ex(const uint8_t* a, const float* a_s, const uint8_t* W, const float* w_s,
                        int N, int K, uint16_t* out, double* acc_out, double* abs_out)
{
    int G = K / ORACLE_GROUP;
    double* ad = (double*)malloc(sizeof(double) * (size_t)K);
    for (int i = 0; i < K; i++) ad[i] = oracle_e4m3_decode(a[i]);
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; n++) {
        double mag;
        double acc = gemm_dot(ad, a_s, W + (size_t)n * K, w_s + (size_t)(n / ORACLE_GROUP) * G, G, &mag);
        if (out) out[n] = oracle_f64_to_bf16(acc);
        if (acc_out) acc_out[n] = acc;
        if (abs_out) abs_out[n] = mag;
    }
    free(ad);
}

static void gemm_row(const uint8_t* a, const float* a_s, const uint8_t* W, const float* w_s,
                     int N, int K, uint16_t* out)
{
    gemm_row_ex(a, a_s, W, w_s, N, K, out, NULL, NULL);
}

/* Grouped GEMM over routes.  For every route r with local expert e in [0, L):
 *   C[r, :] = gemm_row(A[r / a_row_div], A_s[r / a_row_div], B[e], B_s[e]).
 * a_row_div is top-k for the gate/up projection (one activation row per token
 * feeds its k routes) and 1 for the down projection (one row per route).
 * Rows of C for dropped routes are left untouched. */
void oracle_grouped_gemm(const uint8_t* A, const float* A_s, int a_row_div,
                         const uint8_t* B, const float* B_s, int N, int K,
                         const int32_t* topk_ids, int64_t R, int expert_offset, int L,
                         uint16_t* C)
{
    int G = K / ORACLE_GROUP;
    for (int64_t r = 0; r < R; r++) {
        int64_t e = (int64_t)topk_ids[r] - expert_offset;
        if (e < 0 || e >= L) continue;
        int64_t arow = r / a_row_div;
        gemm_row(A + (size_t)arow * K, A_s + (size_t)arow * G,
                 B + (size_t)e * N * K, B_s + (size_t)e * (N / ORACLE_GROUP) * G,
                 N, K, C + (size_t)r * N);
    }
}

/* The same grouped GEMM before its BF16 rounding: acc[r, n] is gemm_dot's fp64
 * value and mag[r, n] its magnitude bound (both [R, N] doubles; rows of
 * dropped routes untouched).  Test infrastructure: a GPU result whose fp32
 * accumulation may land on either side of a BF16 rounding boundary is told
 * apart from a wrong one by these two numbers. */
void oracle_grouped_gemm_f64(const uint8_t* A, const float* A_s, int a_row_div,
                             const uint8_t* B, const float* B_s, int N, int K,
                             const int32_t* topk_ids, int64_t R, int expert_offset, int L,
                             double* acc, double* mag)
{
    int G = K / ORACLE_GROUP;
    for (int64_t r = 0; r < R; r++) {
        int64_t e = (int64_t)topk_ids[r] - expert_offset;
        if (e < 0 || e >= L) continue;
        int64_t arow = r / a_row_div;
        gemm_row_ex(A + (size_t)arow * K, A_s + (size_t)arow * G,
                    B + (size_t)e * N * K, B_s + (size_t)e * (N / ORACLE_GROUP) * G,
                    N, K, NULL, acc + (size_t)r * N, mag + (size_t)r * N);
    }
}

/* ------------------------------------------------------------------------- */
/* W8A8 variant: per-token activation scales, per-output-channel weight scales */
/* [P2 Reviewed changes: w8a8.py, the static FP8 MoE backend; P4 Pull request  */
/*  overview: the W8A8 fused MoE ends with moe_reduce too]                     */
/* The pages name the variant only.  Reading: the same pipeline with one scale */
/* per activation row (the row's amax / 448 over all K, or a given static      */
/* per-tensor scale) and one fp32 scale per weight row (output channel).       */
/* ------------------------------------------------------------------------- */

void oracle_moe_reduce(const uint16_t* y, const float* w, const int32_t* topk_ids, int expert_offset, int L,
                       int64_t M, int k, int H, uint16_t* out);

/* One row's scale: static_scale when > 0, else the group-scale formula applied
 * to the amax over the whole row. */
static float row_scale(const float* x, int K, int fmt, float static_scale)
{
    if (static_scale > 0.0f) return static_scale;
    float amax = 0.0f;
    for (int i = 0; i < K; i++) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    return oracle_group_scale(amax, fmt);
}

/* x: [rows, K] BF16 -> q [rows, K] E4M3 (saturating) and s [rows] fp32. */
void oracle_quant_fp8_rows(const uint16_t* x, int64_t rows, int K, int fmt, float static_scale, uint8_t* q, float* s)
{
    float* row = (float*)malloc(sizeof(float) * (size_t)K);
    for (int64_t r = 0; r < rows; r++) {
        for (int i = 0; i < K; i++) row[i] = bf16_to_f32(x[(size_t)r * K + i]);
        float sc = row_scale(row, K, fmt, static_scale);
        s[r] = sc;
        for (int i = 0; i < K; i++) q[(size_t)r * K + i] = oracle_e4m3_encode(row[i] / sc);
    }
    free(row);
}

/* Fused SwiGLU + per-row quantisation of each live row (rows filtered as in
 * oracle_silu_and_mul_quant_fp8 are not written). */
void oracle_silu_and_mul_quant_fp8_rows(const uint16_t* gate_up, int64_t rows, int I,
                                        const int32_t* row_expert_ids, const int32_t* expert_map, int E,
                                        float clamp_limit, int fmt, float static_scale, uint8_t* q, float* s)
{
    uint16_t* act = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)I);
    for (int64_t r = 0; r < rows; r++) {
        if (!row_is_live(row_expert_ids, expert_map, E, r)) continue;
        oracle_silu_and_mul(gate_up + (size_t)r * 2 * I, 1, I, clamp_limit, act);
        oracle_quant_fp8_rows(act, 1, I, fmt, static_scale, q + (size_t)r * I, s + r);
    }
    free(act);
}

/* out[n] = bf16(a_s * w_s[n] * sum_k dec(a_k) dec(W[n, k])), all in fp64 (the
 * code sum is exact up to K = 2^24 terms); acc_out / abs_out as gemm_row_ex. */
static void gemm_row_channel(const uint8_t* a, float a_s, const uint8_t* W, const float* w_s, int N, int K,
                             uint16_t* out, double* acc_out, double* abs_out)
{
    double* ad = (double*)malloc(sizeof(double) * (size_t)K);
    for (int i = 0; i < K; i++) ad[i] = oracle_e4m3_decode(a[i]);
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; n++) {
        const uint8_t* wr = W + (size_t)n * K;
        double p = 0.0, pa = 0.0;
        for (int i = 0; i < K; i++) {
            double t = ad[i] * oracle_e4m3_decode(wr[i]);
            p += t;
            pa += fabs(t);
        }
        double c = (double)a_s * (double)w_s[n];
        if (out) out[n] = oracle_f64_to_bf16(c * p);
        if (acc_out) acc_out[n] = c * p;
        if (abs_out) abs_out[n] = fabs(c) * pa;
    }
    free(ad);
}

/* Grouped GEMM with per-row activation scales A_s [rows] and per-channel weight
 * scales B_s [L, N]; acc / mag (both NULL, or both [R, N]) receive the
 * unrounded values and magnitudes instead of C. */
void oracle_grouped_gemm_channel(const uint8_t* A, const float* A_s, int a_row_div, const uint8_t* B,
                                 const float* B_s, int N, int K, const int32_t* topk_ids, int64_t R,
                                 int expert_offset, int L, uint16_t* C, double* acc, double* mag)
{
    for (int64_t r = 0; r < R; r++) {
        int64_t e = (int64_t)topk_ids[r] - expert_offset;
        if (e < 0 || e >= L) continue;
        int64_t arow = r / a_row_div;
        gemm_row_channel(A + (size_t)arow * K, A_s[arow], B + (size_t)e * N * K, B_s + (size_t)e * N, N, K,
                         C ? C + (size_t)r * N : NULL, acc ? acc + (size_t)r * N : NULL,
                         mag ? mag + (size_t)r * N : NULL);
    }
}

/* The whole W8A8 layer: w13_s [L, 2I], w2_s [L, H]; a1_static / a2_static > 0
 * are static scales of the hidden states / the SwiGLU output, else per-row
 * dynamic ones (scale_fmt).  Intermediates as oracle_fused_moe (act_s is
 * [M*k] here). */
void oracle_fused_moe_w8a8(const uint16_t* hidden, int64_t M, int H, const int32_t* topk_ids, const float* topk_w,
                           int k, const uint8_t* w13, const float* w13_s, const uint8_t* w2, const float* w2_s,
                           int expert_offset, int L, int I, int scale_fmt, float a1_static, float a2_static,
                           float clamp_limit, uint16_t* out, uint16_t* h13_out, uint8_t* q_out, float* s_out,
                           uint16_t* y_out)
{
    uint8_t* aq = (uint8_t*)malloc((size_t)H);
    uint16_t* h13 = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)2 * I);
    uint8_t* q = (uint8_t*)malloc((size_t)I);
    uint16_t* y = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)k * H);
    float* w = (float*)malloc(sizeof(float) * (size_t)k);
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    for (int64_t t = 0; t < M; t++) {
        float as, s;
        oracle_quant_fp8_rows(hidden + (size_t)t * H, 1, H, scale_fmt, a1_static, aq, &as);
        for (int j = 0; j < k; j++) {
            int64_t r = t * k + j;
            ids[j] = topk_ids[r];
            w[j] = topk_w[r];
            int64_t e = (int64_t)topk_ids[r] - expert_offset;
            if (e < 0 || e >= L) continue;
            gemm_row_channel(aq, as, w13 + (size_t)e * 2 * I * H, w13_s + (size_t)e * 2 * I, 2 * I, H, h13, NULL,
                             NULL);
            oracle_silu_and_mul_quant_fp8_rows(h13, 1, I, NULL, NULL, 0, clamp_limit, scale_fmt, a2_static, q, &s);
            gemm_row_channel(q, s, w2 + (size_t)e * H * I, w2_s + (size_t)e * H, H, I, y + (size_t)j * H, NULL,
                             NULL);
            if (h13_out) memcpy(h13_out + (size_t)r * 2 * I, h13, sizeof(uint16_t) * 2 * I);
            if (q_out) memcpy(q_out + (size_t)r * I, q, (size_t)I);
            if (s_out) s_out[r] = s;
            if (y_out) memcpy(y_out + (size_t)r * H, y + (size_t)j * H, sizeof(uint16_t) * H);
        }
        oracle_moe_reduce(y, w, ids, expert_offset, L, 1, k, H, out + (size_t)t * H);
    }
    free(aq); free(h13); free(q); free(y); free(w); free(ids);
}

/* ------------------------------------------------------------------------- */
/* MXFP4-weight variant                                                        */
/* [P2 Reviewed changes: v4_fp4_grouped_gemm.py, v4_swiglu_quant.py and the    */
/*  v4 FP4 fused MoE backend; P3 Matched GLM serving A/B: MXFP4 is the default */
/*  weight format of the DeepSeek-V4 checkpoint it names]                      */
/* The pages name the variant only.  Reading, from the OCP Microscaling (MX)   */
/* Formats specification v1.0: a weight row is a sequence of E2M1 elements,    */
/* two to a byte with the even-indexed element in the low four bits, and each  */
/* run of 32 consecutive elements along K shares one E8M0 scale byte.  The     */
/* activations stay those of the block-FP8 layer (E4M3 with one scale per 128  */
/* along K; the SwiGLU quantisation is P3's), and every other step is          */
/* unchanged.                                                                  */
/* ------------------------------------------------------------------------- */

#define ORACLE_MX_BLOCK 32

/* E2M1: sign in bit 3, a 2-bit exponent (bias 1) in bits 2..1, one mantissa
 * bit; exponent 0 holds 0 and the subnormal 0.5.  Every code is finite. */
double oracle_e2m1_decode(uint8_t c)
{
    int sign = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -v : v;
}

/* E8M0: 2^(e - 127); the byte 255 is NaN. */
double oracle_e8m0_decode(uint8_t e) { return e == 255 ? NAN : ldexp(1.0, (int)e - 127); }

/* Element i of a packed E2M1 row. */
static uint8_t e2m1_at(const uint8_t* row, int i) { return (uint8_t)((row[i / 2] >> (4 * (i & 1))) & 15); }

/* sum_g a_s[g] * sum_{b in group g} 2^(e_b - 127) * sum_{i in block b} dec(a[i]) * dec(w[i])
 * for one packed weight row w ([K/2] bytes) with its scale bytes ws ([K/32]).
 * A block's sum of 32 products (each at most 5 significant bits) is exact in
 * fp64 and the E8M0 factor is a power of two; the activation-scale product and
 * the sums over blocks round at 2^-53.  abs_sum as in gemm_dot. */
static double gemm_dot_mx(const double* ad, const float* a_s, const uint8_t* w, const uint8_t* ws, int K,
                          double* abs_sum)
{
    double acc = 0.0, mag = 0.0;
    for (int b = 0; b < K / ORACLE_MX_BLOCK; b++) {
        double p = 0.0, pa = 0.0;
        for (int i = b * ORACLE_MX_BLOCK; i < (b + 1) * ORACLE_MX_BLOCK; i++) {
            double t = ad[i] * oracle_e2m1_decode(e2m1_at(w, i));
            p += t;
            pa += fabs(t);
        }
        double c = (double)a_s[(b * ORACLE_MX_BLOCK) / ORACLE_GROUP] * oracle_e8m0_decode(ws[b]);
        acc += c * p;
        mag += fabs(c) * pa;
    }
    if (abs_sum) *abs_sum = mag;
    return acc;
}

/* out[n] = bf16(gemm_dot_mx(a, W[n])) for W [N, K/2] packed rows and W_s
 * [N, K/32] scale bytes; acc_out / abs_out as gemm_row_ex. */
static void gemm_row_mx(const uint8_t* a, const float* a_s, const uint8_t* W, const uint8_t* W_s, int N, int K,
                        uint16_t* out, double* acc_out, double* abs_out)
{
    double* ad = (double*)malloc(sizeof(double) * (size_t)K);
    for (int i = 0; i < K; i++) ad[i] = oracle_e4m3_decode(a[i]);
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; n++) {
        double mag;
        double acc = gemm_dot_mx(ad, a_s, W + (size_t)n * (K / 2), W_s + (size_t)n * (K / ORACLE_MX_BLOCK), K, &mag);
        if (out) out[n] = oracle_f64_to_bf16(acc);
        if (acc_out) acc_out[n] = acc;
        if (abs_out) abs_out[n] = mag;
    }
    free(ad);
}

/* Grouped GEMM with MXFP4 weights B [L, N, K/2], B_s [L, N, K/32] and E4M3
 * activations A [rows, K] with group-128 scales A_s [rows, K/128]; routes and
 * outputs as oracle_grouped_gemm.  acc / mag (both NULL, or both [R, N])
 * receive the unrounded values and magnitudes instead of C. */
void oracle_grouped_gemm_mxfp4(const uint8_t* A, const float* A_s, int a_row_div, const uint8_t* B,
                               const uint8_t* B_s, int N, int K, const int32_t* topk_ids, int64_t R,
                               int expert_offset, int L, uint16_t* C, double* acc, double* mag)
{
    int G = K / ORACLE_GROUP;
    for (int64_t r = 0; r < R; r++) {
        int64_t e = (int64_t)topk_ids[r] - expert_offset;
        if (e < 0 || e >= L) continue;
        int64_t arow = r / a_row_div;
        gemm_row_mx(A + (size_t)arow * K, A_s + (size_t)arow * G, B + (size_t)e * N * (K / 2),
                    B_s + (size_t)e * N * (K / ORACLE_MX_BLOCK), N, K, C ? C + (size_t)r * N : NULL,
                    acc ? acc + (size_t)r * N : NULL, mag ? mag + (size_t)r * N : NULL);
    }
}

/* The whole layer with MXFP4 weights: w13 [L, 2I, H/2], w13_s [L, 2I, H/32],
 * w2 [L, H, I/2], w2_s [L, H, I/32]; everything else and the intermediates as
 * oracle_fused_moe (all tokens). */
void oracle_fused_moe_mxfp4(const uint16_t* hidden, int64_t M, int H, const int32_t* topk_ids,
                            const float* topk_w, int k, const uint8_t* w13, const uint8_t* w13_s,
                            const uint8_t* w2, const uint8_t* w2_s, int expert_offset, int L, int I, int scale_fmt,
                            float clamp_limit, uint16_t* out, uint16_t* h13_out, uint8_t* q_out, float* s_out,
                            uint16_t* y_out)
{
    int GH = H / ORACLE_GROUP, GI = I / ORACLE_GROUP;
    uint8_t* aq = (uint8_t*)malloc((size_t)H);
    float* as = (float*)malloc(sizeof(float) * (size_t)GH);
    uint16_t* h13 = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)2 * I);
    uint8_t* q = (uint8_t*)malloc((size_t)I);
    float* s = (float*)malloc(sizeof(float) * (size_t)GI);
    uint16_t* y = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)k * H);
    float* w = (float*)malloc(sizeof(float) * (size_t)k);
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    for (int64_t t = 0; t < M; t++) {
        oracle_quant_fp8(hidden + (size_t)t * H, 1, H, scale_fmt, aq, as);
        for (int j = 0; j < k; j++) {
            int64_t r = t * k + j;
            ids[j] = topk_ids[r];
            w[j] = topk_w[r];
            int64_t e = (int64_t)topk_ids[r] - expert_offset;
            if (e < 0 || e >= L) continue;
            gemm_row_mx(aq, as, w13 + (size_t)e * 2 * I * (H / 2), w13_s + (size_t)e * 2 * I * (H / ORACLE_MX_BLOCK),
                        2 * I, H, h13, NULL, NULL);
            oracle_silu_and_mul_quant_fp8(h13, 1, I, NULL, NULL, 0, clamp_limit, scale_fmt, q, s);
            gemm_row_mx(q, s, w2 + (size_t)e * H * (I / 2), w2_s + (size_t)e * H * (I / ORACLE_MX_BLOCK), H, I,
                        y + (size_t)j * H, NULL, NULL);
            if (h13_out) memcpy(h13_out + (size_t)r * 2 * I, h13, sizeof(uint16_t) * 2 * I);
            if (q_out) memcpy(q_out + (size_t)r * I, q, (size_t)I);
            if (s_out) memcpy(s_out + (size_t)r * GI, s, sizeof(float) * GI);
            if (y_out) memcpy(y_out + (size_t)r * H, y + (size_t)j * H, sizeof(uint16_t) * H);
        }
        oracle_moe_reduce(y, w, ids, expert_offset, L, 1, k, H, out + (size_t)t * H);
    }
    free(aq); free(as); free(h13); free(q); free(s); free(y); free(w); free(ids);
}

/* ------------------------------------------------------------------------- */
/* moe_reduce: top-k weighted sum back to token order                          */
/* [P4 Pull request overview: weights applied by a dedicated reduction]        */
/* [P4 review discussion: accumulation precision left to each kernel; fp32]    */
/* ------------------------------------------------------------------------- */

/* out[t, n] = bf16(acc), acc = 0 then, for j = 0..k-1 ascending over live
 * routes, acc = fmaf(w[t, j], y[t*k + j, n], acc).  A route is live when
 * topk_ids is NULL or its id minus expert_offset lies in [0, L).  A token with
 * no live route gives +0. */
void oracle_moe_reduce(const uint16_t* y, const float* w, const int32_t* topk_ids,
                       int expert_offset, int L, int64_t M, int k, int H, uint16_t* out)
{
    for (int64_t t = 0; t < M; t++) {
        for (int n = 0; n < H; n++) {
            float acc = 0.0f;
            for (int j = 0; j < k; j++) {
                int64_t r = t * k + j;
                if (topk_ids) {
                    int64_t e = (int64_t)topk_ids[r] - expert_offset;
                    if (e < 0 || e >= L) continue;
                }
                acc = fmaf(w[r], bf16_to_f32(y[(size_t)r * H + n]), acc);
            }
            out[(size_t)t * H + n] = oracle_f32_to_bf16(acc);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Single-group top-k router: router logits -> top-k expert ids and weights    */
/* [P2 Changes: fused single-group top-k router; renormalize option]           */
/* ------------------------------------------------------------------------- */

enum { ORACLE_SCORE_SOFTMAX = 0, ORACLE_SCORE_SIGMOID = 1 };

/* Sigmoid of an fp32 logit, computed in double and rounded once to fp32. */
float oracle_sigmoid_rn(float x) { return (float)(1.0 / (1.0 + exp(-(double)x))); }

/* The value an expert is ranked by.  Softmax is strictly increasing in the
 * logit, so ranking the exact probabilities is ranking the logits themselves.
 * Sigmoid scores are ranked as the fp32 score plus the optional per-expert
 * selection bias, one fp32 add (the bias steers which experts are chosen, not
 * their weights). */
static float router_key(const float* lg, const float* bias, int score_fn, int e)
{
    if (score_fn == ORACLE_SCORE_SOFTMAX) return lg[e];
    float s = oracle_sigmoid_rn(lg[e]);
    return bias ? s + bias[e] : s;
}

/* logits: [M, E] fp32; bias: [E] fp32 or NULL (sigmoid scoring only);
 * topk_ids: [M, k] int32; topk_w: [M, k] fp32.  For each token the k experts
 * with the largest keys are chosen one at a time, largest first; equal keys go
 * to the lower expert id.  Weights, in fp64 and rounded once to fp32:
 *   softmax: exp(l_j - m) / Z with m the largest logit, Z summed over the k
 *            chosen experts when renormalize is set, else over all E;
 *   sigmoid: 1 / (1 + exp(-l_j)), divided by the sum over the k chosen when
 *            renormalize is set;
 * both then times scale. */
void oracle_router_topk(const float* logits, int64_t M, int E, int k, int score_fn, const float* bias,
                        int renormalize, double scale, int32_t* topk_ids, float* topk_w)
{
    char* taken = (char*)malloc((size_t)E);
    double* v = (double*)malloc(sizeof(double) * (size_t)k);
    for (int64_t t = 0; t < M; t++) {
        const float* lg = logits + (size_t)t * E;
        int32_t* ids = topk_ids + (size_t)t * k;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; j++) {
            int best = -1;
            float bk = 0.0f;
            for (int e = 0; e < E; e++) {
                if (taken[e]) continue;
                float key = router_key(lg, bias, score_fn, e);
                if (best < 0 || key > bk) { best = e; bk = key; }
            }
            taken[best] = 1;
            ids[j] = best;
        }
        double z = 0.0;
        if (score_fn == ORACLE_SCORE_SOFTMAX) {
            double m = lg[0];
            for (int e = 1; e < E; e++) if (lg[e] > m) m = lg[e];
            for (int j = 0; j < k; j++) v[j] = exp((double)lg[ids[j]] - m);
            if (renormalize) for (int j = 0; j < k; j++) z += v[j];
            else for (int e = 0; e < E; e++) z += exp((double)lg[e] - m);
        } else {
            for (int j = 0; j < k; j++) v[j] = 1.0 / (1.0 + exp(-(double)lg[ids[j]]));
            if (renormalize) for (int j = 0; j < k; j++) z += v[j];
            else z = 1.0;
        }
        for (int j = 0; j < k; j++) topk_w[(size_t)t * k + j] = (float)(v[j] / z * scale);
    }
    free(v);
    free(taken);
}

/* ------------------------------------------------------------------------- */
/* Group-limited noaux-TC router                                               */
/* [P2 Reviewed changes: route_noaux_tc.py, a noaux-TC routing kernel, which   */
/*  the MoE router switches to]                                                */
/* The pages name the method only.  Reading (the published auxiliary-loss-free */
/* routing with a per-expert selection bias and group-limited selection):      */
/* sigmoid scores; each expert's choice key is its score plus its bias; the E  */
/* experts form n_group groups of E / n_group consecutive ids; a group's score */
/* is the sum of its two largest keys (its one key when groups have one       */
/* expert); the topk_group best groups are kept; the k largest keys among     */
/* their experts are chosen; weights come from the unbiased scores.           */
/* ------------------------------------------------------------------------- */

/* logits: [M, E] fp32; bias: [E] fp32 or NULL; topk_ids / topk_w: [M, k].
 * Keys: RN32(sigmoid_rn(l_e) + bias_e) (sigmoid_rn alone without a bias).
 * Group score: RN32(key_a + key_b), key_a >= key_b the two largest keys of the
 * group.  Groups are chosen one at a time, largest score first, equal scores
 * to the lower group index; experts likewise among the chosen groups, equal
 * keys to the lower expert id.  Weights as oracle_router_topk's sigmoid
 * scoring: 1 / (1 + exp(-l_j)) in fp64, divided by their sum over the k chosen
 * when renormalize is set, times scale, rounded once to fp32.
 * Requires E % n_group == 0, 1 <= topk_group <= n_group and
 * 1 <= k <= topk_group * (E / n_group). */
void oracle_router_noaux_tc(const float* logits, int64_t M, int E, int k, int n_group, int topk_group,
                            const float* bias, int renormalize, double scale, int32_t* topk_ids, float* topk_w)
{
    int gs = E / n_group;
    float* key = (float*)malloc(sizeof(float) * (size_t)E);
    float* gscore = (float*)malloc(sizeof(float) * (size_t)n_group);
    char* gsel = (char*)malloc((size_t)n_group);
    char* taken = (char*)malloc((size_t)E);
    double* v = (double*)malloc(sizeof(double) * (size_t)k);
    for (int64_t t = 0; t < M; t++) {
        const float* lg = logits + (size_t)t * E;
        int32_t* ids = topk_ids + (size_t)t * k;
        for (int e = 0; e < E; e++) {
            float sc = oracle_sigmoid_rn(lg[e]);
            key[e] = bias ? sc + bias[e] : sc;
        }
        /* group scores: the two largest keys of each group, added in fp32 */
        for (int g = 0; g < n_group; g++) {
            int a = -1, b = -1;
            for (int e = g * gs; e < (g + 1) * gs; e++) {
                if (a < 0 || key[e] > key[a]) { b = a; a = e; }
                else if (b < 0 || key[e] > key[b]) { b = e; }
            }
            gscore[g] = b < 0 ? key[a] : key[a] + key[b];
        }
        /* the topk_group best groups */
        memset(gsel, 0, (size_t)n_group);
        for (int j = 0; j < topk_group; j++) {
            int best = -1;
            for (int g = 0; g < n_group; g++) {
                if (gsel[g]) continue;
                if (best < 0 || gscore[g] > gscore[best]) best = g;
            }
            gsel[best] = 1;
        }
        /* the k largest keys among the chosen groups' experts */
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; j++) {
            int best = -1;
            for (int e = 0; e < E; e++) {
                if (taken[e] || !gsel[e / gs]) continue;
                if (best < 0 || key[e] > key[best]) best = e;
            }
            taken[best] = 1;
            ids[j] = best;
        }
        double z = 0.0;
        for (int j = 0; j < k; j++) v[j] = 1.0 / (1.0 + exp(-(double)lg[ids[j]]));
        if (renormalize) for (int j = 0; j < k; j++) z += v[j];
        else z = 1.0;
        for (int j = 0; j < k; j++) topk_w[(size_t)t * k + j] = (float)(v[j] / z * scale);
    }
    free(v); free(taken); free(gsel); free(gscore); free(key);
}

/* ------------------------------------------------------------------------- */
/* Whole layer for a subset of tokens                                          */
/* [P1 Modification: gate/up GEMM -> silu_and_mul_post_quant -> FP8 activation  */
/*  + scale -> down GEMM]; [P4: moe_reduce applies the router weights]          */
/* ------------------------------------------------------------------------- */

/* hidden: [M, H] BF16; topk_ids/topk_w: [M, k]; w13: [L, 2I, H] E4M3 with
 * w13_s: [L, 2I/128, H/128]; w2: [L, H, I] E4M3 with w2_s: [L, H/128, I/128].
 * Computes out[t, :] for each t in tokens[0..n_tokens) (all tokens when tokens
 * is NULL, n_tokens = M).  Intermediates, when the pointers are non-NULL, are
 * written for the same tokens' routes, indexed by route id:
 *   h13 [M*k, 2I] BF16, act_q [M*k, I] E4M3, act_s [M*k, I/128], y [M*k, H].
 * scale_fmt applies to both activation quantisations (hidden states before the
 * gate/up GEMM and the SwiGLU output before the down GEMM).  Each token's
 * output depends only on its own routes, so a subset gives the same values as
 * the whole batch. */
void oracle_fused_moe(const uint16_t* hidden, int64_t M, int H,
                      const int32_t* topk_ids, const float* topk_w, int k,
                      const uint8_t* w13, const float* w13_s, const uint8_t* w2, const float* w2_s,
                      int expert_offset, int L, int I, int scale_fmt, float clamp_limit,
                      const int64_t* tokens, int64_t n_tokens,
                      uint16_t* out, uint16_t* h13_out, uint8_t* q_out, float* s_out, uint16_t* y_out)
{
    int GH = H / ORACLE_GROUP, GI = I / ORACLE_GROUP;
    if (!tokens) n_tokens = M;
    uint8_t* aq = (uint8_t*)malloc((size_t)H);
    float* as = (float*)malloc(sizeof(float) * (size_t)GH);
    uint16_t* h13 = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)2 * I);
    uint8_t* q = (uint8_t*)malloc((size_t)I);
    float* s = (float*)malloc(sizeof(float) * (size_t)GI);
    uint16_t* y = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)k * H);
    float* w = (float*)malloc(sizeof(float) * (size_t)k);
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    for (int64_t ti = 0; ti < n_tokens; ti++) {
        int64_t t = tokens ? tokens[ti] : ti;
        oracle_quant_fp8(hidden + (size_t)t * H, 1, H, scale_fmt, aq, as);
        for (int j = 0; j < k; j++) {
            int64_t r = t * k + j;
            ids[j] = topk_ids[r];
            w[j] = topk_w[r];
            int64_t e = (int64_t)topk_ids[r] - expert_offset;
            if (e < 0 || e >= L) continue;
            gemm_row(aq, as, w13 + (size_t)e * 2 * I * H, w13_s + (size_t)e * (2 * I / ORACLE_GROUP) * GH,
                     2 * I, H, h13);
            oracle_silu_and_mul_quant_fp8(h13, 1, I, NULL, NULL, 0, clamp_limit, scale_fmt, q, s);
            gemm_row(q, s, w2 + (size_t)e * H * I, w2_s + (size_t)e * GH * GI, H, I, y + (size_t)j * H);
            if (h13_out) memcpy(h13_out + (size_t)r * 2 * I, h13, sizeof(uint16_t) * 2 * I);
            if (q_out) memcpy(q_out + (size_t)r * I, q, (size_t)I);
            if (s_out) memcpy(s_out + (size_t)r * GI, s, sizeof(float) * GI);
            if (y_out) memcpy(y_out + (size_t)r * H, y + (size_t)j * H, sizeof(uint16_t) * H);
        }
        /* reduce this token's k routes; ids are re-based to a single token */
        oracle_moe_reduce(y, w, ids, expert_offset, L, 1, k, H, out + (size_t)t * H);
    }
    free(aq); free(as); free(h13); free(q); free(s); free(y); free(w); free(ids);
}

/* Threads OpenMP would use (for reporting the CPU baseline's core count),
 * and a way to change it for timing runs. */
#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
#else
int oracle_num_threads(void) { return 1; }
void oracle_set_threads(int n) { (void)n; }
#endif
