/*
 * moe_oracle.c — reference CPU implementation of the small-M block-scaled-FP4
 * sigmoid-routed MoE layer.  TEST INFRASTRUCTURE ONLY (see moe_oracle.h):
 * only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
 *
 * What the layer computes, and where the pages describe it:
 *   - sigmoid router with renormalized top-k over one expert group:
 *     sgl-nvidia-mega PR #24, "Modifications / Target spec" (spec.py pins one
 *     expert group, sigmoid scores and the renormalized top-8); SGLang-NVIDIA-
 *     Mega README, DeepSeek-V4.1 slot table, row "Router top-k";
 *   - the route step that groups each expert's rows into 8-row tiles, an
 *     expert taken by more than 8 rows getting several tiles: README slot
 *     table, row "Routed experts (moe)";
 *   - one-pass MXFP8 quantization of the activations: README slot table, row
 *     "Shared expert gate_up (shared_ll)";
 *   - block-scaled FP4 gate_up GEMM, SwiGLU, requantization, down GEMM:
 *     README Qwen3.5 slot table, row "mkm"; PR #33 appended table, row
 *     "shared act quant"; NVFP4 K-groups of 16 with FP8 scale rows: SGLang
 *     Spark GB10 Optimizations, section 1;
 *   - top-k weighted finalize fused with the shared-expert add, the residual
 *     add and RMSNorm: README slot table, rows "hop_b" and "two_shot"; README
 *     Qwen3.5 slot table, row "hop"; routed scaling factor in the MoE sum:
 *     SGLang Spark GB10 Optimizations, section 1 (Marlin MoE kernel fix).
 *
 * The pages do not define the arithmetic of the formats or of several steps;
 * the readings taken are stated next to the code that takes them.
 */
#include "moe_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------------ */
/* Number formats.  The pages name E2M1 (FP4), E4M3 (FP8) and E8M0 scales but
 * never define them; the reading is the OCP Microscaling Formats v1.0
 * definitions:
 *   E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent field 0 is
 *         subnormal (m * 0.5); no Inf/NaN; magnitudes 0..6.
 *   E4M3 ("fn"): sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent
 *         field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no Inf; max 448.
 *   E8M0: 2^(c-127); c = 255 is NaN.                                          */

static double T_E2M1[16];
static double T_E4M3[256];
static double T_E8M0[256];
static pthread_once_t tables_once = PTHREAD_ONCE_INIT;

static void build_tables(void)
{
    for (int c = 0; c < 16; ++c) {
        int s = c >> 3, e = (c >> 1) & 3, m = c & 1;
        double mag = (e == 0) ? m * 0.5 : ldexp(1.0 + m * 0.5, e - 1);
        T_E2M1[c] = s ? -mag : mag;
    }
    for (int c = 0; c < 256; ++c) {
        int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
        double mag;
        if (e == 15 && m == 7)
            mag = NAN;
        else if (e == 0)
            mag = ldexp(m / 8.0, -6);
        else
            mag = ldexp(1.0 + m / 8.0, e - 7);
        T_E4M3[c] = s ? -mag : mag;
    }
    for (int c = 0; c < 256; ++c)
        T_E8M0[c] = (c == 255) ? NAN : ldexp(1.0, c - 127);
}

static void tables(void) { pthread_once(&tables_once, build_tables); }

double orc_e2m1_value(int code) { tables(); return T_E2M1[code & 15]; }
double orc_e4m3_value(int code) { tables(); return T_E4M3[code & 255]; }
double orc_e8m0_value(int code) { tables(); return T_E8M0[code & 255]; }

double orc_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round a finite a >= 0 to a binary format with p significant bits and
 * smallest normal exponent emin, round-to-nearest ties-to-even (rint in the
 * default rounding mode).  No upper clamp here. */
static double round_fmt(double a, int p, int emin)
{
    if (a == 0.0)
        return 0.0;
    int e;
    frexp(a, &e); /* a = f * 2^e, f in [0.5, 1): floor(log2 a) = e - 1 */
    int E = e - 1;
    if (E < emin)
        E = emin;
    double quantum = ldexp(1.0, E - (p - 1));
    return rint(a / quantum) * quantum;
}

/* fp64 -> bf16, round to nearest even; overflow to Inf; NaN stays NaN. */
uint16_t orc_bf16_rne(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (isnan(v))
        return sign | 0x7FC0;
    double a = fabs(v);
    double r = isinf(a) ? INFINITY : round_fmt(a, 8, -126);
    const double maxf = ldexp(2.0 - ldexp(1.0, -7), 127);
    if (r > maxf)
        return sign | 0x7F80;
    if (r == 0.0)
        return sign;
    int e;
    frexp(r, &e);
    int E = e - 1;
    if (E < -126) /* subnormal: r is a multiple of 2^-133 */
        return sign | (uint16_t)(r / ldexp(1.0, -133));
    uint16_t mant = (uint16_t)((r / ldexp(1.0, E) - 1.0) * 128.0);
    return sign | (uint16_t)((E + 127) << 7) | mant;
}

/* fp64 -> E4M3, round to nearest even, saturating to +-448 (the MXFP8 rule
 * below saturates, as the OCP spec allows for FP8 elements); NaN -> S.1111.111. */
uint8_t orc_e4m3_rne_sat(double v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0;
    if (isnan(v))
        return sign | 0x7F;
    double a = fabs(v);
    double r = isinf(a) ? 448.0 : round_fmt(a, 4, -6);
    if (r > 448.0)
        r = 448.0;
    if (r == 0.0)
        return sign;
    int e;
    frexp(r, &e);
    int E = e - 1;
    if (E < -6) /* subnormal: multiples of 2^-9 below 2^-6 */
        return sign | (uint8_t)(r / ldexp(1.0, -9));
    int m = (int)((r / ldexp(1.0, E) - 1.0) * 8.0);
    return sign | (uint8_t)(((E + 7) << 3) | m);
}

void orc_e4m3_rne_sat_n(const double *v, int n, uint8_t *out)
{
    for (int i = 0; i < n; ++i)
        out[i] = orc_e4m3_rne_sat(v[i]);
}

void orc_bf16_rne_n(const double *v, int n, uint16_t *out)
{
    for (int i = 0; i < n; ++i)
        out[i] = orc_bf16_rne(v[i]);
}

/* One MXFP8 block of 32 values.  The pages ask for a one-pass MXFP8 quant
 * but do not state the scale rule; the reading is the OCP MX v1.0 rule:
 * shared exponent = floor(log2(amax)) - 8 (8 = E4M3's largest exponent),
 * clamped to the E8M0 range [-127, 127]; elements v / 2^shared rounded to
 * nearest even E4M3 and saturated at 448.  amax = 0 gives code 0 (2^-127).
 * A block holding NaN or Inf gets the NaN scale (0xFF) and NaN elements. */
void orc_mxfp8_quant_block(const double *v, uint8_t *q, uint8_t *s)
{
    double amax = 0.0;
    int special = 0;
    for (int i = 0; i < 32; ++i) {
        if (isnan(v[i]) || isinf(v[i]))
            special = 1;
        else if (fabs(v[i]) > amax)
            amax = fabs(v[i]);
    }
    if (special) {
        *s = 0xFF;
        for (int i = 0; i < 32; ++i)
            q[i] = (signbit(v[i]) ? 0x80 : 0) | 0x7F;
        return;
    }
    int shared = -127;
    if (amax > 0.0) {
        int e;
        frexp(amax, &e);
        shared = (e - 1) - 8;
        if (shared < -127)
            shared = -127;
        if (shared > 127)
            shared = 127;
    }
    *s = (uint8_t)(shared + 127);
    for (int i = 0; i < 32; ++i)
        q[i] = orc_e4m3_rne_sat(ldexp(v[i], -shared));
}

void orc_mxfp8_quant_f64(const double *v, int M, int K, uint8_t *q, uint8_t *s)
{
    for (int r = 0; r < M; ++r)
        for (int b = 0; b < K / 32; ++b)
            orc_mxfp8_quant_block(v + (size_t)r * K + 32 * b, q + (size_t)r * K + 32 * b,
                                  s + (size_t)r * (K / 32) + b);
}

void orc_mxfp8_quant_bf16(const uint16_t *x, int M, int K, uint8_t *q, uint8_t *s)
{
    double blk[32];
    for (int r = 0; r < M; ++r)
        for (int b = 0; b < K / 32; ++b) {
            for (int i = 0; i < 32; ++i)
                blk[i] = orc_bf16_value(x[(size_t)r * K + 32 * b + i]);
            orc_mxfp8_quant_block(blk, q + (size_t)r * K + 32 * b, s + (size_t)r * (K / 32) + b);
        }
}

void orc_mxfp8_dequant(const uint8_t *q, const uint8_t *s, int K, double *out)
{
    tables();
    for (int i = 0; i < K; ++i)
        out[i] = T_E4M3[q[i]] * T_E8M0[s[i / 32]];
}

/* ------------------------------------------------------------------------ */
/* NVFP4 activations (README Qwen3.5 slot table: row "route" quantizes the MoE
 * input to NVFP4 in the router launch, row "mkm" requantizes the SwiGLU output
 * to NVFP4 before FC2).  The pages give no activation-scale rule.  Reading,
 * the NVFP4 weight encoding (E2M1 codes, an E4M3 scale per 16 values, an fp32
 * global) applied to activations with a static global g given by the caller,
 * every decision taken in fp32 so that a GPU computing in fp32 takes the same
 * ones:
 *   a block of 16 values v (fp32) with a non-finite value: scale byte 0x7F
 *     (E4M3 NaN), all codes 0;
 *   else amax = max |v|; s = amax / (6 g) (fp32: the product 6 g rounded, then
 *     the quotient rounded); scale = E4M3 RNE of s, saturating at 448;
 *     sd = its value; sd == 0: all codes 0; else each code = E2M1 RNE of
 *     v / (sd g) (fp32 product, then fp32 quotient), saturating at 6, with
 *     the sign of the quotient;
 *   value = E2M1(code) * E4M3(scale) * g.
 * Codes pack two per byte, the even element in the low nibble (as the
 * weights); scales are one byte per 16 values. */

/* E2M1 code of v: the nearest of the eight magnitudes, ties to the code whose
 * mantissa bit is 0 (even), saturating at 6, with v's sign bit. */
uint8_t orc_e2m1_rne_sat(float v)
{
    tables();
    const int neg = signbit(v) ? 1 : 0;
    const double a = fabs((double)v);
    int best = 7;
    if (a < 6.0) {
        best = 0;
        for (int c = 1; c < 8; ++c) {
            const double dc = fabs(T_E2M1[c] - a), db = fabs(T_E2M1[best] - a);
            if (dc < db || (dc == db && (c & 1) == 0))
                best = c;
        }
    }
    return (uint8_t)((neg << 3) | best);
}

void orc_nvfp4_quant_block(const float *v, float g, uint8_t *q8, uint8_t *sc)
{
    tables();
    float amax = 0.0f;
    int finite = 1;
    for (int i = 0; i < 16; ++i) {
        if (!isfinite(v[i]))
            finite = 0;
        else if (fabsf(v[i]) > amax)
            amax = fabsf(v[i]);
    }
    uint8_t codes[16];
    if (!finite) {
        *sc = 0x7F;
        memset(codes, 0, sizeof(codes));
    } else {
        const float t = 6.0f * g;
        const float sq = amax / t;
        *sc = orc_e4m3_rne_sat((double)sq);
        const float sd = (float)T_E4M3[*sc];
        if (sd == 0.0f) {
            memset(codes, 0, sizeof(codes));
        } else {
            const float d = sd * g;
            for (int i = 0; i < 16; ++i)
                codes[i] = orc_e2m1_rne_sat(v[i] / d);
        }
    }
    for (int i = 0; i < 8; ++i)
        q8[i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
}

void orc_nvfp4_quant_f32(const float *v, int M, int K, float g, uint8_t *q, uint8_t *s)
{
    for (int r = 0; r < M; ++r)
        for (int b = 0; b < K / 16; ++b)
            orc_nvfp4_quant_block(v + (size_t)r * K + 16 * b, g, q + (size_t)r * (K / 2) + 8 * b,
                                  s + (size_t)r * (K / 16) + b);
}

void orc_nvfp4_quant_bf16(const uint16_t *x, int M, int K, float g, uint8_t *q, uint8_t *s)
{
    float blk[16];
    for (int r = 0; r < M; ++r)
        for (int b = 0; b < K / 16; ++b) {
            for (int i = 0; i < 16; ++i)
                blk[i] = (float)orc_bf16_value(x[(size_t)r * K + 16 * b + i]);
            orc_nvfp4_quant_block(blk, g, q + (size_t)r * (K / 2) + 8 * b, s + (size_t)r * (K / 16) + b);
        }
}

void orc_nvfp4_dequant(const uint8_t *q, const uint8_t *s, int K, float g, double *out)
{
    tables();
    for (int i = 0; i < K; ++i) {
        const int code = (i & 1) ? (q[i / 2] >> 4) : (q[i / 2] & 15);
        out[i] = T_E2M1[code] * T_E4M3[s[i / 16]] * (double)g;
    }
}

/* Decode row n of a weight matrix [N, K] into fp64 (exact for every format).
 * MXFP4: E2M1 * E8M0(per 32 along K).  NVFP4: E2M1 * E4M3(per 16 along K) *
 * fp32 global, the two-level NVFP4 scaling of SGLang Spark GB10 Optimizations,
 * section 1 (K-groups of 16 with FP8 scale rows) and the scalar ModelOpt scales
 * of sgl-nvidia-mega PR #33 ("MoE and deferred draft finalization").
 * Packing reading: K contiguous, two codes per byte, low nibble = even K. */
void orc_mat_row(const orc_mat *m, int K, int n, double *out)
{
    tables();
    if (m->fmt == ORC_BF16) {
        for (int k = 0; k < K; ++k)
            out[k] = orc_bf16_value(m->bf16[(size_t)n * K + k]);
        return;
    }
    if (m->fmt == ORC_FP8S) {
        for (int k = 0; k < K; ++k)
            out[k] = T_E4M3[m->packed[(size_t)n * K + k]] * (double)m->gscale;
        return;
    }
    const uint8_t *row = m->packed + (size_t)n * (K / 2);
    for (int k = 0; k < K; ++k) {
        uint8_t byte = row[k / 2];
        int code = (k & 1) ? (byte >> 4) : (byte & 15);
        double scale;
        if (m->fmt == ORC_MXFP4)
            scale = T_E8M0[m->scales[(size_t)n * (K / 32) + k / 32]];
        else
            scale = T_E4M3[m->scales[(size_t)n * (K / 16) + k / 16]] * (double)m->gscale;
        out[k] = T_E2M1[code] * scale;
    }
}

/* ------------------------------------------------------------------------ */
/* Router.  logits[r, e] = sum_h x[r, h] * W_r[e, h] (fp64 here; the layer's
 * GPU logits are fp32 and are checked against these).  The pages put the
 * router GEMM first in the MoE step (README Qwen3.5 slot table, row "route";
 * PR #33 update table, row "route_lin", which also measures router logits
 * against FP64). */
void orc_router_logits(const uint16_t *x, const float *Wr, int M, int H, int E, double *logits)
{
    for (int r = 0; r < M; ++r)
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h)
                acc += orc_bf16_value(x[(size_t)r * H + h]) * (double)Wr[(size_t)e * H + h];
            logits[(size_t)r * E + e] = acc;
        }
}

/* Top-k of one row (PR #24 spec: one expert group, sigmoid scores,
 * renormalized top-k).  Readings where the pages are silent:
 *   - score s = 1 / (1 + exp(-l)) in fp64 from the fp32 logit;
 *   - the optional router bias is added to the score for selection only
 *     (key = s + b); the weights use the unbiased scores;
 *   - order: key descending, equal keys by ascending expert id; slot j holds
 *     the j-th chosen expert;
 *   - weights w_j = (scale * s_j) / (s_0 + ... + s_{k-1}) in fp64 (sum in slot
 *     order), emitted as fp32; scale is the routed scaling factor. */
void orc_topk_row(const float *logits_row, const float *bias, int E, int k, double scale,
                  int32_t *ids, float *w, double *s_sel)
{
    double *s = (double *)malloc(sizeof(double) * E);
    double *key = (double *)malloc(sizeof(double) * E);
    char *taken = (char *)calloc(E, 1);
    for (int e = 0; e < E; ++e) {
        s[e] = 1.0 / (1.0 + exp(-(double)logits_row[e]));
        key[e] = s[e] + (bias ? (double)bias[e] : 0.0);
    }
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e])
                continue;
            if (best < 0 || key[e] > key[best])
                best = e; /* strict '>' keeps the lower id on equal keys */
        }
        taken[best] = 1;
        ids[j] = best;
    }
    double sum = 0.0;
    for (int j = 0; j < k; ++j)
        sum += s[ids[j]];
    for (int j = 0; j < k; ++j) {
        w[j] = (float)((scale * s[ids[j]]) / sum);
        if (s_sel)
            s_sel[j] = s[ids[j]];
    }
    free(s);
    free(key);
    free(taken);
}

/* Route step (README slot table, row "Routed experts (moe)": rows grouped per
 * expert into 8-row tiles, an expert with more than 8 rows taking several).
 * Readings: a bucket lists, expert by expert in ascending id, the pair ids
 * p = r*k + j of the rows that chose that expert, in ascending row order;
 * offsets[e] is where expert e's entries start (offsets[E] = M*k); an expert
 * with n rows has ceil(n/8) tiles of consecutive bucket entries (the last may
 * be partial), listed in (expert, tile) order; an expert with no rows has none. */
void orc_route(const float *logits, const float *bias, int M, int E, int k, double scale,
               int32_t *ids, float *w, int32_t *offsets, int32_t *bucket,
               int32_t *tile_expert, int32_t *tile_begin, int32_t *tile_rows,
               int32_t *num_tiles)
{
    for (int r = 0; r < M; ++r)
        orc_topk_row(logits + (size_t)r * E, bias, E, k, scale, ids + (size_t)r * k,
                     w + (size_t)r * k, NULL);
    int pos = 0, t = 0;
    for (int e = 0; e < E; ++e) {
        offsets[e] = pos;
        for (int r = 0; r < M; ++r)
            for (int j = 0; j < k; ++j)
                if (ids[(size_t)r * k + j] == e)
                    bucket[pos++] = r * k + j;
        int n = pos - offsets[e];
        for (int i = 0; i * 8 < n; ++i) {
            tile_expert[t] = e;
            tile_begin[t] = offsets[e] + 8 * i;
            tile_rows[t] = (n - 8 * i < 8) ? (n - 8 * i) : 8;
            ++t;
        }
    }
    offsets[E] = pos;
    *num_tiles = t;
}

/* ------------------------------------------------------------------------ */
/* SwiGLU of one gate/up pair.  h = silu(g) * u with silu(g) = g / (1 + e^-g)
 * (README Qwen3.5 slot table, row "mkm": FC1, SwiGLU, FC2).  With limit > 0 it
 * is the clamped SwiGLU (README DeepSeek-V4.1 slot table, row "Shared expert
 * gate_up (shared_ll)": SGLang's clamped SwiGLU); the pages give neither the
 * limit nor the clamp's form, so the reading is: the gate is capped from
 * above at limit and the up projection clamped to [-limit, limit], before the
 * product.  limit <= 0: unclamped. */
double orc_swiglu(double g, double u, double limit)
{
    if (limit > 0.0) {
        if (g > limit)
            g = limit;
        if (u > limit)
            u = limit;
        if (u < -limit)
            u = -limit;
    }
    return (g / (1.0 + exp(-g))) * u;
}

/* One expert's gate_up + SwiGLU on one activation row a[H] (already the
 * dequantized MXFP8 values).  Readings: rows [0, I) of W13 are the gate, rows
 * [I, 2I) the up projection; h[n] = orc_swiglu(g[n], u[n], limit). */
void orc_gate_up(const orc_mat *w13, int H, int I, const double *a, double limit, double *h)
{
    double *wrow = (double *)malloc(sizeof(double) * H);
    for (int n = 0; n < I; ++n) {
        double g = 0.0, u = 0.0;
        orc_mat_row(w13, H, n, wrow);
        for (int c = 0; c < H; ++c)
            g += a[c] * wrow[c];
        orc_mat_row(w13, H, I + n, wrow);
        for (int c = 0; c < H; ++c)
            u += a[c] * wrow[c];
        h[n] = orc_swiglu(g, u, limit);
    }
    free(wrow);
}

/* BF16 shared expert (PR #24, "Modifications / Target spec": a BF16 shared
 * expert beside the NVFP4 routed experts).  Reading: the bf16 hidden row is
 * used as is (not quantized), products summed in fp64; the caller rounds h to
 * bf16 before the down projection. */
void orc_gate_up_bf16(const orc_mat *w13, int H, int I, const uint16_t *x_row, double limit, double *h)
{
    double *a = (double *)malloc(sizeof(double) * H);
    for (int c = 0; c < H; ++c)
        a[c] = orc_bf16_value(x_row[c]);
    orc_gate_up(w13, H, I, a, limit, h);
    free(a);
}

/* ---- the static-FP8 shared expert ----
 * README Qwen3.5 slot table, row "route_shared (with route)": the shared
 * expert's gate/up runs on static FP8; sgl-nvidia-mega PR #33, appended table,
 * row "shared act quant": its SiLU-and-mul is fused with the static FP8
 * quantization of the down projection's input, with the FP8 bytes and bf16
 * outputs of the unfused path.  The pages define neither the format nor the
 * rule.  Reading (the plainest FP8 linear with static per-tensor scales):
 * weights are E4M3 codes with one fp32 scale per matrix (orc_mat_row);
 * an input value v (bf16) is stored as the E4M3 code of the fp32 quotient
 * v / s_in (one fp32 rounding, then round to nearest even, saturating at 448;
 * NaN stays NaN); a linear's output is s_in * sum(code values * weights),
 * rounded to bf16, its dtype; h = bf16(silu(g) * u) from those bf16 g, u;
 * h is quantized with the down input's own static scale the same way. */
uint8_t orc_fp8s_quant(float v, float s_in)
{
    const float q = v / s_in; /* the fp32 quotient decides the code */
    return orc_e4m3_rne_sat((double)q);
}

/* gate/up of the static-FP8 shared expert on one bf16 row: h (bf16 bits, [I])
 * and, when gu is not NULL, the bf16 outputs g (gu[0, I)) and u (gu[I, 2I)). */
void orc_gate_up_fp8s(const orc_mat *w13, int H, int I, const uint16_t *x_row, float s_in, double limit,
                      uint16_t *h, uint16_t *gu)
{
    tables();
    double *a = (double *)malloc(sizeof(double) * H);
    double *wrow = (double *)malloc(sizeof(double) * H);
    for (int c = 0; c < H; ++c)
        a[c] = T_E4M3[orc_fp8s_quant((float)orc_bf16_value(x_row[c]), s_in)];
    for (int n = 0; n < I; ++n) {
        double g = 0.0, u = 0.0;
        orc_mat_row(w13, H, n, wrow);
        for (int c = 0; c < H; ++c)
            g += a[c] * wrow[c];
        orc_mat_row(w13, H, I + n, wrow);
        for (int c = 0; c < H; ++c)
            u += a[c] * wrow[c];
        const uint16_t gb = orc_bf16_rne(g * (double)s_in);
        const uint16_t ub = orc_bf16_rne(u * (double)s_in);
        if (gu) {
            gu[n] = gb;
            gu[I + n] = ub;
        }
        h[n] = orc_bf16_rne(orc_swiglu(orc_bf16_value(gb), orc_bf16_value(ub), limit));
    }
    free(a);
    free(wrow);
}

/* down of the static-FP8 shared expert: h (bf16 bits, [I]) quantized with the
 * down input's static scale (codes to hq when not NULL), y [H] in fp64. */
void orc_down_fp8s(const orc_mat *w2, int H, int I, const uint16_t *h, float s_in, double *y, uint8_t *hq)
{
    tables();
    double *a = (double *)malloc(sizeof(double) * I);
    for (int n = 0; n < I; ++n) {
        const uint8_t q = orc_fp8s_quant((float)orc_bf16_value(h[n]), s_in);
        if (hq)
            hq[n] = q;
        a[n] = T_E4M3[q];
    }
    orc_down(w2, H, I, a, y);
    for (int c = 0; c < H; ++c)
        y[c] *= (double)s_in;
    free(a);
}

/* Down projection y[c] = sum_n h[n] * W2[c, n] (README slot table: the second
 * block-scaled GEMM of "Routed experts (moe)"; "FC2" of row "mkm"). */
void orc_down(const orc_mat *w2, int H, int I, const double *h, double *y)
{
    double *wrow = (double *)malloc(sizeof(double) * I);
    for (int c = 0; c < H; ++c) {
        double acc = 0.0;
        orc_mat_row(w2, I, c, wrow);
        for (int n = 0; n < I; ++n)
            acc += h[n] * wrow[n];
        y[c] = acc;
    }
    free(wrow);
}

/* Finalize of one row: the top-k weighted sum plus the shared expert (README
 * slot table, rows "hop_b" and "two_shot"), then the residual add and RMSNorm
 * (README Qwen3.5 slot table, row "hop").  Readings: t = residual + y_sh +
 * sum_j w_j * y_j in fp64 with w_j the emitted fp32 weights; the residual
 * stream is bf16, so residual_out = bf16(t) and RMSNorm reads that rounded
 * value; out = r' / sqrt(mean(r'^2) + eps) * gamma, emitted as bf16. */
void orc_finalize_row(int H, int k, const double *y, const float *w, const double *y_sh,
                      const uint16_t *residual, const uint16_t *gamma, double eps,
                      double *out64, uint16_t *out_bf16, uint16_t *resid_out)
{
    double *rr = (double *)malloc(sizeof(double) * H);
    double ss = 0.0;
    for (int c = 0; c < H; ++c) {
        double t = orc_bf16_value(residual[c]) + (y_sh ? y_sh[c] : 0.0);
        for (int j = 0; j < k; ++j)
            t += (double)w[j] * y[(size_t)j * H + c];
        uint16_t rb = orc_bf16_rne(t);
        if (resid_out)
            resid_out[c] = rb;
        rr[c] = orc_bf16_value(rb);
        ss += rr[c] * rr[c];
    }
    double inv = 1.0 / sqrt(ss / H + eps);
    for (int c = 0; c < H; ++c) {
        double o = rr[c] * inv * orc_bf16_value(gamma[c]);
        if (out64)
            out64[c] = o;
        if (out_bf16)
            out_bf16[c] = orc_bf16_rne(o);
    }
    free(rr);
}

/* ------------------------------------------------------------------------ */
/* The layer on a subset of rows.  Rows are independent, so any subset can be
 * computed on its own; routing of a row only needs that row's logits.  Work is
 * split over (row, slot) items (slot k = the shared expert) so every host core
 * takes part; the finalize of a row runs after all its items. */

typedef struct {
    const orc_layer *L;
    const float *logits;
    const int32_t *rows;
    int nrows;
    int nitems;
    int next;
    int phase;
    pthread_mutex_t mu;
    /* per sampled row */
    int32_t *ids;   /* [nrows, k] */
    float *w;       /* [nrows, k] */
    double *a;      /* [nrows, H] dequantized MXFP8 activations */
    double *y;      /* [nrows, k, H] */
    double *ysh;    /* [nrows, H] */
    uint8_t *hq, *hs;
} rows_job;

/* Expert on a quantized activation: gate_up, SwiGLU, MXFP8 requant of h along
 * I (the pages requantize the SwiGLU output before FC2: README Qwen3.5 slot
 * table, row "mkm"; PR #33 appended table, row "shared act quant"), down. */
static void expert_fp4(const orc_mat *w13, const orc_mat *w2, int H, int I, const double *a,
                       double limit, int act_fmt, float h_g, double *y, uint8_t *hq, uint8_t *hs)
{
    double *h = (double *)malloc(sizeof(double) * I);
    double *hd = (double *)malloc(sizeof(double) * I);
    uint8_t *q = (uint8_t *)malloc(I);
    uint8_t *s = (uint8_t *)malloc(I / 16);
    orc_gate_up(w13, H, I, a, limit, h);
    const int qb = act_fmt == ORC_ACT_NVFP4 ? I / 2 : I;
    const int sb = act_fmt == ORC_ACT_NVFP4 ? I / 16 : I / 32;
    if (act_fmt == ORC_ACT_NVFP4) {
        /* the GPU holds h in fp32: the fp32 rule reads h rounded to fp32 */
        float *hf = (float *)malloc(sizeof(float) * I);
        for (int n = 0; n < I; ++n)
            hf[n] = (float)h[n];
        orc_nvfp4_quant_f32(hf, 1, I, h_g, q, s);
        orc_nvfp4_dequant(q, s, I, h_g, hd);
        free(hf);
    } else {
        orc_mxfp8_quant_f64(h, 1, I, q, s);
        orc_mxfp8_dequant(q, s, I, hd);
    }
    orc_down(w2, H, I, hd, y);
    if (hq)
        memcpy(hq, q, qb);
    if (hs)
        memcpy(hs, s, sb);
    free(h);
    free(hd);
    free(q);
    free(s);
}

/* Phase 0 for sampled row i: routing and the activation quant. */
static void route_row(rows_job *J, int i)
{
    const orc_layer *L = J->L;
    const int H = L->H, E = L->E, k = L->k;
    const int r = J->rows[i];
    float *lrow = (float *)malloc(sizeof(float) * E);
    if (J->logits) {
        memcpy(lrow, J->logits + (size_t)r * E, sizeof(float) * E);
    } else {
        double *l64 = (double *)malloc(sizeof(double) * E);
        orc_router_logits(L->x + (size_t)r * H, L->Wr, 1, H, E, l64);
        for (int e = 0; e < E; ++e)
            lrow[e] = (float)l64[e];
        free(l64);
    }
    orc_topk_row(lrow, L->bias, E, k, L->routed_scale, J->ids + (size_t)i * k,
                 J->w + (size_t)i * k, NULL);
    uint8_t *aq = (uint8_t *)malloc(H);
    uint8_t *as = (uint8_t *)malloc(H / 16);
    if (L->act_fmt == ORC_ACT_NVFP4) {
        orc_nvfp4_quant_bf16(L->x + (size_t)r * H, 1, H, L->x_gscale, aq, as);
        orc_nvfp4_dequant(aq, as, H, L->x_gscale, J->a + (size_t)i * H);
    } else {
        orc_mxfp8_quant_bf16(L->x + (size_t)r * H, 1, H, aq, as);
        orc_mxfp8_dequant(aq, as, H, J->a + (size_t)i * H);
    }
    free(lrow);
    free(aq);
    free(as);
}

/* Phase 1 item: sampled row i, slot j (j == k: the shared expert). */
static void expert_item(rows_job *J, int i, int j)
{
    const orc_layer *L = J->L;
    const int H = L->H, k = L->k, I = L->I;
    const int r = J->rows[i];
    const double *a = J->a + (size_t)i * H;
    if (j < k) {
        int e = J->ids[(size_t)i * k + j];
        const int nv = L->act_fmt == ORC_ACT_NVFP4;
        const int qb = nv ? I / 2 : I, sb = nv ? I / 16 : I / 32;
        expert_fp4(&L->w13[e], &L->w2[e], H, I, a, L->swiglu_limit, L->act_fmt, nv ? L->h_gscale[e] : 0.0f,
                   J->y + ((size_t)i * k + j) * H, J->hq ? J->hq + ((size_t)i * k + j) * qb : NULL,
                   J->hs ? J->hs + ((size_t)i * k + j) * sb : NULL);
        return;
    }
    double *ysh = J->ysh + (size_t)i * H;
    if (L->sfmt == ORC_BF16) {
        double *h = (double *)malloc(sizeof(double) * L->I_sh);
        orc_gate_up_bf16(&L->sh13, H, L->I_sh, L->x + (size_t)r * H, L->swiglu_limit, h);
        for (int n = 0; n < L->I_sh; ++n)
            h[n] = orc_bf16_value(orc_bf16_rne(h[n]));
        orc_down(&L->sh2, H, L->I_sh, h, ysh);
        free(h);
    } else if (L->sfmt == ORC_FP8S) {
        uint16_t *h = (uint16_t *)malloc(sizeof(uint16_t) * L->I_sh);
        orc_gate_up_fp8s(&L->sh13, H, L->I_sh, L->x + (size_t)r * H, L->sh_in13, L->swiglu_limit, h, NULL);
        orc_down_fp8s(&L->sh2, H, L->I_sh, h, L->sh_in2, ysh, NULL);
        free(h);
    } else {
        expert_fp4(&L->sh13, &L->sh2, H, L->I_sh, a, L->swiglu_limit, L->act_fmt, L->sh_h_gscale, ysh, NULL,
                   NULL);
    }
}

static void *rows_worker(void *arg)
{
    rows_job *J = (rows_job *)arg;
    const int per_row = J->L->k + (J->L->sfmt != ORC_NONE ? 1 : 0);
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int it = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (J->phase == 0) {
            if (it >= J->nrows)
                break;
            route_row(J, it);
        } else {
            if (it >= J->nitems)
                break;
            expert_item(J, it / per_row, it % per_row);
        }
    }
    return NULL;
}

static void run_phase(rows_job *J, int phase, int nthreads)
{
    J->phase = phase;
    J->next = 0;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
    for (int t = 0; t < nthreads; ++t)
        pthread_create(&th[t], NULL, rows_worker, J);
    for (int t = 0; t < nthreads; ++t)
        pthread_join(th[t], NULL);
    free(th);
}

/* Computes the sampled rows rows[0..nrows) of the layer.  logits: fp32 [M, E]
 * to route from (NULL: fp32 of the oracle's own fp64 logits).  Every output
 * pointer may be NULL; shapes: out64 [nrows, H], out_bf16 / resid_out
 * [nrows, H] bf16, ids / w [nrows, k], y_routed [nrows, k, H], y_sh
 * [nrows, H], hq [nrows, k, I], hs [nrows, k, I/32].  Returns 0, or -1 on a
 * bad argument. */
int orc_moe_rows(const orc_layer *L, const float *logits, const int32_t *rows, int nrows,
                 int nthreads, double *out64, uint16_t *out_bf16, uint16_t *resid_out,
                 int32_t *ids, float *w, double *y_routed, double *y_sh,
                 uint8_t *hq, uint8_t *hs)
{
    if (!L || !rows || nrows < 0 || L->H % 32 || L->I % 32 || L->k < 1 || L->k > L->E)
        return -1;
    if (L->sfmt != ORC_NONE && L->I_sh % 32)
        return -1;
    if (!logits && !L->Wr)
        return -1;
    if (L->act_fmt == ORC_ACT_NVFP4 &&
        (L->wfmt != ORC_NVFP4 || !L->h_gscale || L->sfmt == ORC_MXFP4))
        return -1;
    if (L->sfmt == ORC_FP8S && !(L->sh_in13 > 0.0f && L->sh_in2 > 0.0f && isfinite(L->sh_in13) && isfinite(L->sh_in2)))
        return -1;
    for (int i = 0; i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= L->M)
            return -1;
    tables();
    const int H = L->H, k = L->k;
    rows_job J;
    memset(&J, 0, sizeof J);
    J.L = L;
    J.logits = logits;
    J.rows = rows;
    J.nrows = nrows;
    J.nitems = nrows * (k + (L->sfmt != ORC_NONE ? 1 : 0));
    J.ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)nrows * k + 4);
    J.w = (float *)malloc(sizeof(float) * (size_t)nrows * k + 4);
    J.a = (double *)malloc(sizeof(double) * (size_t)nrows * H + 8);
    J.y = (double *)malloc(sizeof(double) * (size_t)nrows * k * H + 8);
    J.ysh = (double *)calloc((size_t)nrows * H + 1, sizeof(double));
    J.hq = hq;
    J.hs = hs;
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads <= 0)
        nthreads = orc_num_cores();
    if (nthreads > J.nitems)
        nthreads = J.nitems > 0 ? J.nitems : 1;
    run_phase(&J, 0, nthreads);
    run_phase(&J, 1, nthreads);
    for (int i = 0; i < nrows; ++i) {
        const int r = rows[i];
        orc_finalize_row(H, k, J.y + (size_t)i * k * H, J.w + (size_t)i * k,
                         L->sfmt != ORC_NONE ? J.ysh + (size_t)i * H : NULL,
                         L->residual + (size_t)r * H, L->gamma, L->eps,
                         out64 ? out64 + (size_t)i * H : NULL,
                         out_bf16 ? out_bf16 + (size_t)i * H : NULL,
                         resid_out ? resid_out + (size_t)i * H : NULL);
    }
    if (ids)
        memcpy(ids, J.ids, sizeof(int32_t) * (size_t)nrows * k);
    if (w)
        memcpy(w, J.w, sizeof(float) * (size_t)nrows * k);
    if (y_routed)
        memcpy(y_routed, J.y, sizeof(double) * (size_t)nrows * k * H);
    if (y_sh && L->sfmt != ORC_NONE)
        memcpy(y_sh, J.ysh, sizeof(double) * (size_t)nrows * H);
    free(J.ids);
    free(J.w);
    free(J.a);
    free(J.y);
    free(J.ysh);
    pthread_mutex_destroy(&J.mu);
    return 0;
}

int orc_num_cores(void)
{
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}
