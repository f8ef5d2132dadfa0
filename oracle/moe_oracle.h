/*
 * moe_oracle.h — reference CPU implementation of the small-M block-scaled-FP4
 * sigmoid-routed MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check
 * and the benchmark's CPU-baseline leg may load this library.  The layer's
 * product path (the HIP library) never links, loads or calls it, and the two
 * share no code, header, table or constant.
 *
 * Plain, slow and meant to be read against the pages:
 *   - number formats decoded through 16/256/256-entry tables built from the
 *     formats' closed-form definitions;
 *   - every sum in fp64;
 *   - every quantization point of the layer mirrored (activation MXFP8 or,
 *     for NVFP4 experts on NVFP4 activations, NVFP4 with its static globals
 *     and every code decision in fp32; the SwiGLU-output requant in the same
 *     format; the static-FP8 shared expert's input quant, bf16 gate/up
 *     outputs, bf16 h and its static-FP8 requant; bf16 residual, bf16
 *     output);
 *   - the SwiGLU optionally clamped (orc_swiglu).
 *
 * Every function that cannot be pinned against something other than itself
 * says "parity unpinned" here; at present every exported function has a pin
 * in the CPU test suite (format tables exhaustively, encoders by brute force
 * or an independent fp32 derivation, routing by full sort, expert GEMMs by
 * dense mixtures and textbook cases, the clamp by closed forms, finalize by
 * closed forms).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_NONE = 0, ORC_MXFP4 = 1, ORC_NVFP4 = 2, ORC_BF16 = 3, ORC_FP8S = 4 };

/* One weight matrix [N, K], canonical layout: packed FP4 [N, K/2] (low nibble
 * = even K), scales [N, K/32] E8M0 (MXFP4) or [N, K/16] E4M3 (NVFP4), plus an
 * fp32 per-tensor global (NVFP4); or bf16 [N, K]; or (ORC_FP8S, shared expert
 * only) E4M3 codes [N, K] in `packed` with the fp32 per-tensor weight scale in
 * `gscale`. */
/* Activation formats of the expert GEMMs. */
enum { ORC_ACT_MXFP8 = 0, ORC_ACT_NVFP4 = 1 };

typedef struct {
    int fmt;
    const uint8_t *packed;
    const uint8_t *scales;
    float gscale;
    const uint16_t *bf16;
} orc_mat;

/* The whole layer.  Routed expert e has W13 = w13[e] ([2I, H]) and
 * W2 = w2[e] ([H, I]); unused experts may have null pointers. */
typedef struct {
    int M, H, E, k, I, I_sh;
    int wfmt;            /* ORC_MXFP4 or ORC_NVFP4 */
    int sfmt;            /* ORC_NONE, ORC_MXFP4, ORC_NVFP4, ORC_BF16 or ORC_FP8S */
    double routed_scale;
    double eps;
    const uint16_t *x;         /* bf16 [M, H] */
    const uint16_t *residual;  /* bf16 [M, H] */
    const uint16_t *gamma;     /* bf16 [H] */
    const float *Wr;           /* fp32 [E, H] (only for oracle logits) */
    const float *bias;         /* fp32 [E] or NULL */
    const orc_mat *w13;        /* E entries */
    const orc_mat *w2;         /* E entries */
    orc_mat sh13, sh2;         /* shared expert (fmt ORC_NONE when absent) */
    double swiglu_limit;       /* clamped SwiGLU of every expert (orc_swiglu); <= 0: none */
    int act_fmt;               /* ORC_ACT_MXFP8, or ORC_ACT_NVFP4 (NVFP4 experts only) */
    float x_gscale;            /* NVFP4 activations: global of the layer input */
    const float *h_gscale;     /* NVFP4 activations: global of each routed expert's h [E] */
    float sh_h_gscale;         /* NVFP4 activations: global of the shared expert's h */
    float sh_in13, sh_in2;     /* ORC_FP8S shared expert: static input scales of gate/up and down */
} orc_layer;

/* ---- formats ---- */
double orc_e2m1_value(int code);
double orc_e4m3_value(int code);
double orc_e8m0_value(int code);
double orc_bf16_value(uint16_t bits);
uint16_t orc_bf16_rne(double v);
uint8_t orc_e4m3_rne_sat(double v);
void orc_e4m3_rne_sat_n(const double *v, int n, uint8_t *out);
void orc_bf16_rne_n(const double *v, int n, uint16_t *out);
void orc_mxfp8_quant_block(const double *v, uint8_t *q, uint8_t *s);
void orc_mxfp8_quant_bf16(const uint16_t *x, int M, int K, uint8_t *q, uint8_t *s);
void orc_mxfp8_quant_f64(const double *v, int M, int K, uint8_t *q, uint8_t *s);
void orc_mxfp8_dequant(const uint8_t *q, const uint8_t *s, int K, double *out);
uint8_t orc_e2m1_rne_sat(float v);
void orc_nvfp4_quant_block(const float *v, float g, uint8_t *q8, uint8_t *sc);
void orc_nvfp4_quant_f32(const float *v, int M, int K, float g, uint8_t *q, uint8_t *s);
void orc_nvfp4_quant_bf16(const uint16_t *x, int M, int K, float g, uint8_t *q, uint8_t *s);
void orc_nvfp4_dequant(const uint8_t *q, const uint8_t *s, int K, float g, double *out);
void orc_mat_row(const orc_mat *m, int K, int n, double *out);

/* ---- router ---- */
void orc_router_logits(const uint16_t *x, const float *Wr, int M, int H, int E, double *logits);
void orc_topk_row(const float *logits_row, const float *bias, int E, int k, double scale,
                  int32_t *ids, float *w, double *s_sel);
void orc_route(const float *logits, const float *bias, int M, int E, int k, double scale,
               int32_t *ids, float *w, int32_t *offsets, int32_t *bucket,
               int32_t *tile_expert, int32_t *tile_begin, int32_t *tile_rows,
               int32_t *num_tiles);

/* ---- one expert on one activation row ---- */
double orc_swiglu(double g, double u, double limit);
void orc_gate_up(const orc_mat *w13, int H, int I, const double *a, double limit, double *h);
void orc_gate_up_bf16(const orc_mat *w13, int H, int I, const uint16_t *x_row, double limit, double *h);
void orc_down(const orc_mat *w2, int H, int I, const double *h, double *y);
/* the static-FP8 shared expert (ORC_FP8S): the input quant of one value, the
 * gate/up on a bf16 row (h and optionally g/u as bf16 bits), the down on h */
uint8_t orc_fp8s_quant(float v, float s_in);
void orc_gate_up_fp8s(const orc_mat *w13, int H, int I, const uint16_t *x_row, float s_in, double limit,
                      uint16_t *h, uint16_t *gu);
void orc_down_fp8s(const orc_mat *w2, int H, int I, const uint16_t *h, float s_in, double *y, uint8_t *hq);

/* ---- finalize ---- */
void orc_finalize_row(int H, int k, const double *y, const float *w, const double *y_sh,
                      const uint16_t *residual, const uint16_t *gamma, double eps,
                      double *out64, uint16_t *out_bf16, uint16_t *resid_out);

/* ---- the layer on a subset of rows ---- */
int orc_moe_rows(const orc_layer *L, const float *logits, const int32_t *rows, int nrows,
                 int nthreads, double *out64, uint16_t *out_bf16, uint16_t *resid_out,
                 int32_t *ids, float *w, double *y_routed, double *y_sh,
                 uint8_t *hq, uint8_t *hs);

int orc_num_cores(void);

#ifdef __cplusplus
}
#endif
#endif
