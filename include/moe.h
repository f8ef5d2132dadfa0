/*
 * moe.h — C ABI of the MI355X (gfx950) small-M block-scaled-FP4 sigmoid-routed
 * mixture-of-experts layer.
 *
 * The layer (one decode / verify step of 1 to a few hundred rows):
 *   1. router GEMV and sigmoid top-k with renormalized weights;
 *   2. route step: each expert's rows grouped into 8-row tiles;
 *   3. one-pass MXFP8 quantization of the activations;
 *   4. block-scaled FP4 gate_up GEMM + SwiGLU + MXFP8 requantization;
 *   5. block-scaled FP4 down GEMM;
 *   6. top-k weighted finalize + shared-expert add + residual add + RMSNorm.
 * Where each step is described (page, section): see the comment of each entry.
 *
 * Conventions shared by every entry point
 *   - Memory: every data pointer is device memory owned by the caller.  The
 *     library never allocates, frees or synchronizes, and keeps no global
 *     mutable state; calls are thread-safe.
 *   - Streams: every call enqueues work on `stream` and returns immediately.
 *     Grid sizes depend on shape arguments only, so calls can be captured in
 *     a HIP graph; data-dependent counts stay on the device.
 *   - Types: bf16 is passed as uint16_t bit patterns; FP4 (E2M1) as packed
 *     bytes, two codes per byte, low nibble = even K index; E4M3 and E8M0 as
 *     uint8_t codes.  All arrays are row-major and contiguous.
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued, so a call that returns an error enqueued nothing.  No C++
 *     exception crosses the ABI.  moe_status_str() describes a code.
 *   - Limits (MOE_ERR_UNSUPPORTED otherwise): H % 128 == 0, I % 128 == 0,
 *     1 <= k <= min(E, 32), 1 <= E <= 1024, 1 <= M <= 4096, H <= 16384,
 *     I <= 8192, and a format pair the library implements; for routed expert
 *     GEMMs and the layer also M*k*H*4 <= 2^31 - 2^20 (the fp32 output of
 *     every (row, slot) pair stays under 2 GiB: the kernels address it with
 *     32-bit buffer offsets).
 *
 * Number formats (the pages name them; their definitions are those of the
 * OCP Microscaling Formats v1.0 specification): E2M1 elements; MXFP4 = E2M1
 * with one E8M0 scale 2^(c-127) per 32 consecutive K; NVFP4 = E2M1 with one
 * E4M3 scale per 16 consecutive K and one fp32 global per expert and
 * projection; MXFP8 = E4M3 elements with one E8M0 scale per 32 along K.
 */
#ifndef MOE_MI355_H
#define MOE_MI355_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 10

enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* null pointer, negative size, inconsistent shape */
    MOE_ERR_UNSUPPORTED = 2, /* outside the limits above or an unimplemented format */
    MOE_ERR_WORKSPACE = 3,   /* workspace null, too small or misaligned */
    MOE_ERR_HIP = 4,         /* a launch failed; the HIP error was cleared */
    MOE_ERR_SCRATCH = 5      /* moe_layer_noalloc: the layer needs more than its static scratch */
};

/* Weight formats. */
enum moe_fmt {
    MOE_FMT_NONE = 0,  /* no shared expert */
    MOE_FMT_MXFP4 = 1, /* packed E2M1 + E8M0 per 32 along K */
    MOE_FMT_NVFP4 = 2, /* packed E2M1 + E4M3 per 16 along K + fp32 global per expert */
    MOE_FMT_BF16 = 3,  /* bf16 (shared expert only) */
    MOE_FMT_FP8S = 4   /* static FP8: E4M3 + one fp32 scale per matrix (shared expert only) */
};

/* One projection of E experts (or of the shared expert, E = 1), each a
 * matrix [N, K].  Standard layout, K contiguous:
 *   MXFP4: w = packed [E, N, K/2] (two E2M1 per byte, low nibble first),
 *          scales = E8M0 [E, N, K/32], global unused;
 *   NVFP4: w = packed [E, N, K/2], scales = E4M3 [E, N, K/16], global = fp32 [E];
 *   BF16:  w = bf16 [E, N, K], scales and global unused;
 *   FP8S:  w = E4M3 codes [E, N, K], scales unused, global = fp32 [E], the
 *          per-tensor weight scale (value = E4M3(code) * global).
 * The expert GEMMs and moe_layer take FP4 weights in the load-order layout
 * that moe_pack_fp4 produces from the standard one (same values, other
 * places); bf16 weights are taken as they are.
 * Gate_up weights (W13) have N = 2I with rows [0, I) the gate projection and
 * rows [I, 2I) the up projection; down weights (W2) have N = H, K = I. */
/* Activation formats of the expert GEMMs (moe_layer_desc.act_fmt). */
enum {
    MOE_ACT_MXFP8 = 0, /* E4M3 + E8M0 per 32 (every weight format) */
    MOE_ACT_NVFP4 = 1  /* E2M1 + E4M3 per 16 + an fp32 global (NVFP4 weights: W4A4) */
};

typedef struct moe_weights {
    int fmt;
    const void *w;
    const uint8_t *scales;
    const float *global_scale;
} moe_weights;

/* Routing of M rows with top-k over E experts (P = M*k (row, slot) pairs,
 * pair id p = r*k + j).  Produced by moe_route_topk, read by the expert GEMMs.
 *   topk_ids       int32 [M, k]  chosen experts, slot order = rank
 *   topk_w         fp32  [M, k]  renormalized, scaled routing weights
 *   expert_offsets int32 [E + 1] start of each expert's entries in `bucket`
 *   bucket         int32 [P]     pair ids, expert by expert (ascending id),
 *                                ascending row within an expert
 *   tile_expert, tile_begin, tile_rows  int32 [moe_tile_capacity(M,E,k)]
 *                                8-row tiles of consecutive bucket entries in
 *                                (expert, tile) order; entries past
 *                                num_tiles are unspecified
 *   num_tiles      int32 [1]
 *   active_experts int32 [min(E, P)]  experts with at least one row, ascending;
 *                                entries past num_active are unspecified
 *   num_active     int32 [1]
 *   active_offsets int32 [min(E, P) + 1]  active_offsets[s] =
 *                                expert_offsets[active_experts[s]] for s <
 *                                num_active, P from num_active on (so slot s
 *                                holds bucket entries [active_offsets[s],
 *                                active_offsets[s+1]) and unused slots none) */
typedef struct moe_routing {
    int32_t *topk_ids;
    float *topk_w;
    int32_t *expert_offsets;
    int32_t *bucket;
    int32_t *tile_expert;
    int32_t *tile_begin;
    int32_t *tile_rows;
    int32_t *num_tiles;
    int32_t *active_experts;
    int32_t *num_active;
    int32_t *active_offsets;
} moe_routing;

/* The whole layer's parameters. */
typedef struct moe_layer_desc {
    int M, H, E, k, I, I_sh;     /* I_sh: shared-expert intermediate (0 when none) */
    float routed_scale;          /* routed scaling factor applied to topk_w */
    float eps;                   /* RMSNorm epsilon */
    const float *w_router;       /* fp32 [E, H] */
    const float *router_bias;    /* fp32 [E] selection bias, or NULL */
    moe_weights w13, w2;         /* routed experts: [E, 2I, H] and [E, H, I] */
    moe_weights sh13, sh2;       /* shared expert: [2I_sh, H] and [H, I_sh]; fmt NONE = absent */
    const uint16_t *gamma;       /* bf16 [H] RMSNorm weight */
    float swiglu_limit;          /* clamped SwiGLU of every expert (see moe_expert_gate_up); 0: unclamped */
    /* NVFP4 activations (act_fmt MOE_ACT_NVFP4, NVFP4 experts; shared expert
     * NONE, NVFP4 or BF16): x is quantized with x_global in the router launch
     * (moe_quant_act_nvfp4), each routed expert's h with h_globals[e] and the
     * shared expert's h with *sh_h_global (static globals, device fp32). */
    int act_fmt;
    float x_global;
    const float *h_globals;      /* [E] */
    const float *sh_h_global;    /* [1], or NULL without an NVFP4 shared expert */
    /* Static-FP8 shared expert (sh13.fmt MOE_FMT_FP8S; any act_fmt): the
     * static input scales of its gate/up (applied to the bf16 x) and of its
     * down projection (applied to h), as moe_expert_gate_up_fp8s takes them. */
    float sh_in_scale;
    float sh_h_scale;
} moe_layer_desc;

const char *moe_status_str(int status);
int moe_abi_version(void);

/* Upper bound on the number of 8-row tiles: sum_e ceil(n_e/8) <= ceil(P/8) + min(E, P). */
int moe_tile_capacity(int M, int E, int k);

/* ---------------------------------------------------------------------------
 * moe_pack_fp4 — puts FP4 expert weights into the order in which the gfx950
 * expert GEMMs load them; done once, when the weights are loaded.
 *   Pages: SGLang Spark GB10 Optimizations, section 1 (NVFP4 weights with one
 *   FP8 scale per 16 values along K); README DeepSeek-V4.1 slot table, row
 *   "Routed experts (moe)" (block-scaled expert GEMMs).
 * In: fmt MXFP4 or NVFP4; w, scales in the standard layout above (device).
 * Out: w_out (E*N*K/2 bytes) and scales_out (moe_packed_scale_bytes bytes),
 *   device memory not overlapping the inputs.  With S = K/128, Q = ceil(S/4),
 *   rb a block of 16 rows and lane l = 16g + i (row 16rb + i):
 *     w_out      [E][N/16][S][64][16]: lane l of step s holds the row's bytes
 *                [64s + 16g, +16);
 *     MX scales  [E][N/16][Q][64][4]: byte u = E8M0 of K block 4(4q+u) + g;
 *     NV scales  [E][N/16][Q][64][8]: bytes 2u, 2u+1 = E4M3 of K blocks
 *                8(4q+u) + 2g and + 1;
 *   entries of steps past S are zero.  NVFP4 global scales are not touched.
 * Limits: E >= 1, N % 16 == 0, K % 128 == 0. */
size_t moe_packed_scale_bytes(int fmt, int E, int N, int K);
int moe_pack_fp4(int fmt, int E, int N, int K, const uint8_t *w, const uint8_t *scales,
                 uint8_t *w_out, uint8_t *scales_out, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_route_topk — router GEMV, sigmoid top-k with renormalized weights, and
 * the route step that groups each expert's rows into 8-row tiles.
 *   Pages: sgl-nvidia-mega PR #24, "Modifications / Target spec" (one expert
 *   group, sigmoid scores, renormalized top-8); SGLang-NVIDIA-Mega README,
 *   DeepSeek-V4.1 slot table, rows "Router top-k" (one CTA per row) and
 *   "Routed experts (moe)" (8-row tiles, several tiles for an expert with more
 *   than 8 rows); README Qwen3.5 slot table, row "route" (router GEMM).
 * Arithmetic: logits[r,e] = sum_h x[r,h] * w_router[e,h] with fp32 products
 *   and fp32 accumulation; score s = 1/(1+exp(-logit)) in fp64; selection key
 *   = s + bias[e] (fp64; bias only selects); top-k by key descending, equal keys
 *   by ascending expert id; w_j = routed_scale * s_j / sum_j s_j (fp64, sum in
 *   slot order) rounded to fp32.
 * Inputs: exactly one of x (bf16 [M, H]) or logits_in (fp32 [M, E]); with x,
 *   w_router (fp32 [E, H]) is required and logits_out (fp32 [M, E]) receives
 *   the logits (required with x, ignored with logits_in).  bias: fp32 [E] or
 *   NULL.  Outputs: every pointer of *route.
 * Workspace: moe_route_workspace_bytes(M, H, E, k) bytes (H = 0 when routing
 *   from logits_in), 256-byte aligned, contents need no initialization. */
size_t moe_route_workspace_bytes(int M, int H, int E, int k);
int moe_route_topk(const uint16_t *x, const float *logits_in, const float *w_router,
                   const float *bias, int M, int H, int E, int k, float routed_scale,
                   float *logits_out, const moe_routing *route, void *workspace,
                   size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_quant_act_mxfp8 — one-pass MXFP8 quantization of bf16 rows.
 *   Pages: SGLang-NVIDIA-Mega README, DeepSeek-V4.1 slot table, row "Shared
 *   expert gate_up (shared_ll)" (one-pass MXFP8 quant of the activations).
 * Rule (OCP MX v1.0; the pages do not state one): per 32 consecutive values,
 *   shared exponent = floor(log2 amax) - 8 clamped to [-127, 127], scale code
 *   = shared + 127; elements = E4M3 of x / 2^shared, round to nearest even,
 *   saturated to +-448, sign kept (-0 -> 0x80).  A block holding NaN or Inf
 *   gets scale 0xFF and NaN codes.
 * x: bf16 [M, K]; K % 32 == 0.
 * route == NULL: q: uint8 [M, K], s: uint8 [M, K/32] in row order.
 * route != NULL (a routing of the M rows with top-k k): q [M*k, K], s
 *   [M*k, K/32] in bucket order, row b holding x row bucket[b] / k (each row's
 *   codes are the same as in row order), which is the order the routed
 *   expert GEMMs read. */
int moe_quant_act_mxfp8(const uint16_t *x, int M, int K, const moe_routing *route, int k,
                        uint8_t *q, uint8_t *s, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_quant_act_nvfp4 — one-pass NVFP4 quantization of bf16 rows (the input
 * of NVFP4 experts run with NVFP4 activations).
 *   Pages: README Qwen3.5 slot table, row "route" (the MoE input quantized to
 *   NVFP4 in the router's launch); SGLang Spark GB10 Optimizations, section 1
 *   (NVFP4 K-groups of 16 with FP8 scales).
 * Rule (the pages state none; the NVFP4 weight encoding with a static global,
 * every step in fp32): per 16 values, a block holding a NaN or Inf gets scale
 * 0x7F and codes 0; else s = amax / (6 * global) (product rounded, then the
 * quotient), scale = E4M3 RNE of s saturating at 448, sd its value; sd == 0
 * gives codes 0; else code = E2M1 RNE of x / (sd * global) (product, then the
 * quotient) saturating at 6, with the quotient's sign.  value = E2M1(code) *
 * E4M3(scale) * global.
 * x: bf16 [M, K]; global: fp32 > 0 (finite); q: uint8 [rows, K/2], two codes
 * per byte, the even element in the low nibble; s: uint8 [rows, K/16].
 * route == NULL: rows = M, row order; else rows = M*k in bucket order (row b
 * = token route->bucket[b] / k), as moe_quant_act_mxfp8.  K % 32 == 0. */
int moe_quant_act_nvfp4(const uint16_t *x, int M, int K, float global, const moe_routing *route, int k,
                        uint8_t *q, uint8_t *s, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_expert_gate_up — gate_up GEMM of every routed expert over its rows,
 * SwiGLU, and requantization of the result for the down GEMM.
 *   Pages: README Qwen3.5 slot table, row "mkm" (FC1, SwiGLU, requant, FC2);
 *   README DeepSeek-V4.1 slot table, row "Routed experts (moe)" (block-scaled
 *   GEMMs over 8-row tiles); sgl-nvidia-mega PR #33 appended table, row
 *   "shared act quant" (SiLU-and-mul fused with the down input's quant);
 *   SGLang Spark GB10 Optimizations, section 1 (NVFP4 K-groups of 16).
 * g = A W13[:I]^T, u = A W13[I:]^T with exact products summed in fp32,
 * except that MXFP4 weights run on the scaled FP4 x FP8 matrix instruction,
 * which adds the products of each 128-long K step with a reduced internal
 * precision (measured: about 2^-13 of that step's sum of |products|) before
 * the fp32 accumulation; h = silu(g) * u in fp32.  swiglu_limit > 0 selects the clamped SwiGLU (README
 * DeepSeek-V4.1 slot table, row "Shared expert gate_up (shared_ll)"): g is
 * capped from above at the limit and u clamped to [-limit, limit] before the
 * product; 0 is the plain SwiGLU; negative or NaN is MOE_ERR_INVALID_ARG.
 * FP4 weights (packed by moe_pack_fp4): A is MXFP8
 * (a_q, a_s) [Pr, H] and h is written as MXFP8 (h_q [Pr, I], h_s [Pr, I/32])
 * with the rule of moe_quant_act_mxfp8.  BF16 weights: A is bf16 a_bf16
 * [M, H] and h is written rounded to bf16 (h_bf16 [Pr, I]).
 * route != NULL: experts e of w13 over their routed rows; A and h are in
 *   bucket order (row b = bucket position b, Pr = M*k; moe_quant_act_mxfp8
 *   with the same route writes A so).  route == NULL ("dense"): one expert
 *   (w13 holds E = 1) over all M rows in order (Pr = M); used for the shared
 *   expert.
 * Workspace: moe_gate_up_workspace_bytes(...) bytes (may be 0), 256-byte
 *   aligned; no initialization needed. */
size_t moe_gate_up_workspace_bytes(int fmt, int M, int H, int I, int E, int k, int dense);
int moe_expert_gate_up(const moe_weights *w13, const uint8_t *a_q, const uint8_t *a_s,
                       const uint16_t *a_bf16, const moe_routing *route, int M, int H, int I,
                       int E, int k, float swiglu_limit, uint8_t *h_q, uint8_t *h_s, uint16_t *h_bf16,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_expert_gate_up_tok — moe_expert_gate_up of routed FP4 experts with the
 * MXFP8 activations in token order.
 *   Pages: as moe_expert_gate_up (README Qwen3.5 slot table, row "mkm";
 *   DeepSeek-V4.1 slot table, row "Routed experts (moe)": the expert GEMMs
 *   read the step's input rows, quantized once by the one-pass MXFP8 quant).
 * A is (a_q [M, H], a_s [M, H/32]) as moe_quant_act_mxfp8 writes it without a
 * route: row r = token r.  Each pass of an expert's rows reads its rows'
 * tokens through the bucket (bucket position b reads token bucket[b] / k), so
 * the k rows that pick a token share one copy and no bucket-order copy
 * (M*k rows) is written.  Everything else — route (required), weights, h in
 * bucket order (h_q [M*k, I], h_s [M*k, I/32]), the clamped SwiGLU, the
 * workspace (moe_gate_up_workspace_bytes(fmt, M, H, I, E, k, 0) bytes) and the
 * errors — is that of moe_expert_gate_up, whose h bytes it reproduces exactly
 * from the same activations. */
int moe_expert_gate_up_tok(const moe_weights *w13, const uint8_t *a_q, const uint8_t *a_s,
                           const moe_routing *route, int M, int H, int I, int E, int k,
                           float swiglu_limit, uint8_t *h_q, uint8_t *h_s, void *workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_expert_down — down GEMM y = h W2^T per routed pair (or per row, dense).
 *   Pages: README DeepSeek-V4.1 slot table, row "Routed experts (moe)" (the
 *   second block-scaled GEMM); README Qwen3.5 slot table, row "mkm" (FC2).
 * h is what moe_expert_gate_up wrote (MXFP8 h_q/h_s for FP4 weights, h_bf16
 * for BF16).  y: fp32 [M*k, H] indexed by pair id (route != NULL) or fp32
 * [M, H] by row (dense).  Exact products summed in fp32; MXFP4 weights with
 * the reduced-precision sum of each 128-long K step described at
 * moe_expert_gate_up. */
int moe_expert_down(const moe_weights *w2, const uint8_t *h_q, const uint8_t *h_s,
                    const uint16_t *h_bf16, const moe_routing *route, int M, int H, int I,
                    int E, int k, float *y, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_expert_gate_up_nvfp4a / moe_expert_down_nvfp4a — the expert GEMMs of
 * NVFP4 experts with NVFP4 activations (W4A4).
 *   Pages: README Qwen3.5 slot table, row "mkm" (top-10, FC1, SwiGLU, the
 *   NVFP4 requantization and FC2) and row "route" (the NVFP4 input).
 * gate_up: as moe_expert_gate_up for NVFP4 weights, with A the NVFP4 codes
 *   a_q [Pr, H/2] and scales a_s [Pr, H/16] of global a_global (what
 *   moe_quant_act_nvfp4 writes; route == NULL: Pr = M rows in order, else
 *   bucket order), and h written as NVFP4 (h_q [Pr, I/2], h_s [Pr, I/16]) by
 *   the rule of moe_quant_act_nvfp4 applied to the fp32 h, with global
 *   h_globals[e] of the row's expert (device fp32 [E]; route == NULL: [1]).
 *   Products exact (the E2M1 x E4M3 operands are exact in f16), fp32 sums.
 *   No workspace.
 * down: y as moe_expert_down, with h the NVFP4 codes and scales above and
 *   h_globals their globals.
 * Weights must be NVFP4 (else MOE_ERR_UNSUPPORTED); a_global > 0 finite. */
int moe_expert_gate_up_nvfp4a(const moe_weights *w13, const uint8_t *a_q, const uint8_t *a_s, float a_global,
                              const moe_routing *route, int M, int H, int I, int E, int k, float swiglu_limit,
                              const float *h_globals, uint8_t *h_q, uint8_t *h_s, hipStream_t stream);
int moe_expert_down_nvfp4a(const moe_weights *w2, const uint8_t *h_q, const uint8_t *h_s, const float *h_globals,
                           const moe_routing *route, int M, int H, int I, int E, int k, float *y,
                           hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_expert_gate_up_fp8s / moe_expert_down_fp8s — the static-FP8 shared
 * expert (dense over all M rows).
 *   Pages: README Qwen3.5 slot table, row "route_shared (with route)" (the
 *   shared expert's static-FP8 gate/up, which the layer runs in the router's
 *   launch); sgl-nvidia-mega PR #33, appended table, row "shared act quant"
 *   (its SiLU-and-mul fused with the static FP8 quantization of the down
 *   projection's input).
 * The pages fix no rule; the one implemented: an input value v (bf16) is the
 * E4M3 code of the correctly rounded fp32 quotient v / s (round to nearest
 * even, saturating at +-448, NaN kept NaN), s the input's static scale; a
 * linear's output is s * the weight scale * the sum of the code products
 * (exact products; the FP8 matrix instruction adds each 32-long K step's
 * products with a reduced internal precision before the fp32 accumulation,
 * measured at rel-L2 about 4e-5 against fp32 sums).
 * gate_up: w13 FP8S [1, 2I, H] (rows [0, I) gate, [I, 2I) up); x bf16 [M, H]
 *   quantized with s_in; g and u rounded to bf16; h = bf16(silu(g) * u) (the
 *   clamped form with swiglu_limit > 0, as moe_expert_gate_up); h_q uint8
 *   [M, I] = E4M3 codes of h quantized with s_h.  Workspace:
 *   moe_gate_up_workspace_bytes(MOE_FMT_FP8S, M, H, I, 1, 1, 1) bytes,
 *   256-byte aligned, no initialization needed.
 * down: w2 FP8S [1, H, I]; h_q as above with its scale s_h; y fp32 [M, H].
 * s_in, s_h: finite and > 0 (else MOE_ERR_INVALID_ARG); weights must be
 * MOE_FMT_FP8S (else MOE_ERR_UNSUPPORTED). */
int moe_expert_gate_up_fp8s(const moe_weights *w13, const uint16_t *x, float s_in, float s_h, int M, int H, int I,
                            float swiglu_limit, uint8_t *h_q, void *workspace, size_t workspace_bytes,
                            hipStream_t stream);
int moe_expert_down_fp8s(const moe_weights *w2, const uint8_t *h_q, float s_h, int M, int H, int I, float *y,
                         hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_finalize_rmsnorm — top-k weighted sum of the expert outputs fused with
 * the shared-expert add, the residual add and RMSNorm.
 *   Pages: README DeepSeek-V4.1 slot table, rows "MoE all-reduce + mHC post +
 *   next norm (hop_b)" and "two_shot" (finalize folded with the shared-expert
 *   add); README Qwen3.5 slot table, row "hop" (fused residual add + RMSNorm);
 *   SGLang Spark GB10 Optimizations, section 1 (routed scaling in the MoE sum).
 * t = residual + y_sh + sum_j topk_w[r,j] * y[r*k+j] (fp32); residual_out =
 * bf16(t) (round to nearest even); out = bf16(r' * rsqrt(mean(r'^2) + eps) *
 * gamma) with r' = residual_out.
 * y: fp32 [M*k, H]; topk_w: fp32 [M, k]; y_sh: fp32 [M, H] or NULL; residual,
 * out: bf16 [M, H] (residual may alias out or residual_out, row by row); gamma:
 * bf16 [H]; residual_out: bf16 [M, H] or NULL. */
int moe_finalize_rmsnorm(const float *y, const float *topk_w, const float *y_sh,
                         const uint16_t *residual, const uint16_t *gamma, float eps, int M,
                         int H, int k, uint16_t *out, uint16_t *residual_out,
                         hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_finalize_rmsnorm_mxfp8 — moe_finalize_rmsnorm that also writes the next
 * layer's input as MXFP8.
 *   Pages: README DeepSeek-V4.1 slot table, row "MoE all-reduce + mHC post +
 *   next norm (hop_b)" (the norm's consumer writes the next input's MXFP8
 *   scales so the next GEMM runs on its low-latency path) and row "two_shot"
 *   (the post quantizes the next input to MXFP8); row "Shared expert gate_up
 *   (shared_ll)" for the one-pass MXFP8 quant.
 * Arguments as moe_finalize_rmsnorm, plus out_q: uint8 [M, H] E4M3 codes and
 * out_s: uint8 [M, H/32] E8M0 scale codes, the quant of `out` exactly as
 * moe_quant_act_mxfp8 would produce it from `out` (both NULL: no quant, the
 * same as moe_finalize_rmsnorm; one NULL: MOE_ERR_INVALID_ARG).  Caller-owned
 * device buffers, written in full. */
int moe_finalize_rmsnorm_mxfp8(const float *y, const float *topk_w, const float *y_sh,
                               const uint16_t *residual, const uint16_t *gamma, float eps, int M,
                               int H, int k, uint16_t *out, uint16_t *residual_out, uint8_t *out_q,
                               uint8_t *out_s, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_layer — the whole layer (all steps above) in one call on one stream.
 *   Pages: README Qwen3.5 slot table, row "mkm" (top-k, FC1, SwiGLU, requant
 *   and FC2 as one unit); README "Design" (built at load, nothing allocated
 *   in a step, coverage decided by row count alone).
 * x: bf16 [M, H]; residual: bf16 [M, H] (may equal x); out: bf16 [M, H];
 * residual_out: bf16 [M, H] or NULL.  Optional debug outputs (NULL to skip):
 * logits_out fp32 [M, E], topk_ids_out int32 [M, k], topk_w_out fp32 [M, k].
 * Workspace: moe_layer_workspace_bytes(desc) bytes, 256-byte aligned; no
 * initialization needed; one workspace must not be used by two calls that
 * overlap in time. */
size_t moe_layer_workspace_bytes(const moe_layer_desc *desc);
int moe_layer(const moe_layer_desc *desc, const uint16_t *x, const uint16_t *residual,
              uint16_t *out, uint16_t *residual_out, float *logits_out, int32_t *topk_ids_out,
              float *topk_w_out, void *workspace, size_t workspace_bytes, hipStream_t stream);
/* moe_layer_mxfp8_out — moe_layer whose finalize also writes the next layer's
 * input as MXFP8 (out_q uint8 [M, H], out_s uint8 [M, H/32], as in
 * moe_finalize_rmsnorm_mxfp8; both NULL is moe_layer, one NULL is
 * MOE_ERR_INVALID_ARG).  Same launches as moe_layer. */
int moe_layer_mxfp8_out(const moe_layer_desc *desc, const uint16_t *x, const uint16_t *residual,
                        uint16_t *out, uint16_t *residual_out, uint8_t *out_q, uint8_t *out_s,
                        float *logits_out, int32_t *topk_ids_out, float *topk_w_out, void *workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_layer_noalloc — moe_layer without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).
 * The scratch lives in a static device array of MOE_NOALLOC_SCRATCH_BYTES
 * (32 MiB) that the library holds on every device it runs on until the
 * process ends.  The call allocates nothing and frees nothing; its first call
 * on a device resolves the array's address there (so make it once outside
 * capture), with that device current and `stream` belonging to it.
 * Arguments and results as moe_layer.  A layer whose workspace
 * (moe_layer_workspace_bytes) exceeds the array is refused with
 * MOE_ERR_SCRATCH before anything is enqueued (every five-workload shape up
 * to 48 rows fits; 384 rows at hidden 7168 and intermediate 2048 does not).
 * Every call on a device shares that device's array, which keeps the last
 * call's contents (nothing in it needs to start at zero): calls that overlap
 * in time on one device, on any streams, race and give wrong results. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
int moe_layer_noalloc(const moe_layer_desc *desc, const uint16_t *x, const uint16_t *residual,
                      uint16_t *out, uint16_t *residual_out, float *logits_out, int32_t *topk_ids_out,
                      float *topk_w_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif
