// moe_internal.h — host-side launchers of the layer's kernels (private).
// Every launcher assumes its arguments were validated by the C ABI layer and
// returns the HIP error of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// Workspace pieces are carved at 256-byte boundaries.
inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

// bf16 shared expert: split-K partials (workspace), reduced by a second stage.
// A Bf16Side describes one stage, which the routing launches can run as extra
// workgroups (the stages do not depend on the routing).
struct Bf16Side {
    const uint16_t* w;  // bf16 weights [N][K]: W13 (N = 2I, K = H) or W2 (N = H, K = I)
    int I, H, M;        // intermediate, hidden, rows
    int splits;         // gate_up K splits
    const uint16_t* x;  // bf16 [M][H] (gate_up input)
    float* part;        // fp32 [splits][M][2I] (gate_up partials)
    uint16_t* h;        // bf16 [M][I] (SwiGLU output, down input)
    float* y;           // fp32 [M][H] (down output)
    int blocks;         // workgroups of the stage
    float limit;        // clamped SwiGLU limit (0: unclamped)
    // static-FP8 shared expert (fp8 != 0): E4M3 weights w8 [N][K] with the
    // per-tensor scale *wscale (device); gate_up quantizes x with the static
    // input scale s_in and writes raw partial sums; the SwiGLU stage scales
    // them by s_in * *wscale, rounds g, u and h to bf16 and writes h as E4M3
    // codes hq [M][I] quantized with s_out; down reads hq with its static
    // scale s_in and scales the sums by s_in * *wscale.
    int fp8;
    const uint8_t* w8;
    const float* wscale;
    float s_in, s_out;
    uint8_t* hq;
};
enum Bf16Stage { kBf16None = 0, kBf16GateUp = 1, kBf16Swiglu = 2, kBf16Down = 3 };
// An empty side: no extra workgroups.
inline Bf16Side no_side() {
    Bf16Side s{};
    return s;
}
// The partial logits: split-major [splits][M][E] fp32 (sp = 0), or, at 16 or
// fewer rows, expert-contiguous [M][E][sp] with sp = splits rounded up to a
// multiple of 4 (an expert's partials of a row in whole 16-byte loads for the
// top-k; at more rows the router's scattered 4-byte stores cost more).  One
// split is the logits [M][E] either way.
struct RouterPlan {
    int splits;     // K chunks whose partial logits the top-k step sums
    int kchunk;     // elements of H per chunk (multiple of 32)
    int row_groups; // groups of up to 64 rows
    int sp;         // expert-contiguous slots per expert, or 0 (split-major)
};
RouterPlan router_plan(int M, int H, int E);
inline size_t router_partials_floats(const RouterPlan& p, int M, int E) {
    return (size_t)(p.sp ? p.sp : p.splits) * M * E;
}

// The routing launches optionally run one bf16 shared-expert stage each as
// extra workgroups: side1 with the router, side2 with the top-k, side3 with
// the bucketing (stage kBf16None and blocks 0 for none).
// With xq != nullptr the launch also writes the MXFP8 of x in token order
// (codes xq [M][H], scales xs [M][H/32]).
// xg4 > 0: the token-order copy of x is NVFP4 with global xg4 (codes [M][H/2],
// scales [M][H/16]) instead of MXFP8.
hipError_t launch_router_partials(const uint16_t* x, const float* w_router, int M, int H, int E,
                                  const RouterPlan& plan, float* partials, uint8_t* xq, uint8_t* xs,
                                  const Bf16Side& side1, int stage1, hipStream_t stream, float xg4 = 0.0f);
// logits: the router partials (splits of them), or given logits (splits = 1).
// Router and top-k of each row in one workgroup, with the token-order quant
// of x as extra workgroups, for small routers (small_router): no partials.
constexpr int kSmallRouterE = 64;
constexpr int kSmallRouterRows = 64;
bool small_router(int M, int H, int E);
hipError_t launch_router_topk_row(const uint16_t* x, const float* w_router, const float* bias, int M, int H,
                                  int E, int k, float routed_scale, float* logits_out, const moe_routing& route,
                                  uint8_t* xq, uint8_t* xs, float xg4, hipStream_t stream);
// The route step alone in its launch (after the top-k ids are written).
hipError_t launch_bucket(int M, int E, int k, const moe_routing& route, hipStream_t stream, int H, int2* yrec);
hipError_t launch_topk(const float* partials, int splits, int sp, const float* bias, int M, int E, int k,
                       float routed_scale, float* logits_out, const moe_routing& route, const Bf16Side& side2,
                       int stage2, hipStream_t stream);
hipError_t launch_topk_bucket(const float* partials, int splits, int sp, const float* bias, int M, int E,
                              int k, float routed_scale, float* logits_out,
                              const moe_routing& route, const Bf16Side& side2, int stage2,
                              const Bf16Side& side3, int stage3, hipStream_t stream, int H = 0,
                              int2* yrec = nullptr);

// FP4 weights in the load-order layout (moe_pack_fp4).
size_t packed_scale_bytes(int fmt, int E, int N, int K);
hipError_t launch_pack_fp4(int fmt, int E, int N, int K, const uint8_t* w, const uint8_t* sc, uint8_t* w_out,
                           uint8_t* sc_out, hipStream_t stream);

hipError_t launch_quant_mxfp8(const uint16_t* x, int M, int K, uint8_t* q, uint8_t* s,
                              hipStream_t stream);
// NVFP4 activations with global g: codes [rows][K/2], scales [rows][K/16];
// bucket != nullptr: row b is token bucket[b] / k (rows = M*k), else row order.
hipError_t launch_quant_nvfp4(const uint16_t* x, const int32_t* bucket, int k, int rows, int K, float g, uint8_t* q,
                              uint8_t* s, hipStream_t stream);
// MXFP8 rows in bucket order: qp/sp row b holds token bucket[b] / k (P = M*k
// rows); with qt != nullptr also the M token-ordered rows into qt/st.
hipError_t launch_quant_pairs(const uint16_t* x, const int32_t* bucket, int k, int M, int K, uint8_t* qp,
                              uint8_t* sp, uint8_t* qt, uint8_t* st, hipStream_t stream);
// Pairs up to which the fused layer's gate_up workgroups resolve their slot
// from the top-k ids themselves (two per thread), with no route step.
constexpr int kIdsPairs = 512;

// Slots a gate_up resolved from the top-k ids, recorded for the down launch:
// active experts ([min(E,P)]), their bucket ranges ([min(E,P) + 1]), their
// count, and the bucket ([P]) in the route step's order.
struct SlotRecord {
    int32_t *act, *off, *na, *bkt;
    int2* yrec = nullptr;  // [P] grouped-y row of each pair (ygroup_rec), or nullptr
};

// The fused layer's per-pair down outputs y (fp32) are grouped: the bucket
// rows of one expert split into groups of at most kYGroupRows (the rows of one
// 16-row MFMA block of a down pass), and a group of n rows holds its column
// blocks of kYBlockCols one after another, each [n][kYBlockCols].  A down
// workgroup, which owns whole column blocks of a pass, then writes one
// contiguous span per group instead of one short run per row.  Row u of an
// expert whose n rows start at bucket row base: its first column block starts
// ygroup_rec(...).x floats into y, and its column blocks are
// ygroup_rec(...).y * kYBlockCols floats apart.  H is a multiple of
// kYBlockCols, and y's size (< 2^31 bytes) keeps every offset in an int.
constexpr int kYGroupRows = 16, kYBlockCols = 128;
__host__ __device__ inline int2 ygroup_rec(int base, int n, int u, int H) {
    const int g = u & ~(kYGroupRows - 1);
    const int rows = n - g < kYGroupRows ? n - g : kYGroupRows;
    return make_int2((base + g) * H + (u - g) * kYBlockCols, rows);
}

// Expert GEMM jobs.  A routed job covers slots [0, U_max) of the active-expert
// list; a dense job is one expert over all M rows.
struct ExpertJob {
    moe_weights w;          // weights (E experts or one)
    int N_out;              // gate_up: I ; down: H (output features)
    int K;                  // reduction length (gate_up: H ; down: I)
    bool dense;
    // routed
    const int32_t* offsets;
    const int32_t* bucket;
    const int32_t* active;
    const int32_t* num_active;
    const int32_t* active_offsets;  // [slots + 1] bucket range of each slot
    int slots;              // U_max for routed, 1 for dense
    int k;                  // top-k (pair id -> row)
    int M;
    // Few-pair routed path (M*k <= kIdsPairs): with ids != nullptr every
    // workgroup resolves its slot from the top-k ids (no route step needed
    // before it).  With a_tok the gate_up activations are in token order
    // ([M][K]: pair p reads row p / k, the pairs of a pass gathered through
    // the resolved list or the bucket).
    const int32_t* ids = nullptr;
    bool a_tok = false;
    const SlotRecord* record = nullptr;  // gate_up with ids: record the resolved slots
    const int32_t* count = nullptr;      // active list whose entries past *count are stale
    bool ygroup = false;                 // down: y grouped (ygroup_rec) instead of [rows][N_out]
    float swiglu_limit = 0.0f;           // gate_up: clamped SwiGLU limit (0: unclamped)
    // NVFP4 activations (NVFP4 weights only): the activations are NVFP4 codes
    // [rows][K/2] + E4M3 scales [rows][K/16] with global a_global, or
    // a_globals[e] per expert (device, [E]; dense: [1]); a gate_up writes h
    // as NVFP4 with global h_global, or h_globals[e].
    bool a_nvfp4 = false;
    float a_global = 0.0f, h_global = 0.0f;
    const float* a_globals = nullptr;
    const float* h_globals = nullptr;
};

// gate_up over FP4 experts.  When the plan splits K, fp32 partials go to
// `partials` (gate_up_fp4_partials_bytes; 0 means no split and no buffer) and a
// second launch reduces them, applies SwiGLU and requantizes h.
// A second FP4 job (the shared expert) with its operands: it rides along the
// launch of the first (its items after the first's) when both have the same
// format and run over all of K, else it gets a launch of its own.
struct SecondJob {
    const ExpertJob* job = nullptr;
    const uint8_t* a_q = nullptr;
    const uint8_t* a_s = nullptr;
    uint8_t* h_q = nullptr;
    uint8_t* h_s = nullptr;
    float* partials = nullptr;  // for a launch of its own
};
struct SecondDown {
    const ExpertJob* job = nullptr;
    const uint8_t* h_q = nullptr;
    const uint8_t* h_s = nullptr;
    float* y = nullptr;
};

// A bf16 or static-FP8 shared-expert stage may ride along the gate_up launch
// (side, stage).
size_t gate_up_fp4_partials_bytes(const ExpertJob& job);
hipError_t launch_gate_up_fp4(const ExpertJob& job, const uint8_t* a_q, const uint8_t* a_s,
                              uint8_t* h_q, uint8_t* h_s, float* partials, hipStream_t stream,
                              const Bf16Side& side = Bf16Side{}, int stage = 0, const SecondJob& second = SecondJob{});
hipError_t launch_down_fp4(const ExpertJob& job, const uint8_t* h_q, const uint8_t* h_s,
                           float* y, hipStream_t stream, const SecondDown& second = SecondDown{});

size_t gate_up_bf16_partials_bytes(int M, int H, int I);
Bf16Side bf16_side(const ExpertJob& gate_up_or_down, int I, int H, int M, const uint16_t* x, float* part,
                   uint16_t* h, float* y, int stage);
// The static-FP8 shared expert's stages (weights: job.w.w E4M3 codes,
// job.w.global_scale the device weight scale).  gate_up: s_in = the input's
// static scale, s_out = h's; down: s_in = h's.
size_t gate_up_fp8s_partials_bytes(int M, int H, int I);
Bf16Side fp8s_side(const ExpertJob& gate_up_or_down, int I, int H, int M, const uint16_t* x, float* part,
                   uint8_t* hq, float* y, float s_in, float s_out, int stage);
hipError_t launch_gate_up_fp8s(const ExpertJob& job, const uint16_t* x, float s_in, float s_h, uint8_t* hq,
                               float* partials, hipStream_t stream);
hipError_t launch_down_fp8s(const ExpertJob& job, const uint8_t* hq, float s_h, float* y, hipStream_t stream);
hipError_t launch_gate_up_bf16(const ExpertJob& job, const uint16_t* a, uint16_t* h,
                               float* partials, hipStream_t stream);
hipError_t launch_down_bf16(const ExpertJob& job, const uint16_t* h, float* y, hipStream_t stream);

// y [M*k][H] by pair, or grouped when yrec != nullptr (pair p's row at
// yrec[p]); y_sh [M][H], or grouped as a dense down writes it (rows 0..M-1 as
// one expert's) when ysh_grouped.
hipError_t launch_finalize(const float* y, const float* topk_w, const float* y_sh,
                           const uint16_t* residual, const uint16_t* gamma, float eps, int M,
                           int H, int k, uint16_t* out, uint16_t* residual_out, uint8_t* out_q,
                           uint8_t* out_s, hipStream_t stream, const int2* yrec = nullptr,
                           bool ysh_grouped = false);

}  // namespace moe
