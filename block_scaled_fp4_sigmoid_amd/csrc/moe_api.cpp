// moe_api.cpp — the C ABI of the MoE layer: argument validation, workspace
// layout and launch sequencing (host only; the kernels live in k_*.hip).
//
// Every argument is checked before anything is enqueued, so an error return
// means nothing was launched (the pages' no-silent-fallback rule: an
// unsupported setup is refused with a reason, SGLang-NVIDIA-Mega README,
// "Design").  Grid sizes depend only on shapes (README "Design": coverage is
// decided by row count alone, so captured graphs replay the decision).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/moe.h"
#include "moe_internal.h"

using namespace moe;

namespace {

constexpr int kMaxM = 4096;
constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;
constexpr int kMaxH = 16384;
constexpr int kMaxI = 8192;

// Routed calls address the per-pair buffers (y [M*k, H] fp32, bucket-order
// activations) with 32-bit buffer offsets; the byte size of y must stay below
// the out-of-range offset the kernels use for masked lanes (2^31).
constexpr int64_t kMaxPairBytes = (int64_t{1} << 31) - (int64_t{1} << 20);

int check_pair_bytes(int M, int k, int H) {
    return (int64_t)M * k * H * 4 > kMaxPairBytes ? MOE_ERR_UNSUPPORTED : MOE_OK;
}

bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

// The fused layer writes y grouped (ygroup_rec) from this many bytes of y on.
// A down workgroup's writes then form one span per 16-row group instead of a
// short run per row (384 rows, 88 MB of y: 1046 -> 1021 us per step); the
// finalize pays one dependent load for each pair's row, about 1 us, more than
// the down saves below a few MB (7 rows of top-10 at H 4096, 1.1 MB: +1 us).
#ifndef MOE_Y_GROUP_BYTES
#define MOE_Y_GROUP_BYTES (4u << 20)
#endif
bool y_grouped(int M, int k, int H) { return (int64_t)M * k * H * 4 >= (int64_t)MOE_Y_GROUP_BYTES; }

// A static FP8 input scale: finite and positive.
bool static_scale_ok(float s) { return s > 0.0f && s <= 3.4e38f; }

int check_dims(int M, int H, int E, int k) {
    if (M < 1 || H < 1 || E < 1 || k < 1) return MOE_ERR_INVALID_ARG;
    if (M > kMaxM || E > kMaxE || k > std::min(E, kMaxK)) return MOE_ERR_UNSUPPORTED;
    if (H % 128 != 0 || H > kMaxH) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int check_routing(const moe_routing* r) {
    if (!r || !r->topk_ids || !r->topk_w || !r->expert_offsets || !r->bucket || !r->tile_expert ||
        !r->tile_begin || !r->tile_rows || !r->num_tiles || !r->active_experts || !r->num_active ||
        !r->active_offsets)
        return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

int check_fp4_weights(const moe_weights* w) {
    if (!w) return MOE_ERR_INVALID_ARG;
    if (w->fmt != MOE_FMT_MXFP4 && w->fmt != MOE_FMT_NVFP4) return MOE_ERR_UNSUPPORTED;
    if (!w->w || !w->scales) return MOE_ERR_INVALID_ARG;
    if (w->fmt == MOE_FMT_NVFP4 && !w->global_scale) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

int hip_status(hipError_t e) {
    if (e == hipSuccess) return MOE_OK;
    (void)hipGetLastError();
    return MOE_ERR_HIP;
}

// Sequential carve of a workspace at 256-byte boundaries.
struct Carver {
    char* base;
    size_t off = 0;
    explicit Carver(void* b) : base(static_cast<char*>(b)) {}
    template <typename T>
    T* take(size_t count) {
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off += align_up(count * sizeof(T));
        return p;
    }
};

struct RouteWs {
    float* partials;
};

RouteWs carve_route(Carver& c, int M, int H, int E) {
    RouteWs w;
    const RouterPlan p = router_plan(M, H, E);
    w.partials = c.take<float>(router_partials_floats(p, M, E));
    return w;
}

ExpertJob routed_job(const moe_weights& w, int N_out, int K, const moe_routing& r, int M, int E,
                     int k) {
    ExpertJob j;
    j.w = w;
    j.N_out = N_out;
    j.K = K;
    j.dense = false;
    j.offsets = r.expert_offsets;
    j.bucket = r.bucket;
    j.active = r.active_experts;
    j.num_active = r.num_active;
    j.active_offsets = r.active_offsets;
    j.slots = std::min(E, M * k);
    j.k = k;
    j.M = M;
    return j;
}

ExpertJob dense_job(const moe_weights& w, int N_out, int K, int M) {
    ExpertJob j;
    j.w = w;
    j.N_out = N_out;
    j.K = K;
    j.dense = true;
    j.offsets = j.bucket = j.active = j.num_active = j.active_offsets = nullptr;
    j.slots = 1;
    j.k = 1;
    j.M = M;
    return j;
}

}  // namespace

extern "C" {

const char* moe_status_str(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument (null pointer, bad size or inconsistent shape)";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape or format (see the limits in moe.h)";
        case MOE_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
        case MOE_ERR_HIP: return "a HIP launch failed";
        case MOE_ERR_SCRATCH:
            return "the layer needs more scratch than moe_layer_noalloc's static buffer holds "
                   "(MOE_NOALLOC_SCRATCH_BYTES per device); use moe_layer with a workspace";
        default: return "unknown status";
    }
}

int moe_abi_version(void) { return MOE_ABI_VERSION; }

int moe_tile_capacity(int M, int E, int k) {
    if (M < 1 || E < 1 || k < 1) return 0;
    const int P = M * k;
    return (P + 7) / 8 + std::min(E, P);
}

size_t moe_packed_scale_bytes(int fmt, int E, int N, int K) {
    if ((fmt != MOE_FMT_MXFP4 && fmt != MOE_FMT_NVFP4) || E < 1 || N < 16 || N % 16 != 0 || K < 128 ||
        K % 128 != 0)
        return 0;
    return packed_scale_bytes(fmt, E, N, K);
}

int moe_pack_fp4(int fmt, int E, int N, int K, const uint8_t* w, const uint8_t* scales, uint8_t* w_out,
                 uint8_t* scales_out, hipStream_t stream) {
    if (fmt != MOE_FMT_MXFP4 && fmt != MOE_FMT_NVFP4) return MOE_ERR_UNSUPPORTED;
    if (!w || !scales || !w_out || !scales_out || E < 1 || N < 16 || K < 128) return MOE_ERR_INVALID_ARG;
    if (N % 16 != 0 || K % 128 != 0 || (long)E * N > (1L << 28) || K > kMaxH) return MOE_ERR_UNSUPPORTED;
    return hip_status(launch_pack_fp4(fmt, E, N, K, w, scales, w_out, scales_out, stream));
}

size_t moe_route_workspace_bytes(int M, int H, int E, int k) {
    const int Hc = H == 0 ? 128 : H;  // H = 0: routing from logits_in
    if (check_dims(M, Hc, E, k) != MOE_OK) return 0;
    Carver c(nullptr);
    carve_route(c, M, Hc, E);
    return c.off;
}

int moe_route_topk(const uint16_t* x, const float* logits_in, const float* w_router,
                   const float* bias, int M, int H, int E, int k, float routed_scale,
                   float* logits_out, const moe_routing* route, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
    if ((x == nullptr) == (logits_in == nullptr)) return MOE_ERR_INVALID_ARG;
    if (x && (!w_router || !logits_out)) return MOE_ERR_INVALID_ARG;
    const int Hc = x ? H : 128;
    if (int st = check_dims(M, Hc, E, k)) return st;
    if (int st = check_routing(route)) return st;
    if (!workspace || !aligned256(workspace)) return MOE_ERR_WORKSPACE;
    Carver c(workspace);
    RouteWs w = carve_route(c, M, Hc, E);
    if (c.off > workspace_bytes) return MOE_ERR_WORKSPACE;
    hipError_t e;
    if (x) {
        const RouterPlan p = router_plan(M, H, E);
        e = launch_router_partials(x, w_router, M, H, E, p, w.partials, nullptr, nullptr, no_side(), kBf16None,
                                   stream);
        if (e == hipSuccess)
            e = launch_topk_bucket(w.partials, p.splits, p.sp, bias, M, E, k, routed_scale, logits_out, *route, no_side(),
                                   kBf16None, no_side(), kBf16None, stream);
    } else {
        e = launch_topk_bucket(logits_in, 1, 0, bias, M, E, k, routed_scale, nullptr, *route, no_side(), kBf16None,
                               no_side(), kBf16None, stream);
    }
    return hip_status(e);
}

int moe_quant_act_mxfp8(const uint16_t* x, int M, int K, const moe_routing* route, int k, uint8_t* q,
                        uint8_t* s, hipStream_t stream) {
    if (!x || !q || !s || M < 1 || K < 32) return MOE_ERR_INVALID_ARG;
    if (K % 32 != 0 || K > kMaxH) return MOE_ERR_UNSUPPORTED;
    if (!route) {
        if (M > kMaxM * kMaxK) return MOE_ERR_UNSUPPORTED;
        return hip_status(launch_quant_mxfp8(x, M, K, q, s, stream));
    }
    if (!route->bucket) return MOE_ERR_INVALID_ARG;
    if (k < 1 || k > kMaxK || M > kMaxM) return MOE_ERR_UNSUPPORTED;
    return hip_status(launch_quant_pairs(x, route->bucket, k, M, K, q, s, nullptr, nullptr, stream));
}

int moe_quant_act_nvfp4(const uint16_t* x, int M, int K, float global, const moe_routing* route, int k, uint8_t* q,
                        uint8_t* s, hipStream_t stream) {
    if (!x || !q || !s || M < 1 || K < 32) return MOE_ERR_INVALID_ARG;
    if (!(global > 0.0f) || !(global <= 3.4e38f)) return MOE_ERR_INVALID_ARG;
    if (K % 32 != 0 || K > kMaxH) return MOE_ERR_UNSUPPORTED;
    if (!route) {
        if (M > kMaxM * kMaxK) return MOE_ERR_UNSUPPORTED;
        return hip_status(launch_quant_nvfp4(x, nullptr, 1, M, K, global, q, s, stream));
    }
    if (!route->bucket) return MOE_ERR_INVALID_ARG;
    if (k < 1 || k > kMaxK || M > kMaxM) return MOE_ERR_UNSUPPORTED;
    return hip_status(launch_quant_nvfp4(x, route->bucket, k, M * k, K, global, q, s, stream));
}

size_t moe_gate_up_workspace_bytes(int fmt, int M, int H, int I, int E, int k, int dense) {
    if (check_dims(M, H, dense ? 1 : E, dense ? 1 : k) != MOE_OK) return 0;
    if (I < 128 || I % 128 != 0 || I > kMaxI) return 0;
    if (fmt == MOE_FMT_BF16) return dense ? gate_up_bf16_partials_bytes(M, H, I) : 0;
    if (fmt == MOE_FMT_FP8S) return dense ? gate_up_fp8s_partials_bytes(M, H, I) : 0;
    if (fmt != MOE_FMT_MXFP4 && fmt != MOE_FMT_NVFP4) return 0;
    moe_weights w{};
    w.fmt = fmt;
    moe_routing r{};
    const ExpertJob job = dense ? dense_job(w, I, H, M) : routed_job(w, I, H, r, M, E, k);
    return gate_up_fp4_partials_bytes(job);
}

int moe_expert_gate_up(const moe_weights* w13, const uint8_t* a_q, const uint8_t* a_s,
                       const uint16_t* a_bf16, const moe_routing* route, int M, int H, int I,
                       int E, int k, float swiglu_limit, uint8_t* h_q, uint8_t* h_s, uint16_t* h_bf16,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!w13) return MOE_ERR_INVALID_ARG;
    if (!(swiglu_limit >= 0.0f)) return MOE_ERR_INVALID_ARG;
    const bool dense = route == nullptr;
    if (int st = check_dims(M, H, dense ? 1 : E, dense ? 1 : k)) return st;
    if (I < 128 || I % 128 != 0 || I > kMaxI) return MOE_ERR_UNSUPPORTED;
    if (w13->fmt == MOE_FMT_BF16) {
        if (!dense) return MOE_ERR_UNSUPPORTED;  // bf16 weights: shared expert only
        if (!w13->w || !a_bf16 || !h_bf16) return MOE_ERR_INVALID_ARG;
        const size_t need = moe_gate_up_workspace_bytes(MOE_FMT_BF16, M, H, I, 1, 1, 1);
        if (!workspace || !aligned256(workspace) || workspace_bytes < need) return MOE_ERR_WORKSPACE;
        float* part = static_cast<float*>(workspace);
        ExpertJob job = dense_job(*w13, I, H, M);
        job.swiglu_limit = swiglu_limit;
        return hip_status(launch_gate_up_bf16(job, a_bf16, h_bf16, part, stream));
    }
    if (int st = check_fp4_weights(w13)) return st;
    if (!a_q || !a_s || !h_q || !h_s) return MOE_ERR_INVALID_ARG;
    if (!dense) {
        if (int st = check_routing(route)) return st;
        if (int st = check_pair_bytes(M, k, H)) return st;
    }
    ExpertJob job = dense ? dense_job(*w13, I, H, M) : routed_job(*w13, I, H, *route, M, E, k);
    job.swiglu_limit = swiglu_limit;
    const size_t need = gate_up_fp4_partials_bytes(job);
    if (need && (!workspace || !aligned256(workspace) || workspace_bytes < need)) return MOE_ERR_WORKSPACE;
    return hip_status(launch_gate_up_fp4(job, a_q, a_s, h_q, h_s, static_cast<float*>(workspace), stream));
}

int moe_expert_gate_up_tok(const moe_weights* w13, const uint8_t* a_q, const uint8_t* a_s,
                           const moe_routing* route, int M, int H, int I, int E, int k, float swiglu_limit,
                           uint8_t* h_q, uint8_t* h_s, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
    if (!w13 || !route || !a_q || !a_s || !h_q || !h_s) return MOE_ERR_INVALID_ARG;
    if (!(swiglu_limit >= 0.0f)) return MOE_ERR_INVALID_ARG;
    if (int st = check_dims(M, H, E, k)) return st;
    if (I < 128 || I % 128 != 0 || I > kMaxI) return MOE_ERR_UNSUPPORTED;
    if (w13->fmt != MOE_FMT_MXFP4 && w13->fmt != MOE_FMT_NVFP4) return MOE_ERR_UNSUPPORTED;
    if (int st = check_fp4_weights(w13)) return st;
    if (int st = check_routing(route)) return st;
    if (int st = check_pair_bytes(M, k, H)) return st;
    ExpertJob job = routed_job(*w13, I, H, *route, M, E, k);
    job.swiglu_limit = swiglu_limit;
    job.a_tok = true;  // pass rows gather their tokens through the bucket
    const size_t need = gate_up_fp4_partials_bytes(job);
    if (need && (!workspace || !aligned256(workspace) || workspace_bytes < need)) return MOE_ERR_WORKSPACE;
    return hip_status(launch_gate_up_fp4(job, a_q, a_s, h_q, h_s, static_cast<float*>(workspace), stream));
}

int moe_expert_down(const moe_weights* w2, const uint8_t* h_q, const uint8_t* h_s,
                    const uint16_t* h_bf16, const moe_routing* route, int M, int H, int I,
                    int E, int k, float* y, hipStream_t stream) {
    if (!w2 || !y) return MOE_ERR_INVALID_ARG;
    const bool dense = route == nullptr;
    if (int st = check_dims(M, H, dense ? 1 : E, dense ? 1 : k)) return st;
    if (I < 128 || I % 128 != 0 || I > kMaxI) return MOE_ERR_UNSUPPORTED;
    if (w2->fmt == MOE_FMT_BF16) {
        if (!dense) return MOE_ERR_UNSUPPORTED;
        if (!w2->w || !h_bf16) return MOE_ERR_INVALID_ARG;
        return hip_status(launch_down_bf16(dense_job(*w2, H, I, M), h_bf16, y, stream));
    }
    if (int st = check_fp4_weights(w2)) return st;
    if (!h_q || !h_s) return MOE_ERR_INVALID_ARG;
    if (!dense) {
        if (int st = check_routing(route)) return st;
        if (int st = check_pair_bytes(M, k, H)) return st;
    }
    const ExpertJob job = dense ? dense_job(*w2, H, I, M) : routed_job(*w2, H, I, *route, M, E, k);
    return hip_status(launch_down_fp4(job, h_q, h_s, y, stream));
}

int moe_expert_gate_up_nvfp4a(const moe_weights* w13, const uint8_t* a_q, const uint8_t* a_s, float a_global,
                              const moe_routing* route, int M, int H, int I, int E, int k, float swiglu_limit,
                              const float* h_globals, uint8_t* h_q, uint8_t* h_s, hipStream_t stream) {
    if (!w13 || !a_q || !a_s || !h_globals || !h_q || !h_s) return MOE_ERR_INVALID_ARG;
    if (!(swiglu_limit >= 0.0f)) return MOE_ERR_INVALID_ARG;
    if (!(a_global > 0.0f) || !(a_global <= 3.4e38f)) return MOE_ERR_INVALID_ARG;
    const bool dense = route == nullptr;
    if (int st = check_dims(M, H, dense ? 1 : E, dense ? 1 : k)) return st;
    if (I < 128 || I % 128 != 0 || I > kMaxI) return MOE_ERR_UNSUPPORTED;
    if (w13->fmt != MOE_FMT_NVFP4) return MOE_ERR_UNSUPPORTED;
    if (int st = check_fp4_weights(w13)) return st;
    if (!dense) {
        if (int st = check_routing(route)) return st;
        if (int st = check_pair_bytes(M, k, H)) return st;
    }
    ExpertJob job = dense ? dense_job(*w13, I, H, M) : routed_job(*w13, I, H, *route, M, E, k);
    job.swiglu_limit = swiglu_limit;
    job.a_nvfp4 = true;
    job.a_global = a_global;
    job.h_globals = h_globals;
    return hip_status(launch_gate_up_fp4(job, a_q, a_s, h_q, h_s, nullptr, stream));
}

int moe_expert_down_nvfp4a(const moe_weights* w2, const uint8_t* h_q, const uint8_t* h_s, const float* h_globals,
                           const moe_routing* route, int M, int H, int I, int E, int k, float* y, hipStream_t stream) {
    if (!w2 || !h_q || !h_s || !h_globals || !y) return MOE_ERR_INVALID_ARG;
    const bool dense = route == nullptr;
    if (int st = check_dims(M, H, dense ? 1 : E, dense ? 1 : k)) return st;
    if (I < 128 || I % 128 != 0 || I > kMaxI) return MOE_ERR_UNSUPPORTED;
    if (w2->fmt != MOE_FMT_NVFP4) return MOE_ERR_UNSUPPORTED;
    if (int st = check_fp4_weights(w2)) return st;
    if (!dense) {
        if (int st = check_routing(route)) return st;
        if (int st = check_pair_bytes(M, k, H)) return st;
    }
    ExpertJob job = dense ? dense_job(*w2, H, I, M) : routed_job(*w2, H, I, *route, M, E, k);
    job.a_nvfp4 = true;
    job.a_globals = h_globals;
    return hip_status(launch_down_fp4(job, h_q, h_s, y, stream));
}

int moe_expert_gate_up_fp8s(const moe_weights* w13, const uint16_t* x, float s_in, float s_h, int M, int H, int I,
                            float swiglu_limit, uint8_t* h_q, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
    if (!w13 || !x || !h_q) return MOE_ERR_INVALID_ARG;
    if (!static_scale_ok(s_in) || !static_scale_ok(s_h) || !(swiglu_limit >= 0.0f)) return MOE_ERR_INVALID_ARG;
    if (int st = check_dims(M, H, 1, 1)) return st;
    if (I < 128 || I % 128 != 0 || I > kMaxI) return MOE_ERR_UNSUPPORTED;
    if (w13->fmt != MOE_FMT_FP8S) return MOE_ERR_UNSUPPORTED;
    if (!w13->w || !w13->global_scale) return MOE_ERR_INVALID_ARG;
    const size_t need = gate_up_fp8s_partials_bytes(M, H, I);
    if (!workspace || !aligned256(workspace) || workspace_bytes < need) return MOE_ERR_WORKSPACE;
    ExpertJob job = dense_job(*w13, I, H, M);
    job.swiglu_limit = swiglu_limit;
    return hip_status(launch_gate_up_fp8s(job, x, s_in, s_h, h_q, static_cast<float*>(workspace), stream));
}

int moe_expert_down_fp8s(const moe_weights* w2, const uint8_t* h_q, float s_h, int M, int H, int I, float* y,
                         hipStream_t stream) {
    if (!w2 || !h_q || !y) return MOE_ERR_INVALID_ARG;
    if (!static_scale_ok(s_h)) return MOE_ERR_INVALID_ARG;
    if (int st = check_dims(M, H, 1, 1)) return st;
    if (I < 128 || I % 128 != 0 || I > kMaxI) return MOE_ERR_UNSUPPORTED;
    if (w2->fmt != MOE_FMT_FP8S) return MOE_ERR_UNSUPPORTED;
    if (!w2->w || !w2->global_scale) return MOE_ERR_INVALID_ARG;
    return hip_status(launch_down_fp8s(dense_job(*w2, H, I, M), h_q, s_h, y, stream));
}

int moe_finalize_rmsnorm_mxfp8(const float* y, const float* topk_w, const float* y_sh,
                               const uint16_t* residual, const uint16_t* gamma, float eps, int M, int H,
                               int k, uint16_t* out, uint16_t* residual_out, uint8_t* out_q, uint8_t* out_s,
                               hipStream_t stream) {
    if (!y || !topk_w || !residual || !gamma || !out || M < 1 || H < 1 || k < 1)
        return MOE_ERR_INVALID_ARG;
    if ((out_q == nullptr) != (out_s == nullptr)) return MOE_ERR_INVALID_ARG;
    if (H % 128 != 0 || H > kMaxH || k > kMaxK || M > kMaxM) return MOE_ERR_UNSUPPORTED;
    if (!(eps >= 0.0f)) return MOE_ERR_INVALID_ARG;
    return hip_status(
        launch_finalize(y, topk_w, y_sh, residual, gamma, eps, M, H, k, out, residual_out, out_q, out_s, stream));
}

int moe_finalize_rmsnorm(const float* y, const float* topk_w, const float* y_sh,
                         const uint16_t* residual, const uint16_t* gamma, float eps, int M, int H,
                         int k, uint16_t* out, uint16_t* residual_out, hipStream_t stream) {
    return moe_finalize_rmsnorm_mxfp8(y, topk_w, y_sh, residual, gamma, eps, M, H, k, out, residual_out, nullptr,
                                      nullptr, stream);
}

// ---- the whole layer --------------------------------------------------------

namespace {

// NVFP4 activations of a layer job: a gate_up reads x with its global and
// writes h with the expert's (routed: h_globals[e], shared: *sh_h_global); a
// down reads h with the same.
void set_a4(ExpertJob& j, const moe_layer_desc* d, bool shared, bool gate_up) {
    if (d->act_fmt != MOE_ACT_NVFP4) return;
    j.a_nvfp4 = true;
    const float* hg = shared ? d->sh_h_global : d->h_globals;
    if (gate_up) {
        j.a_global = d->x_global;
        j.h_globals = hg;
    } else {
        j.a_globals = hg;
    }
}

int check_desc(const moe_layer_desc* d) {
    if (!d) return MOE_ERR_INVALID_ARG;
    if (int st = check_dims(d->M, d->H, d->E, d->k)) return st;
    if (int st = check_pair_bytes(d->M, d->k, d->H)) return st;
    if (d->I < 128 || d->I % 128 != 0 || d->I > kMaxI) return MOE_ERR_UNSUPPORTED;
    if (!d->w_router || !d->gamma) return MOE_ERR_INVALID_ARG;
    if (!(d->eps >= 0.0f)) return MOE_ERR_INVALID_ARG;
    if (!(d->swiglu_limit >= 0.0f)) return MOE_ERR_INVALID_ARG;
    if (d->act_fmt != MOE_ACT_MXFP8 && d->act_fmt != MOE_ACT_NVFP4) return MOE_ERR_INVALID_ARG;
    if (d->act_fmt == MOE_ACT_NVFP4) {
        if (d->w13.fmt != MOE_FMT_NVFP4 || d->sh13.fmt == MOE_FMT_MXFP4) return MOE_ERR_UNSUPPORTED;
        if (!(d->x_global > 0.0f) || !(d->x_global <= 3.4e38f) || !d->h_globals) return MOE_ERR_INVALID_ARG;
        if (d->sh13.fmt == MOE_FMT_NVFP4 && !d->sh_h_global) return MOE_ERR_INVALID_ARG;
    }
    if (int st = check_fp4_weights(&d->w13)) return st;
    if (int st = check_fp4_weights(&d->w2)) return st;
    if (d->w13.fmt != d->w2.fmt) return MOE_ERR_UNSUPPORTED;
    const int sf = d->sh13.fmt;
    if (sf != d->sh2.fmt) return MOE_ERR_INVALID_ARG;
    if (sf != MOE_FMT_NONE) {
        if (d->I_sh < 128 || d->I_sh % 128 != 0 || d->I_sh > kMaxI) return MOE_ERR_UNSUPPORTED;
        if (sf == MOE_FMT_BF16) {
            if (!d->sh13.w || !d->sh2.w) return MOE_ERR_INVALID_ARG;
        } else if (sf == MOE_FMT_FP8S) {
            if (!d->sh13.w || !d->sh2.w || !d->sh13.global_scale || !d->sh2.global_scale) return MOE_ERR_INVALID_ARG;
            if (!static_scale_ok(d->sh_in_scale) || !static_scale_ok(d->sh_h_scale)) return MOE_ERR_INVALID_ARG;
        } else {
            if (int st = check_fp4_weights(&d->sh13)) return st;
            if (int st = check_fp4_weights(&d->sh2)) return st;
        }
    }
    return MOE_OK;
}

struct LayerWs {
    RouteWs route;
    int32_t *ids, *offsets, *bucket, *tile_e, *tile_b, *tile_r, *num_tiles, *active, *num_active, *act_off;
    float* w;
    uint8_t *xq, *xs, *xqt, *xst, *hq, *hs, *hsq, *hss;
    uint16_t* hsb;
    float* sh_part;
    float* part;     // routed gate_up split-K partials
    float* sh_fpart; // FP4 shared gate_up split-K partials
    float *y, *ysh;
    int32_t *r_act, *r_off, *r_na, *r_bkt;  // slots recorded by the few-pairs gate_up
    int2* yrec;                             // each pair's row of the grouped y
};

LayerWs carve_layer(Carver& c, const moe_layer_desc* d) {
    LayerWs L;
    const int M = d->M, H = d->H, E = d->E, k = d->k, I = d->I, Ish = d->I_sh;
    const int P = M * k;
    const int T = moe_tile_capacity(M, E, k);
    const bool sh = d->sh13.fmt != MOE_FMT_NONE;
    const bool shb = d->sh13.fmt == MOE_FMT_BF16;
    const bool sh8 = d->sh13.fmt == MOE_FMT_FP8S;
    L.route = carve_route(c, M, H, E);
    L.ids = c.take<int32_t>(P);
    L.w = c.take<float>(P);
    L.offsets = c.take<int32_t>(E + 1);
    L.bucket = c.take<int32_t>(P);
    L.tile_e = c.take<int32_t>(T);
    L.tile_b = c.take<int32_t>(T);
    L.tile_r = c.take<int32_t>(T);
    L.num_tiles = c.take<int32_t>(1);
    L.active = c.take<int32_t>(std::min(E, P));
    L.num_active = c.take<int32_t>(1);
    L.act_off = c.take<int32_t>(std::min(E, P) + 1);
    // token order: gate_up gathers its rows (and the FP4 shared expert reads them)
    L.xq = L.xs = nullptr;
    // scales: one byte per 32 values (MXFP8) or per 16 (NVFP4 activations)
    const int sdiv = d->act_fmt == MOE_ACT_NVFP4 ? 16 : 32;
    L.xqt = c.take<uint8_t>((size_t)M * H);
    L.xst = c.take<uint8_t>((size_t)M * H / sdiv);
    L.hq = c.take<uint8_t>((size_t)P * I);
    L.hs = c.take<uint8_t>((size_t)P * I / sdiv);
    L.hsq = L.hss = nullptr;
    L.hsb = nullptr;
    L.sh_part = nullptr;
    if (sh && !shb && !sh8) {
        L.hsq = c.take<uint8_t>((size_t)M * Ish);
        L.hss = c.take<uint8_t>((size_t)M * Ish / sdiv);
    }
    if (shb) {
        L.hsb = c.take<uint16_t>((size_t)M * Ish);
        L.sh_part = c.take<float>(gate_up_bf16_partials_bytes(M, H, Ish) / sizeof(float));
    }
    if (sh8) {  // static-FP8 h codes and the gate_up partial sums
        L.hsq = c.take<uint8_t>((size_t)M * Ish);
        L.sh_part = c.take<float>(gate_up_fp8s_partials_bytes(M, H, Ish) / sizeof(float));
    }
    {
        moe_weights w = d->w13;
        moe_routing r{};
        L.part = c.take<float>(gate_up_fp4_partials_bytes(routed_job(w, I, H, r, M, E, k)) / sizeof(float));
    }
    L.sh_fpart = nullptr;
    if (sh && !shb && !sh8)
        L.sh_fpart = c.take<float>(gate_up_fp4_partials_bytes(dense_job(d->sh13, Ish, H, M)) / sizeof(float));
    L.y = c.take<float>((size_t)P * H);
    L.ysh = sh ? c.take<float>((size_t)M * H) : nullptr;
    L.r_act = c.take<int32_t>(std::min(E, P));
    L.r_off = c.take<int32_t>(std::min(E, P) + 1);
    L.r_na = c.take<int32_t>(1);
    L.r_bkt = c.take<int32_t>(P);
    L.yrec = c.take<int2>(P);
    return L;
}

}  // namespace

size_t moe_layer_workspace_bytes(const moe_layer_desc* desc) {
    if (check_desc(desc) != MOE_OK) return 0;
    Carver c(nullptr);
    carve_layer(c, desc);
    return c.off;
}

int moe_layer_mxfp8_out(const moe_layer_desc* d, const uint16_t* x, const uint16_t* residual,
                        uint16_t* out, uint16_t* residual_out, uint8_t* out_q, uint8_t* out_s,
                        float* logits_out, int32_t* topk_ids_out, float* topk_w_out, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
    if (int st = check_desc(d)) return st;
    if (!x || !residual || !out) return MOE_ERR_INVALID_ARG;
    if ((out_q == nullptr) != (out_s == nullptr)) return MOE_ERR_INVALID_ARG;
    if (!workspace || !aligned256(workspace)) return MOE_ERR_WORKSPACE;
    Carver c(workspace);
    LayerWs L = carve_layer(c, d);
    if (c.off > workspace_bytes) return MOE_ERR_WORKSPACE;
    const int M = d->M, H = d->H, E = d->E, k = d->k, I = d->I, Ish = d->I_sh;
    const int sf = d->sh13.fmt;

    moe_routing r;
    r.topk_ids = topk_ids_out ? topk_ids_out : L.ids;
    r.topk_w = topk_w_out ? topk_w_out : L.w;
    r.expert_offsets = L.offsets;
    r.bucket = L.bucket;
    r.tile_expert = L.tile_e;
    r.tile_begin = L.tile_b;
    r.tile_rows = L.tile_r;
    r.num_tiles = L.num_tiles;
    r.active_experts = L.active;
    r.num_active = L.num_active;
    r.active_offsets = L.act_off;

    // A bf16 or static-FP8 shared expert does not depend on the routing: its
    // three stages run as extra workgroups of the router, top-k and
    // bucketing (or gate_up) launches; the static-FP8 gate/up in the router
    // launch (README Qwen3.5 slot table, row "route_shared"), its SiLU-and-mul
    // with the static FP8 quant of the down input in the top-k launch (PR #33
    // appended table, row "shared act quant").
    const bool sh8 = sf == MOE_FMT_FP8S;
    const bool shb = sf == MOE_FMT_BF16 || sh8;  // the shared expert rides as side stages
    ExpertJob sh_gu = dense_job(d->sh13, Ish, H, M);
    sh_gu.swiglu_limit = d->swiglu_limit;
    const bool a4 = d->act_fmt == MOE_ACT_NVFP4;
    const float xg4 = a4 ? d->x_global : 0.0f;
    if (sf == MOE_FMT_NVFP4) set_a4(sh_gu, d, true, true);
    const ExpertJob sh_dn = dense_job(d->sh2, H, Ish, M);
    const auto side = [&](const ExpertJob& j, float s_in, float s_out, int stage) {
        return sh8 ? fp8s_side(j, Ish, H, M, x, L.sh_part, L.hsq, L.ysh, s_in, s_out, stage)
                   : bf16_side(j, Ish, H, M, x, L.sh_part, L.hsb, L.ysh, stage);
    };
    const Bf16Side s1 = shb ? side(sh_gu, d->sh_in_scale, d->sh_h_scale, kBf16GateUp) : no_side();
    const Bf16Side s2 = shb ? side(sh_gu, d->sh_in_scale, d->sh_h_scale, kBf16Swiglu) : no_side();
    const Bf16Side s3 = shb ? side(sh_dn, d->sh_h_scale, 0.0f, kBf16Down) : no_side();
    const RouterPlan p = router_plan(M, H, E);
    const bool row_router = !shb && small_router(M, H, E);
    const bool fp4_shared = sf != MOE_FMT_NONE && !shb;
    if (M * k <= kIdsPairs) {
        // Five launches (four with a small router: router and top-k in one):
        // (router + token-order MXFP8 of x) -> top-k -> gate_up
        // (workgroups resolve their expert from the ids, in the route step's
        // order, and gather token rows; one per slot records it) -> down
        // (slots from the record) -> finalize.  No bucket or 8-row tiles are
        // materialized: nothing in these launches reads them.  The bf16 or
        // static-FP8 shared expert's stages ride along the first three.  A
        // large y is written grouped (ygroup_rec): gate_up's record gives the
        // finalize each pair's row.
        // a small router and its top-k take one launch (no shared stage to carry)
        hipError_t e;
        if (row_router) {
            e = launch_router_topk_row(x, d->w_router, d->router_bias, M, H, E, k, d->routed_scale, logits_out, r,
                                       L.xqt, L.xst, xg4, stream);
        } else {
            e = launch_router_partials(x, d->w_router, M, H, E, p, L.route.partials, L.xqt, L.xst, s1,
                                       shb ? kBf16GateUp : kBf16None, stream, xg4);
            if (e == hipSuccess)
                e = launch_topk(L.route.partials, p.splits, p.sp, d->router_bias, M, E, k, d->routed_scale, logits_out,
                                r, s2, shb ? kBf16Swiglu : kBf16None, stream);
        }
        ExpertJob gu = routed_job(d->w13, I, H, r, M, E, k);
        gu.swiglu_limit = d->swiglu_limit;
        set_a4(gu, d, false, true);
        gu.ids = r.topk_ids;
        gu.a_tok = true;
        const bool yg = y_grouped(M, k, H);
        const SlotRecord rec{L.r_act, L.r_off, L.r_na, L.r_bkt, yg ? L.yrec : nullptr};
        gu.record = &rec;
        // the FP4 shared expert rides along the routed launches
        const ExpertJob& sgu = sh_gu;
        ExpertJob sdn = dense_job(d->sh2, H, Ish, M);
        if (sf == MOE_FMT_NVFP4) set_a4(sdn, d, true, false);
        sdn.ygroup = yg;
        const SecondJob s_gu = fp4_shared ? SecondJob{&sgu, L.xqt, L.xst, L.hsq, L.hss, L.sh_fpart} : SecondJob{};
        const SecondDown s_dn = fp4_shared ? SecondDown{&sdn, L.hsq, L.hss, L.ysh} : SecondDown{};
        if (e == hipSuccess)
            e = launch_gate_up_fp4(gu, L.xqt, L.xst, L.hq, L.hs, L.part, stream, s3, shb ? kBf16Down : kBf16None,
                                   s_gu);
        // down resolves its slots from gate_up's record (one round of loads)
        ExpertJob dn = routed_job(d->w2, H, I, r, M, E, k);
        set_a4(dn, d, false, false);
        dn.active = rec.act;
        dn.active_offsets = rec.off;
        dn.bucket = rec.bkt;
        dn.count = rec.na;
        dn.ygroup = yg;
        if (e == hipSuccess) e = launch_down_fp4(dn, L.hq, L.hs, L.y, stream, s_dn);
        if (e == hipSuccess)
            e = launch_finalize(L.y, r.topk_w, L.ysh, residual, d->gamma, d->eps, M, H, k, out, residual_out,
                                out_q, out_s, stream, yg ? L.yrec : nullptr, fp4_shared && yg);
        return hip_status(e);
    }
    // Six launches (five with a small router): (router + token-order MXFP8
    // of x) -> top-k -> route step
    // -> gate_up (gathers each pass's token rows through the bucket) -> down
    // -> finalize.  A large y is written grouped: the route step gives the
    // finalize each pair's row.
    const bool yg = y_grouped(M, k, H);
    hipError_t e;
    if (row_router) {
        e = launch_router_topk_row(x, d->w_router, d->router_bias, M, H, E, k, d->routed_scale, logits_out, r, L.xqt,
                                   L.xst, xg4, stream);
        if (e == hipSuccess) e = launch_bucket(M, E, k, r, stream, H, yg ? L.yrec : nullptr);
    } else {
        e = launch_router_partials(x, d->w_router, M, H, E, p, L.route.partials, L.xqt, L.xst, s1,
                                   shb ? kBf16GateUp : kBf16None, stream, xg4);
        if (e == hipSuccess)
            e = launch_topk_bucket(L.route.partials, p.splits, p.sp, d->router_bias, M, E, k, d->routed_scale,
                                   logits_out, r, s2, shb ? kBf16Swiglu : kBf16None, s3, shb ? kBf16Down : kBf16None,
                                   stream, H, yg ? L.yrec : nullptr);
    }
    ExpertJob gu = routed_job(d->w13, I, H, r, M, E, k);
    gu.swiglu_limit = d->swiglu_limit;
    set_a4(gu, d, false, true);
    gu.a_tok = true;
    const ExpertJob& sgu = sh_gu;
    ExpertJob sdn = dense_job(d->sh2, H, Ish, M);
    if (sf == MOE_FMT_NVFP4) set_a4(sdn, d, true, false);
    sdn.ygroup = yg;
    const SecondJob s_gu = fp4_shared ? SecondJob{&sgu, L.xqt, L.xst, L.hsq, L.hss, L.sh_fpart} : SecondJob{};
    const SecondDown s_dn = fp4_shared ? SecondDown{&sdn, L.hsq, L.hss, L.ysh} : SecondDown{};
    if (e == hipSuccess)
        e = launch_gate_up_fp4(gu, L.xqt, L.xst, L.hq, L.hs, L.part, stream, no_side(), kBf16None, s_gu);
    ExpertJob dn = routed_job(d->w2, H, I, r, M, E, k);
    set_a4(dn, d, false, false);
    dn.ygroup = yg;
    if (e == hipSuccess) e = launch_down_fp4(dn, L.hq, L.hs, L.y, stream, s_dn);
    if (e == hipSuccess)
        e = launch_finalize(L.y, r.topk_w, L.ysh, residual, d->gamma, d->eps, M, H, k, out, residual_out,
                            out_q, out_s, stream, yg ? L.yrec : nullptr, fp4_shared && yg);
    return hip_status(e);
}

int moe_layer(const moe_layer_desc* d, const uint16_t* x, const uint16_t* residual,
              uint16_t* out, uint16_t* residual_out, float* logits_out, int32_t* topk_ids_out,
              float* topk_w_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return moe_layer_mxfp8_out(d, x, residual, out, residual_out, nullptr, nullptr, logits_out, topk_ids_out,
                               topk_w_out, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---- the layer without an allocation: a static scratch buffer per device ----

static_assert(MOE_NOALLOC_SCRATCH_BYTES % 256 == 0, "the scratch is carved at 256-byte boundaries");

// The scratch of moe_layer_noalloc.  In host code `scratch` names a host-side
// stand-in, not device memory: the kernels get its device address, which
// hipGetSymbolAddress resolves once per device (each device holds its own
// copy of the array, at its own address, until the process ends).
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device; null until its first call

// The scratch's device address on the current device, resolved on the first
// call there (with that device current).
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return MOE_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return MOE_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" int moe_layer_noalloc(const moe_layer_desc* d, const uint16_t* x, const uint16_t* residual,
                                 uint16_t* out, uint16_t* residual_out, float* logits_out,
                                 int32_t* topk_ids_out, float* topk_w_out, hipStream_t stream) {
    if (int st = check_desc(d)) return st;
    if (!x || !residual || !out) return MOE_ERR_INVALID_ARG;
    Carver c(nullptr);
    carve_layer(c, d);
    if (c.off > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
    void* ws = nullptr;
    if (int st = scratch_address(&ws)) return st;
    // every scratch region is written before it is read within the call (the
    // workspace of moe_layer needs no initialization), so the previous call's
    // contents are never seen
    return moe_layer_mxfp8_out(d, x, residual, out, residual_out, nullptr, nullptr, logits_out, topk_ids_out,
                               topk_w_out, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}
