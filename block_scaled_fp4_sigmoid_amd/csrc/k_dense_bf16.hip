// k_dense_bf16.hip — launches of the bf16 or static-FP8 shared expert (dense
// over all M rows) on its own: gate_up (+ the SwiGLU stage) and down.  The stages
// themselves are in dense_bf16_dev.h; the layer runs them as extra
// workgroups of its routing launches instead.
//
// Pages: sgl-nvidia-mega PR #24, "Modifications / Target spec" (NVFP4 routed
// experts beside a BF16 shared expert).
#include "dense_bf16_dev.h"
#include "moe_internal.h"

namespace moe {

// gate_up K splits: about 256 workgroups, at most 32 splits (the SwiGLU stage
// loads all of a value's partials in one round).
int bf16_splits(int H, int I) {
    const int cbs = I / 32;
    const int nsteps = H / 32;
    int splits = 1;
    for (int d = 1; d <= nsteps && d <= 32; ++d)
        if (nsteps % d == 0 && cbs * d <= 256) splits = d;
    return splits;
}

size_t gate_up_bf16_partials_bytes(int M, int H, int I) {
    return align_up((size_t)bf16_splits(H, I) * M * 2 * I * sizeof(float));
}

Bf16Side bf16_side(const ExpertJob& gate_up_or_down, int I, int H, int M, const uint16_t* x, float* part,
                   uint16_t* h, float* y, int stage) {
    Bf16Side S{};
    S.w = static_cast<const uint16_t*>(gate_up_or_down.w.w);
    S.I = I;
    S.H = H;
    S.M = M;
    S.splits = bf16_splits(H, I);
    S.x = x;
    S.part = part;
    S.h = h;
    S.y = y;
    S.limit = gate_up_or_down.swiglu_limit;
    S.blocks = stage == kBf16GateUp ? (I / 32) * S.splits
               : stage == kBf16Swiglu ? (M * I + 255) / 256
               : stage == kBf16Down ? H / 64
                                    : 0;
    return S;
}

// Static-FP8 gate_up K splits: over 128-K steps (the FP8 stage streams 64-K
// blocks), about 512 workgroups, at most 32 splits.  Twice the bf16 stage's
// workgroups: each one quantizes its x slice on the fly, a chain of divisions
// that shorter slices cut (W4A4 verify step 79.6 -> 78.8 us; the bf16 stage,
// which only loads its x, gets slower with more splits: skew 198 -> 201 us).
int fp8s_splits(int H, int I) {
    const int cbs = I / 32;
    const int nsteps = H / 128;
    int splits = 1;
    for (int d = 1; d <= nsteps && d <= 32; ++d)
        if (nsteps % d == 0 && cbs * d <= 512) splits = d;
    return splits;
}

size_t gate_up_fp8s_partials_bytes(int M, int H, int I) {
    return align_up((size_t)fp8s_splits(H, I) * M * 2 * I * sizeof(float));
}

Bf16Side fp8s_side(const ExpertJob& gate_up_or_down, int I, int H, int M, const uint16_t* x, float* part,
                   uint8_t* hq, float* y, float s_in, float s_out, int stage) {
    Bf16Side S{};
    S.fp8 = 1;
    S.w8 = static_cast<const uint8_t*>(gate_up_or_down.w.w);
    S.wscale = gate_up_or_down.w.global_scale;
    S.I = I;
    S.H = H;
    S.M = M;
    S.splits = fp8s_splits(H, I);
    S.x = x;
    S.part = part;
    S.hq = hq;
    S.y = y;
    S.s_in = s_in;
    S.s_out = s_out;
    S.limit = gate_up_or_down.swiglu_limit;
    S.blocks = stage == kBf16GateUp ? (I / 32) * S.splits
               : stage == kBf16Swiglu ? (M * I + 255) / 256
               : stage == kBf16Down ? H / 64
                                    : 0;
    return S;
}

__global__ __launch_bounds__(256) void k_bf16_stage(Bf16Side S, int stage) {
    bf16_side_block(S, stage, blockIdx.x);
}

static hipError_t launch_stage(const Bf16Side& S, int stage, hipStream_t stream) {
    hipLaunchKernelGGL(k_bf16_stage, dim3(S.blocks), dim3(256), 0, stream, S, stage);
    return hipGetLastError();
}

hipError_t launch_gate_up_bf16(const ExpertJob& job, const uint16_t* a, uint16_t* h, float* part,
                               hipStream_t stream) {
    const int I = job.N_out, H = job.K, M = job.M;
    hipError_t e = launch_stage(bf16_side(job, I, H, M, a, part, h, nullptr, kBf16GateUp), kBf16GateUp, stream);
    if (e != hipSuccess) return e;
    return launch_stage(bf16_side(job, I, H, M, a, part, h, nullptr, kBf16Swiglu), kBf16Swiglu, stream);
}

hipError_t launch_down_bf16(const ExpertJob& job, const uint16_t* h, float* y, hipStream_t stream) {
    const int H = job.N_out, I = job.K, M = job.M;
    return launch_stage(bf16_side(job, I, H, M, nullptr, nullptr, const_cast<uint16_t*>(h), y, kBf16Down), kBf16Down,
                        stream);
}

hipError_t launch_gate_up_fp8s(const ExpertJob& job, const uint16_t* x, float s_in, float s_h, uint8_t* hq,
                               float* part, hipStream_t stream) {
    const int I = job.N_out, H = job.K, M = job.M;
    hipError_t e = launch_stage(fp8s_side(job, I, H, M, x, part, hq, nullptr, s_in, s_h, kBf16GateUp), kBf16GateUp,
                                stream);
    if (e != hipSuccess) return e;
    return launch_stage(fp8s_side(job, I, H, M, x, part, hq, nullptr, s_in, s_h, kBf16Swiglu), kBf16Swiglu, stream);
}

hipError_t launch_down_fp8s(const ExpertJob& job, const uint8_t* hq, float s_h, float* y, hipStream_t stream) {
    const int H = job.N_out, I = job.K, M = job.M;
    return launch_stage(fp8s_side(job, I, H, M, nullptr, nullptr, const_cast<uint8_t*>(hq), y, s_h, 0.0f, kBf16Down),
                        kBf16Down, stream);
}

}  // namespace moe
