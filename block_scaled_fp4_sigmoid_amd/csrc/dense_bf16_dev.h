// dense_bf16_dev.h — the bf16 shared expert (dense over all M rows) as device
// functions of one workgroup each, so its three stages can run either as
// launches of their own or as extra workgroups of the routing launches (they
// do not depend on the routing).
//
// Pages: sgl-nvidia-mega PR #24, "Modifications / Target spec" (NVFP4 routed
// experts beside a BF16 shared expert); SGLang-NVIDIA-Mega README,
// DeepSeek-V4.1 slot table, rows "hop_b" / "two_shot" (the shared expert's
// output is added in the finalize).
//
// Stages: gate_up splits K over S workgroups per 32-column block and writes
// fp32 partials; the SwiGLU stage adds them in split order (deterministic),
// applies SwiGLU and rounds h to bf16; down computes y = h W2^T.  Stages are
// separated by launch boundaries, so every partial is visible without a
// device-scope fence (on this GPU such a fence writes back the L2 and costs
// far more than a launch).
//
// Operand layout (checked on the hardware): v_mfma_f32_16x16x32_bf16, lane
// (i, g) holds K [8g, 8g+8) of row/column i; output lane l holds
// D[4(l/16)+r][l%16], r = 0..3.
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kBf16Pass = 64;  // rows per pass: 4 N-blocks of 16

// bf16 A x bf16 B over K range [k0, k1) (multiple of 32) for NB N-blocks.
// Loads for 8 K-steps are issued together before their MFMAs; NB is a
// compile-time constant, so no branch separates an MFMA from the read of its
// accumulator.
template <int NB>
__device__ __forceinline__ void wave_gemm_bf16(const uint16_t* __restrict__ wrow,
                                               const uint16_t* __restrict__ act, int K, int k0, int k1,
                                               const int* s_row, v4f (&acc)[4]) {
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, g = lane >> 4;
    int rowj[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) rowj[j] = s_row[16 * j + m];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
    constexpr int U = 8;
    for (int kb = k0; kb < k1; kb += 32 * U) {
        v4i a[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kk = kb + 32 * u;
            a[u] = (kk < k1) ? load16_nt(wrow + kk + 8 * g) : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            v4i b[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int kk = kb + 32 * u;
                b[u] = (rowj[j] >= 0 && kk < k1) ? load16(act + (size_t)rowj[j] * K + kk + 8 * g) : v4i{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[u]),
                                                                 __builtin_bit_cast(v8bf, b[u]), acc[j], 0, 0, 0);
        }
    }
}

template <int NB>
__device__ __forceinline__ void wave_gemm_bf16_nb(int nb, const uint16_t* wrow, const uint16_t* act, int K,
                                                  int k0, int k1, const int* s_row, v4f (&acc)[4]) {
    if constexpr (NB > 1)
        if (nb < NB) return wave_gemm_bf16_nb<NB - 1>(nb, wrow, act, K, k0, k1, s_row, acc);
    wave_gemm_bf16<NB>(wrow, act, K, k0, k1, s_row, acc);
}

// gate_up workgroup bid of (I/32) x splits: rows [0, I) gate, [I, 2I) up.
__device__ inline void bf16_gate_up_block(const Bf16Side& S, int bid) {
    const int I = S.I, H = S.H, M = S.M;
    const int cb = bid / S.splits, ks = bid % S.splits;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int m = lane & 15, g = lane >> 4;
    const int wr = (wave >> 1) * I + cb * 32 + (wave & 1) * 16 + m;
    const uint16_t* wrow = S.w + (size_t)wr * H;
    const int kc = H / S.splits;
    __shared__ int s_row[kBf16Pass];
    for (int t0 = 0; t0 < M; t0 += kBf16Pass) {
        const int npass = min(kBf16Pass, M - t0);
        const int nb = (npass + 15) / 16;
        if (threadIdx.x < kBf16Pass) s_row[threadIdx.x] = threadIdx.x < npass ? t0 + threadIdx.x : -1;
        __syncthreads();
        v4f acc[4];
        wave_gemm_bf16_nb<4>(nb, wrow, S.x, H, ks * kc, (ks + 1) * kc, s_row, acc);
        // partial G: [split][row][2I]; this lane: features wr-block rows 4g+r
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = 16 * j + m;
            if (j < nb && t < npass) {
                const int col = (wave >> 1) * I + cb * 32 + (wave & 1) * 16 + 4 * g;
                *reinterpret_cast<v4f*>(S.part + ((size_t)ks * M + t0 + t) * (2 * I) + col) = acc[j];
            }
        }
        __syncthreads();
    }
}

// SwiGLU workgroup bid: 256 consecutive (row, column) entries of h.
__device__ inline void bf16_swiglu_block(const Bf16Side& S, int bid) {
    const int I = S.I, M = S.M, splits = S.splits;
    const int idx = bid * 256 + threadIdx.x;
    if (idx >= M * I) return;
    const int t = idx / I, col = idx % I;
    // all partials in one round of loads (splits <= 32), added in split order
    float pg[32], pu[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) {
        const float* pr = S.part + ((size_t)(u < splits ? u : 0) * M + t) * (2 * I);
        pg[u] = u < splits ? pr[col] : 0.f;
        pu[u] = u < splits ? pr[I + col] : 0.f;
    }
    float gt = pg[0], up = pu[0];
#pragma unroll
    for (int u = 1; u < 32; ++u) {
        if (u < splits) {
            gt += pg[u];
            up += pu[u];
        }
    }
    const float hv = swiglu(gt, up, S.limit);
    S.h[(size_t)t * I + col] = (uint16_t)f32_to_bf16_rne(hv);
}

// down workgroup bid of H/64: 64 output features over all rows.
__device__ inline void bf16_down_block(const Bf16Side& S, int bid) {
    const int H = S.H, I = S.I, M = S.M;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int m = lane & 15, g = lane >> 4;
    const int f0 = bid * 64 + wave * 16;
    const uint16_t* wrow = S.w + (size_t)(f0 + m) * I;
    __shared__ int s_row[kBf16Pass];
    for (int t0 = 0; t0 < M; t0 += kBf16Pass) {
        const int npass = min(kBf16Pass, M - t0);
        const int nb = (npass + 15) / 16;
        if (threadIdx.x < kBf16Pass) s_row[threadIdx.x] = threadIdx.x < npass ? t0 + threadIdx.x : -1;
        __syncthreads();
        v4f acc[4];
        wave_gemm_bf16_nb<4>(nb, wrow, S.h, I, 0, I, s_row, acc);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = 16 * j + m;
            if (j < nb && t < npass) *reinterpret_cast<v4f*>(S.y + (size_t)(t0 + t) * H + f0 + 4 * g) = acc[j];
        }
        __syncthreads();
    }
}

__device__ inline void bf16_side_block(const Bf16Side& S, int stage, int bid) {
    if (stage == kBf16GateUp)
        bf16_gate_up_block(S, bid);
    else if (stage == kBf16Swiglu)
        bf16_swiglu_block(S, bid);
    else if (stage == kBf16Down)
        bf16_down_block(S, bid);
}

}  // namespace moe
