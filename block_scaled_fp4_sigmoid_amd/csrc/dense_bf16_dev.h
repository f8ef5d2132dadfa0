// dense_bf16_dev.h — the bf16 and the static-FP8 shared expert (dense over
// all M rows) as device functions of one workgroup each, so their three
// stages can run either as launches of their own or as extra workgroups of
// the routing launches (they do not depend on the routing).
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

// The pass's row indices (-1 past the rows): one LDS array that every stage
// below shares, so a launch carrying any stage holds only these 256 bytes.
__device__ __forceinline__ int* side_rows_lds() {
    __shared__ int s_row[kBf16Pass];
    return s_row;
}

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
    int* s_row = side_rows_lds();
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
    int* s_row = side_rows_lds();
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

// ---- the static-FP8 shared expert -------------------------------------------
// README Qwen3.5 slot table, row "route_shared (with route)": the shared
// expert's static-FP8 gate/up rides the router front's launch; sgl-nvidia-mega
// PR #33, appended table, row "shared act quant": its SiLU-and-mul is fused
// with the static FP8 quantization of the down input.  Weights are E4M3 codes
// with one fp32 scale per matrix.  An input value v (bf16) becomes the E4M3
// code (round to nearest even, saturating at 448, NaN kept) of the correctly
// rounded fp32 quotient v / s_in; a linear's output is s_in * scale * the sum
// of the code products (exact products, fp32 sums).  The gate/up outputs and
// h are rounded to bf16, the linear's dtype, and h is quantized like the
// input with the down projection's static scale.
//
// v_mfma_f32_16x16x32_fp8_fp8 takes its operands like the bf16 instruction
// (lane (i, g) holds 8 K values of row / column i); a lane loads 16 weight
// bytes, K [16g, 16g + 16) of a 64-K block, and feeds the block's first MFMA
// the low 8 and its second the high 8.  The activation operands use the same
// K placement: the MFMA sums over K, so only the agreement of A and B counts.
// No LDS beyond the shared row list: a stage rides launches whose own LDS
// budget it must not raise.

// Two values -> two E4M3 codes (16 bits): nearest even, saturating at 448
// (the conversion rounds to nearest even below 448 and overflows to NaN from
// 464 up, so clamp first), NaN kept as the NaN code with its sign.
__device__ __forceinline__ uint32_t e4m3x2_static(float a, float b) {
    const uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(a, -448.0f), 448.0f),
                                                                 fminf(fmaxf(b, -448.0f), 448.0f), 0, false) &
                       0xffffu;
    const uint32_t na = ((__float_as_uint(a) >> 24) & 0x80u) | 0x7Fu;
    const uint32_t nb = ((__float_as_uint(b) >> 24) & 0x80u) | 0x7Fu;
    const uint32_t lo = a != a ? na : (r & 0xffu);
    const uint32_t hi = b != b ? nb : (r >> 8);
    return lo | (hi << 8);
}

// 8 bf16 values -> their 8 static-FP8 codes (v / s_in), as one MFMA operand.
__device__ __forceinline__ long static_fp8x8(const v4i& v, float s_in) {
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t d0 = (uint32_t)v[2 * h], d1 = (uint32_t)v[2 * h + 1];
        const uint32_t c0 = e4m3x2_static(__fdiv_rn(bf16_to_f32(d0 & 0xffffu), s_in),
                                          __fdiv_rn(bf16_to_f32(d0 >> 16), s_in));
        const uint32_t c1 = e4m3x2_static(__fdiv_rn(bf16_to_f32(d1 & 0xffffu), s_in),
                                          __fdiv_rn(bf16_to_f32(d1 >> 16), s_in));
        w[h] = c0 | (c1 << 16);
    }
    return (long)(((uint64_t)w[1] << 32) | w[0]);
}

__device__ __forceinline__ long lo64(const v4i& v) { return (long)(((uint64_t)(uint32_t)v.y << 32) | (uint32_t)v.x); }
__device__ __forceinline__ long hi64(const v4i& v) { return (long)(((uint64_t)(uint32_t)v.w << 32) | (uint32_t)v.z); }

// E4M3 weights x activations over K range [k0, k1) (multiples of 64) for NB
// N-blocks.  QUANT: act is bf16 [rows][K], quantized with s_in on the fly;
// else act is E4M3 codes [rows][K].  Loads of 4 64-K blocks are issued
// together; no branch separates an MFMA from the read of its accumulator.
template <int NB, bool QUANT>
__device__ __forceinline__ void wave_gemm_fp8s(const uint8_t* __restrict__ wrow, const void* __restrict__ act,
                                               int K, int k0, int k1, const int* s_row, float s_in,
                                               v4f (&acc)[4]) {
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, g = lane >> 4;
    int rowj[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) rowj[j] = s_row[16 * j + m];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
    // Blocks past k1 and rows past the pass load from an in-bounds place (the
    // range's first block, row 0) and are replaced by zeros with a select:
    // every load is unconditional, so no branch sits between the MFMAs.
    // Quantizing on the fly keeps two blocks in flight (four need twice the
    // registers, which the launches this stage rides along cannot spare).
    constexpr int U = QUANT ? 2 : 4;
    const v4i zero = {0, 0, 0, 0};
    for (int kb = k0; kb < k1; kb += 64 * U) {
        v4i a[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kk = kb + 64 * u;
            const v4i w = load16_nt(wrow + (kk < k1 ? kk : k0) + 16 * g);
            a[u] = kk < k1 ? w : zero;
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            long b0[U], b1[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int kk = kb + 64 * u;
                const bool ok = rowj[j] >= 0 && kk < k1;
                const int kc = (ok ? kk : k0) + 16 * g;
                if constexpr (QUANT) {
                    const uint16_t* xr = static_cast<const uint16_t*>(act) + (size_t)(ok ? rowj[j] : 0) * K;
                    const v4i x0 = load16(xr + kc), x1 = load16(xr + kc + 8);
                    b0[u] = static_fp8x8(ok ? x0 : zero, s_in);
                    b1[u] = static_fp8x8(ok ? x1 : zero, s_in);
                } else {
                    const uint8_t* hr = static_cast<const uint8_t*>(act) + (size_t)(ok ? rowj[j] : 0) * K;
                    const v4i hv = load16(hr + kc);
                    b0[u] = lo64(ok ? hv : zero);
                    b1[u] = hi64(ok ? hv : zero);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(lo64(a[u]), b0[u], acc[j], 0, 0, 0);
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(hi64(a[u]), b1[u], acc[j], 0, 0, 0);
            }
        }
    }
}

template <int NB, bool QUANT>
__device__ __forceinline__ void wave_gemm_fp8s_nb(int nb, const uint8_t* wrow, const void* act, int K, int k0,
                                                  int k1, const int* s_row, float s_in, v4f (&acc)[4]) {
    if constexpr (NB > 1)
        if (nb < NB) return wave_gemm_fp8s_nb<NB - 1, QUANT>(nb, wrow, act, K, k0, k1, s_row, s_in, acc);
    wave_gemm_fp8s<NB, QUANT>(wrow, act, K, k0, k1, s_row, s_in, acc);
}

// gate_up workgroup bid of (I/32) x splits: raw partial sums (codes times
// codes times the weight scale left out), rows [0, I) gate, [I, 2I) up.
// Passes of 16 rows (one N-block: the on-the-fly quant's registers); a later
// pass reads the workgroup's weights again, from the cache.
__device__ inline void fp8s_gate_up_block(const Bf16Side& S, int bid) {
    const int I = S.I, H = S.H, M = S.M;
    const int cb = bid / S.splits, ks = bid % S.splits;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int m = lane & 15, g = lane >> 4;
    const int wr = (wave >> 1) * I + cb * 32 + (wave & 1) * 16 + m;
    const uint8_t* wrow = S.w8 + (size_t)wr * H;
    const int kc = H / S.splits;
    int* s_row = side_rows_lds();
    for (int t0 = 0; t0 < M; t0 += 16) {
        const int npass = min(16, M - t0);
        if (threadIdx.x < 16) s_row[threadIdx.x] = threadIdx.x < npass ? t0 + threadIdx.x : -1;
        __syncthreads();
        v4f acc[4];
        wave_gemm_fp8s<1, true>(wrow, S.x, H, ks * kc, (ks + 1) * kc, s_row, S.s_in, acc);
        if (m < npass) {
            const int col = (wave >> 1) * I + cb * 32 + (wave & 1) * 16 + 4 * g;
            *reinterpret_cast<v4f*>(S.part + ((size_t)ks * M + t0 + m) * (2 * I) + col) = acc[0];
        }
        __syncthreads();
    }
}

__device__ __forceinline__ float bf16_round(float v) { return bf16_to_f32(f32_to_bf16_rne(v)); }

// SwiGLU + the static FP8 quant of the down input: workgroup bid covers 256
// consecutive (row, column) entries of h.
__device__ inline void fp8s_actq_block(const Bf16Side& S, int bid) {
    const int I = S.I, M = S.M, splits = S.splits;
    const int idx = bid * 256 + threadIdx.x;
    if (idx >= M * I) return;
    const int t = idx / I, col = idx % I;
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
    const float sc = S.s_in * S.wscale[0];
    const float hv = bf16_round(swiglu(bf16_round(gt * sc), bf16_round(up * sc), S.limit));
    S.hq[(size_t)t * I + col] = (uint8_t)(e4m3x2_static(__fdiv_rn(hv, S.s_out), 0.0f) & 0xffu);
}

// down workgroup bid of H/64: 64 output features over all rows.
__device__ inline void fp8s_down_block(const Bf16Side& S, int bid) {
    const int H = S.H, I = S.I, M = S.M;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int m = lane & 15, g = lane >> 4;
    const int f0 = bid * 64 + wave * 16;
    const uint8_t* wrow = S.w8 + (size_t)(f0 + m) * I;
    const float sc = S.s_in * S.wscale[0];
    int* s_row = side_rows_lds();
    for (int t0 = 0; t0 < M; t0 += kBf16Pass) {
        const int npass = min(kBf16Pass, M - t0);
        const int nb = (npass + 15) / 16;
        if (threadIdx.x < kBf16Pass) s_row[threadIdx.x] = threadIdx.x < npass ? t0 + threadIdx.x : -1;
        __syncthreads();
        v4f acc[4];
        wave_gemm_fp8s_nb<4, false>(nb, wrow, S.hq, I, 0, I, s_row, 0.0f, acc);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = 16 * j + m;
            if (j < nb && t < npass) *reinterpret_cast<v4f*>(S.y + (size_t)(t0 + t) * H + f0 + 4 * g) = acc[j] * sc;
        }
        __syncthreads();
    }
}

__device__ inline void bf16_side_block(const Bf16Side& S, int stage, int bid) {
    if (S.fp8) {
        if (stage == kBf16GateUp)
            fp8s_gate_up_block(S, bid);
        else if (stage == kBf16Swiglu)
            fp8s_actq_block(S, bid);
        else if (stage == kBf16Down)
            fp8s_down_block(S, bid);
        return;
    }
    if (stage == kBf16GateUp)
        bf16_gate_up_block(S, bid);
    else if (stage == kBf16Swiglu)
        bf16_swiglu_block(S, bid);
    else if (stage == kBf16Down)
        bf16_down_block(S, bid);
}

}  // namespace moe
