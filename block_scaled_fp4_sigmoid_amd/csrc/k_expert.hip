// k_expert.hip — expert GEMMs of the MoE layer on gfx950 matrix cores:
// gate_up + SwiGLU + MXFP8 requant, and down, for MXFP4 / NVFP4 experts and
// for a bf16 shared expert.
//
// Pages: SGLang-NVIDIA-Mega README, DeepSeek-V4.1 slot table, row "Routed
// experts (moe)" (a pair of block-scaled GEMMs over 8-row tiles; an expert
// with more than 8 rows takes several tiles); README Qwen3.5 slot table, row
// "mkm" (FC1, SwiGLU, requant, FC2); sgl-nvidia-mega PR #24, "Modifications /
// Target spec" (NVFP4 routed experts beside a BF16 shared expert); SGLang Spark
// GB10 Optimizations, section 1 (NVFP4 K-groups of 16, FP8 scale rows) and
// section 4 (a sparse FP4 GEMV for MoE decode).
//
// Work decomposition (weight streaming, HBM-bound): one workgroup per (active
// expert, block of output features) covering ALL rows routed to that expert,
// so every expert weight byte is read once per call no matter how many 8-row
// tiles the expert has; rows are consumed 16 at a time (two 8-row tiles) as
// the N side of the MFMA, with weights on the M side.
//
// Operand layouts (checked on the hardware):
//   v_mfma_scale_f32_16x16x128_f8f6f4, FP4 operand: lane (row i, group g)
//     holds K [32g, 32g+32) as 16 packed bytes; FP8 operand: lane (col n, g)
//     holds K [16g, 16g+16) in bytes 0-15 and K [64+16g, 64+16g+16) in bytes
//     16-31; the E8M0 scale of (row/col i, K block b) comes from lane 16b+i.
//   v_mfma_f32_16x16x32_{f16,bf16}: lane (i, g) holds K [8g, 8g+8).
//   Output D (16x16): lane l holds D[4(l/16)+r][l%16], r = 0..3.
#include "moe_device.h"
#include "moe_internal.h"

#include <algorithm>

namespace moe {

struct JobDev {
    const uint8_t* w;        // packed FP4 or bf16 bytes
    const uint8_t* scales;
    const float* gscale;
    int N_out, K;
    int dense;
    const int32_t* offsets;
    const int32_t* bucket;
    const int32_t* active;
    const int32_t* num_active;
    int slots, k, M;
};

static JobDev to_dev(const ExpertJob& j) {
    JobDev d;
    d.w = static_cast<const uint8_t*>(j.w.w);
    d.scales = j.w.scales;
    d.gscale = j.w.global_scale;
    d.N_out = j.N_out;
    d.K = j.K;
    d.dense = j.dense ? 1 : 0;
    d.offsets = j.offsets;
    d.bucket = j.bucket;
    d.active = j.active;
    d.num_active = j.num_active;
    d.slots = j.slots;
    d.k = j.k;
    d.M = j.M;
    return d;
}

struct Tokens {
    int e, base, n;
};

__device__ __forceinline__ bool resolve(const JobDev& J, int slot, Tokens& t) {
    if (J.dense) {
        t.e = 0;
        t.base = 0;
        t.n = J.M;
        return true;
    }
    if (slot >= *J.num_active) return false;
    const int e = J.active[slot];
    t.e = e;
    t.base = J.offsets[e];
    t.n = J.offsets[e + 1] - t.base;
    return true;
}

constexpr int kFmtMX = MOE_FMT_MXFP4;
constexpr int kFmtNV = MOE_FMT_NVFP4;
constexpr int kPass = 64;  // rows per pass: 4 N-blocks of 16

// E4M3 scale code -> (fp32 value used for its exponent, f16 mantissa factor):
// value = 2^floor(log2 v) * m, m in [1, 2); zero -> m = 0; NaN -> m = NaN.
__device__ __forceinline__ void nv_scale_split(uint32_t code, float& sv, _Float16& m) {
    sv = __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
    const uint32_t b = __float_as_uint(sv);
    if ((b & 0x7fffffffu) == 0u) {
        m = (_Float16)0.0f;
    } else if ((b & 0x7f800000u) == 0x7f800000u) {
        m = (_Float16)__uint_as_float(0x7fc00000u);
    } else {
        m = (_Float16)__uint_as_float((b & 0x007fffffu) | 0x3f800000u);
    }
}

// 8 packed E2M1 (one dword) -> 8 f16 = e2m1 * 2^floor(log2 sv) * m (exact).
__device__ __forceinline__ v8h nv_dequant8(uint32_t w, float sv, _Float16 m) {
    const v2h mm = {m, m};
    v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sv, 0) * mm;
    v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sv, 1) * mm;
    v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sv, 2) * mm;
    v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sv, 3) * mm;
    return v8h{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// 8 E4M3 activation codes (two dwords) -> 8 f16 scaled by 2^floor(log2 sf).
__device__ __forceinline__ v8h fp8x8_to_f16(uint32_t d0, uint32_t d1, float sf) {
    const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, sf, false);
    const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, sf, true);
    const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, sf, false);
    const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, sf, true);
    return v8h{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Largest E8M0 scale code of each pass row (NVFP4 path: activations enter the
// f16 MFMA as E4M3 * 2^(s - smax), which stays within f16 range).
__device__ void pass_row_smax(const uint8_t* act_s, int K, const int* s_row, int npass,
                              int* s_smax) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nsd = K / 128;  // scale dwords per row
    for (int tt = 0; tt < 16; ++tt) {
        const int t = wave * 16 + tt;
        if (t >= npass) break;
        const uint32_t* sr = reinterpret_cast<const uint32_t*>(act_s + (size_t)s_row[t] * (K / 32));
        uint32_t mx = 0;
        for (int d = lane; d < nsd; d += 64) {
            const uint32_t v = sr[d];
            mx = max(mx, max(max(v & 0xffu, (v >> 8) & 0xffu), max((v >> 16) & 0xffu, v >> 24)));
        }
        for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
        if (lane == 0) s_smax[t] = (int)mx;
    }
}

// One wave's 16 weight rows x (up to 4) N-blocks of pass rows, full K.
// wrow: packed row of this lane (row i = lane%16); srow: its scale row.
template <int FMT>
__device__ __forceinline__ void wave_gemm_fp4(const uint8_t* __restrict__ wrow,
                                              const uint8_t* __restrict__ srow,
                                              const uint8_t* __restrict__ act_q,
                                              const uint8_t* __restrict__ act_s, int K,
                                              const int* s_row, const int* s_smax, int nb,
                                              v4f acc[4]) {
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, g = lane >> 4;
    int rowj[4];
    uint32_t smaxj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        rowj[j] = (j < nb) ? s_row[16 * j + m] : -1;
        smaxj[j] = (FMT == kFmtNV && rowj[j] >= 0) ? (uint32_t)s_smax[16 * j + m] : 0u;
        acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    const int steps = K / 128;
#pragma unroll 2
    for (int s = 0; s < steps; ++s) {
        const v4i a = load16_nt(wrow + 64 * s + 16 * g);
        if constexpr (FMT == kFmtMX) {
            const uint32_t sa = *reinterpret_cast<const uint32_t*>(srow + 4 * s) >> (8 * g);
            const v8i A = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (j < nb) {
                    v8i B = {0, 0, 0, 0, 0, 0, 0, 0};
                    uint32_t sb = 127u;
                    if (rowj[j] >= 0) {
                        const uint8_t* xr = act_q + (size_t)rowj[j] * K + 128 * s + 16 * g;
                        const v4i b0 = load16(xr), b1 = load16(xr + 64);
                        B = v8i{b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
                        sb = *reinterpret_cast<const uint32_t*>(act_s + (size_t)rowj[j] * (K / 32) + 4 * s) >> (8 * g);
                    }
                    acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc[j], 4, 0, 0, (int)sa, 0, (int)sb);
                }
            }
        } else {
            const uint32_t sc2 = *reinterpret_cast<const uint16_t*>(srow + 8 * s + 2 * g);
            float sv0, sv1;
            _Float16 m0, m1;
            nv_scale_split(sc2 & 0xffu, sv0, m0);
            nv_scale_split(sc2 >> 8, sv1, m1);
            const v8h A0 = nv_dequant8((uint32_t)a.x, sv0, m0);
            const v8h A1 = nv_dequant8((uint32_t)a.y, sv0, m0);
            const v8h A2 = nv_dequant8((uint32_t)a.z, sv1, m1);
            const v8h A3 = nv_dequant8((uint32_t)a.w, sv1, m1);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (j < nb) {
                    v8h B0 = {}, B1 = {}, B2 = {}, B3 = {};
                    if (rowj[j] >= 0) {
                        const uint8_t* xr = act_q + (size_t)rowj[j] * K + 128 * s + 32 * g;
                        const v4i b0 = load16(xr), b1 = load16(xr + 16);
                        const uint32_t sb = (*reinterpret_cast<const uint32_t*>(act_s + (size_t)rowj[j] * (K / 32) + 4 * s) >> (8 * g)) & 0xffu;
                        const int de = max((int)sb - (int)smaxj[j], -126);
                        const float sf = exp2i(de);
                        B0 = fp8x8_to_f16((uint32_t)b0.x, (uint32_t)b0.y, sf);
                        B1 = fp8x8_to_f16((uint32_t)b0.z, (uint32_t)b0.w, sf);
                        B2 = fp8x8_to_f16((uint32_t)b1.x, (uint32_t)b1.y, sf);
                        B3 = fp8x8_to_f16((uint32_t)b1.z, (uint32_t)b1.w, sf);
                    }
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, B0, acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, B1, acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A2, B2, acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A3, B3, acc[j], 0, 0, 0);
                }
            }
        }
    }
}

// Per-row factor that turns an NVFP4 accumulator into the product value:
// 2^(smax - 127) (activation offset) * global.
__device__ __forceinline__ float nv_row_factor(int smax, float gs) { return ldexpf(gs, smax - 127); }

// Quantize 8 consecutive h values (part q4 of a 32-value block shared by 4
// consecutive lanes) to MXFP8; returns the 8 codes, writes the scale code.
__device__ __forceinline__ uint2 mx_quant8_group4(const float hv[8], uint8_t& scale_out) {
    uint32_t amax = 0;
    int special = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint32_t b = __float_as_uint(hv[c]) & 0x7fffffffu;
        amax = max(amax, b);
        special |= f32_bits_special(b) ? 1 : 0;
    }
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1, 64));
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2, 64));
    special |= __shfl_xor(special, 1, 64);
    special |= __shfl_xor(special, 2, 64);
    uint32_t w0 = 0, w1 = 0;
    if (special) {
        scale_out = 0xff;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const uint32_t code = ((__float_as_uint(hv[c]) >> 24) & 0x80u) | 0x7fu;
            if (c < 4) w0 |= code << (8 * c);
            else w1 |= code << (8 * (c - 4));
        }
    } else {
        const int shared = mx_shared_exp(amax);
        scale_out = (uint8_t)(shared + 127);
        const float f = exp2i(-shared);
        w0 = e4m3x2_sat(hv[0] * f, hv[1] * f) | (e4m3x2_sat(hv[2] * f, hv[3] * f) << 16);
        w1 = e4m3x2_sat(hv[4] * f, hv[5] * f) | (e4m3x2_sat(hv[6] * f, hv[7] * f) << 16);
    }
    return make_uint2(w0, w1);
}

// ---------------------------------------------------------------------------
// gate_up, FP4 experts.  Item = (slot, 32 output columns); waves 0/1 stream
// gate rows cb*32 + [0,16) / [16,32), waves 2/3 the matching up rows.

template <int FMT>
__global__ __launch_bounds__(256) void k_gate_up_fp4(JobDev J, const uint8_t* __restrict__ a_q,
                                                     const uint8_t* __restrict__ a_s,
                                                     uint8_t* __restrict__ h_q,
                                                     uint8_t* __restrict__ h_s) {
    const int I = J.N_out, H = J.K;
    const int CB = I / 32;
    const int slot = blockIdx.x / CB, cb = blockIdx.x % CB;
    Tokens tk;
    if (!resolve(J, slot, tk)) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int m = lane & 15, g = lane >> 4;
    const int wr = (wave >> 1) * I + cb * 32 + (wave & 1) * 16 + m;
    const size_t grow = (size_t)tk.e * (2 * I) + wr;
    const uint8_t* wrow = J.w + grow * (H / 2);
    const uint8_t* srow = J.scales + grow * (FMT == kFmtMX ? H / 32 : H / 16);
    const float gs = (FMT == kFmtNV) ? J.gscale[tk.e] : 1.0f;

    __shared__ int s_row[kPass];
    __shared__ int s_smax[kPass];
    __shared__ float s_G[kPass][65];

    for (int t0 = 0; t0 < tk.n; t0 += kPass) {
        const int npass = min(kPass, tk.n - t0);
        const int nb = (npass + 15) / 16;
        if (threadIdx.x < kPass) {
            const int t = threadIdx.x;
            int row = -1;
            if (t < npass) {
                const int b = tk.base + t0 + t;
                row = J.dense ? b : J.bucket[b] / J.k;
            }
            s_row[t] = row;
        }
        __syncthreads();
        if (FMT == kFmtNV) {
            pass_row_smax(a_s, H, s_row, npass, s_smax);
            __syncthreads();
        }
        v4f acc[4];
        wave_gemm_fp4<FMT>(wrow, srow, a_q, a_s, H, s_row, s_smax, nb, acc);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < nb) {
#pragma unroll
                for (int r = 0; r < 4; ++r) s_G[16 * j + m][wave * 16 + 4 * g + r] = acc[j][r];
            }
        }
        __syncthreads();
        // SwiGLU + MXFP8 requant: 4 lanes per row, 8 columns each.
        const int t = threadIdx.x >> 2, q4 = threadIdx.x & 3;
        float hv[8];
        float fac = 1.0f;
        if (FMT == kFmtNV && t < npass) fac = nv_row_factor(s_smax[t], gs);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int col = 8 * q4 + c;
            float gt = 0.f, up = 0.f;
            if (t < npass) {
                gt = s_G[t][col];
                up = s_G[t][32 + col];
                if (FMT == kFmtNV) {
                    gt *= fac;
                    up *= fac;
                }
            }
            hv[c] = gt / (1.0f + __expf(-gt)) * up;
        }
        uint8_t sc;
        const uint2 codes = mx_quant8_group4(hv, sc);
        if (t < npass) {
            const size_t orow = (size_t)tk.base + t0 + t;
            *reinterpret_cast<uint2*>(h_q + orow * I + cb * 32 + 8 * q4) = codes;
            if (q4 == 0) h_s[orow * (I / 32) + cb] = sc;
        }
        __syncthreads();
    }
}

hipError_t launch_gate_up_fp4(const ExpertJob& job, const uint8_t* a_q, const uint8_t* a_s,
                              uint8_t* h_q, uint8_t* h_s, hipStream_t stream) {
    const JobDev J = to_dev(job);
    const int blocks = job.slots * (job.N_out / 32);
    if (job.w.fmt == MOE_FMT_MXFP4)
        hipLaunchKernelGGL(k_gate_up_fp4<kFmtMX>, dim3(blocks), dim3(256), 0, stream, J, a_q, a_s, h_q, h_s);
    else
        hipLaunchKernelGGL(k_gate_up_fp4<kFmtNV>, dim3(blocks), dim3(256), 0, stream, J, a_q, a_s, h_q, h_s);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// down, FP4 experts.  Item = (slot, RB output features); wave w owns RB/4
// consecutive features as RB/64 blocks of 16.

static int down_rows_per_item(int H, int I) {
    int rb = std::min(256, std::max(64, 131072 / I));
    while (rb > 64 && H % rb != 0) rb >>= 1;
    return rb;
}

template <int FMT>
__global__ __launch_bounds__(256) void k_down_fp4(JobDev J, int RB, const uint8_t* __restrict__ h_q,
                                                  const uint8_t* __restrict__ h_s,
                                                  float* __restrict__ y) {
    const int H = J.N_out, I = J.K;
    const int NRB = H / RB;
    const int slot = blockIdx.x / NRB, rb = blockIdx.x % NRB;
    Tokens tk;
    if (!resolve(J, slot, tk)) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int m = lane & 15, g = lane >> 4;
    const int per_wave = RB / 4;
    const float gs = (FMT == kFmtNV) ? J.gscale[tk.e] : 1.0f;

    __shared__ int s_row[kPass];
    __shared__ int s_out[kPass];
    __shared__ int s_smax[kPass];

    for (int t0 = 0; t0 < tk.n; t0 += kPass) {
        const int npass = min(kPass, tk.n - t0);
        const int nb = (npass + 15) / 16;
        if (threadIdx.x < kPass) {
            const int t = threadIdx.x;
            int row = -1, orow = -1;
            if (t < npass) {
                row = tk.base + t0 + t;
                orow = J.dense ? row : J.bucket[row];
            }
            s_row[t] = row;
            s_out[t] = orow;
        }
        __syncthreads();
        if (FMT == kFmtNV) {
            pass_row_smax(h_s, I, s_row, npass, s_smax);
            __syncthreads();
        }
        for (int mb = 0; mb < per_wave / 16; ++mb) {
            const int f0 = rb * RB + wave * per_wave + mb * 16;  // first feature of this block
            const size_t grow = (size_t)tk.e * H + f0 + m;
            const uint8_t* wrow = J.w + grow * (I / 2);
            const uint8_t* srow = J.scales + grow * (FMT == kFmtMX ? I / 32 : I / 16);
            v4f acc[4];
            wave_gemm_fp4<FMT>(wrow, srow, h_q, h_s, I, s_row, s_smax, nb, acc);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 16 * j + m;
                if (j < nb && t < npass) {
                    v4f v = acc[j];
                    if (FMT == kFmtNV) {
                        const float fac = nv_row_factor(s_smax[t], gs);
                        v = v * fac;
                    }
                    *reinterpret_cast<v4f*>(y + (size_t)s_out[t] * H + f0 + 4 * g) = v;
                }
            }
        }
        __syncthreads();
    }
}

hipError_t launch_down_fp4(const ExpertJob& job, const uint8_t* h_q, const uint8_t* h_s,
                           float* y, hipStream_t stream) {
    const JobDev J = to_dev(job);
    const int RB = down_rows_per_item(job.N_out, job.K);
    const int blocks = job.slots * (job.N_out / RB);
    if (job.w.fmt == MOE_FMT_MXFP4)
        hipLaunchKernelGGL(k_down_fp4<kFmtMX>, dim3(blocks), dim3(256), 0, stream, J, RB, h_q, h_s, y);
    else
        hipLaunchKernelGGL(k_down_fp4<kFmtNV>, dim3(blocks), dim3(256), 0, stream, J, RB, h_q, h_s, y);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bf16 shared expert (dense over all M rows).  gate_up splits K across S
// workgroups per 32-column block; partial sums go to the workspace and the
// last workgroup of a column block (device-scope counter) adds them in split
// order (deterministic), applies SwiGLU and rounds h to bf16.

struct Bf16Plan {
    int splits;
};

static Bf16Plan bf16_plan(int H, int I) {
    const int cbs = I / 32;
    const int nsteps = H / 32;
    int splits = 1;
    for (int d = 1; d <= nsteps; ++d)
        if (nsteps % d == 0 && cbs * d <= 512) splits = d;
    return Bf16Plan{splits};
}

size_t gate_up_bf16_partials_bytes(int M, int H, int I) {
    const Bf16Plan p = bf16_plan(H, I);
    return align_up((size_t)p.splits * M * 2 * I * sizeof(float));
}

__device__ __forceinline__ void wave_gemm_bf16(const uint16_t* __restrict__ wrow,
                                               const uint16_t* __restrict__ act, int K, int k0,
                                               int k1, const int* s_row, int nb, v4f acc[4]) {
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, g = lane >> 4;
    int rowj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        rowj[j] = (j < nb) ? s_row[16 * j + m] : -1;
        acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll 4
    for (int kk = k0; kk < k1; kk += 32) {
        const v4i a = load16_nt(wrow + kk + 8 * g);
        const v8bf A = __builtin_bit_cast(v8bf, a);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < nb) {
                v4i b = {0, 0, 0, 0};
                if (rowj[j] >= 0) b = load16(act + (size_t)rowj[j] * K + kk + 8 * g);
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(v8bf, b), acc[j], 0, 0, 0);
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_gate_up_bf16(JobDev J, int splits,
                                                      const uint16_t* __restrict__ a,
                                                      uint16_t* __restrict__ h,
                                                      float* __restrict__ part,
                                                      int* __restrict__ counters) {
    const int I = J.N_out, H = J.K, M = J.M;
    const int cb = blockIdx.x / splits, ks = blockIdx.x % splits;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int m = lane & 15, g = lane >> 4;
    const int wr = (wave >> 1) * I + cb * 32 + (wave & 1) * 16 + m;
    const uint16_t* wrow = reinterpret_cast<const uint16_t*>(J.w) + (size_t)wr * H;
    const int kc = H / splits;
    __shared__ int s_row[kPass];
    __shared__ int s_last;
    for (int t0 = 0; t0 < M; t0 += kPass) {
        const int npass = min(kPass, M - t0);
        const int nb = (npass + 15) / 16;
        if (threadIdx.x < kPass) s_row[threadIdx.x] = threadIdx.x < npass ? t0 + threadIdx.x : -1;
        __syncthreads();
        v4f acc[4];
        wave_gemm_bf16(wrow, a, H, ks * kc, (ks + 1) * kc, s_row, nb, acc);
        // partial G: [split][row][2I]; this lane: feature wr's block rows 4g+r
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = 16 * j + m;
            if (j < nb && t < npass) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int col = (wave >> 1) * I + cb * 32 + (wave & 1) * 16 + 4 * g + r;
                    part[((size_t)ks * M + t0 + t) * (2 * I) + col] = acc[j][r];
                }
            }
        }
        __syncthreads();
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) s_last = (atomicAdd(&counters[cb], 1) == splits - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    // reduce in split order, SwiGLU, round to bf16: thread -> (row, column)
    for (int idx = threadIdx.x; idx < M * 32; idx += 256) {
        const int t = idx / 32, c = idx % 32;
        const int col = cb * 32 + c;
        float gt = 0.f, up = 0.f;
        for (int s = 0; s < splits; ++s) {
            const float* pr = part + ((size_t)s * M + t) * (2 * I);
            gt += load_agent(pr + col);
            up += load_agent(pr + I + col);
        }
        const float hv = gt / (1.0f + __expf(-gt)) * up;
        h[(size_t)t * I + col] = (uint16_t)f32_to_bf16_rne(hv);
    }
    if (threadIdx.x == 0) counters[cb] = 0;
}

hipError_t launch_gate_up_bf16(const ExpertJob& job, const uint16_t* a, uint16_t* h,
                               float* part, int* counters, hipStream_t stream) {
    const JobDev J = to_dev(job);
    const Bf16Plan p = bf16_plan(job.K, job.N_out);
    const int blocks = (job.N_out / 32) * p.splits;
    hipLaunchKernelGGL(k_gate_up_bf16, dim3(blocks), dim3(256), 0, stream, J, p.splits, a, h, part, counters);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_down_bf16(JobDev J, const uint16_t* __restrict__ hin,
                                                   float* __restrict__ y) {
    const int H = J.N_out, I = J.K, M = J.M;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int m = lane & 15, g = lane >> 4;
    const int f0 = blockIdx.x * 64 + wave * 16;
    const uint16_t* wrow = reinterpret_cast<const uint16_t*>(J.w) + (size_t)(f0 + m) * I;
    __shared__ int s_row[kPass];
    for (int t0 = 0; t0 < M; t0 += kPass) {
        const int npass = min(kPass, M - t0);
        const int nb = (npass + 15) / 16;
        if (threadIdx.x < kPass) s_row[threadIdx.x] = threadIdx.x < npass ? t0 + threadIdx.x : -1;
        __syncthreads();
        v4f acc[4];
        wave_gemm_bf16(wrow, hin, I, 0, I, s_row, nb, acc);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = 16 * j + m;
            if (j < nb && t < npass)
                *reinterpret_cast<v4f*>(y + (size_t)(t0 + t) * H + f0 + 4 * g) = acc[j];
        }
        __syncthreads();
    }
}

hipError_t launch_down_bf16(const ExpertJob& job, const uint16_t* h, float* y, hipStream_t stream) {
    const JobDev J = to_dev(job);
    hipLaunchKernelGGL(k_down_bf16, dim3(job.N_out / 64), dim3(256), 0, stream, J, h, y);
    return hipGetLastError();
}

}  // namespace moe
