// k_stream.hip — block-scaled FP4 expert GEMMs on gfx950 matrix cores:
// gate_up (+ SwiGLU + MXFP8 requant) and down, for MXFP4 and NVFP4 experts.
//
// Pages: SGLang-NVIDIA-Mega README, DeepSeek-V4.1 slot table, row "Routed
// experts (moe)" (a pair of block-scaled GEMMs over 8-row tiles; an expert
// with more than 8 rows takes several tiles); README Qwen3.5 slot table, row
// "mkm" (FC1, SwiGLU, requant, FC2); sgl-nvidia-mega PR #24, "Modifications /
// Target spec" (NVFP4 routed experts); SGLang Spark GB10 Optimizations,
// section 1 (NVFP4 K-groups of 16 with FP8 scale rows) and section 4 (a
// sparse FP4 GEMV for MoE decode).
//
// Work decomposition (weight streaming, HBM-bound).  An item is (active
// expert, block of weight rows, K range).  Its workgroup
//   1. issues the first D 128-K steps of its weight loads as soon as the
//      expert is known,
//   2. copies the expert's activation rows (up to R rows per pass) for its K
//      range into LDS,
//   3. streams its weight rows through a per-wave register ring D steps deep,
//      with no barrier inside the K loop (the B operands come from LDS),
//   4. writes the result: gate_up over the whole K fuses SwiGLU and the
//      MXFP8 requant; gate_up split over K writes fp32 partials that a second
//      launch adds in split order; down writes fp32 per (row, slot).
// Every expert weight byte is read once per call however many 8-row tiles the
// expert has (up to R rows per pass).  Ring refills past the item's K range
// read through a buffer resource at an offset past its record count, which
// returns zeros without touching memory, so the ring has no branches (a
// branch between an MFMA and the read of its accumulator is also what the
// compiler does not always pad correctly on this target).
//
// Operand layouts (checked on the hardware):
//   v_mfma_scale_f32_16x16x128_f8f6f4, FP4 operand: lane (row i, group g)
//     holds K [32g, 32g+32) as 16 packed bytes; FP8 operand: lane (col n, g)
//     holds K [16g, 16g+16) in bytes 0-15 and K [64+16g, 64+16g+16) in bytes
//     16-31; the E8M0 scale of (row/col i, K block b) comes from lane 16b+i.
//   v_mfma_f32_16x16x32_f16: lane (i, g) holds K [8g, 8g+8).
//   Output D (16x16): lane l holds D[4(l/16)+r][l%16], r = 0..3.
// Weights are the M side (16 rows per block), activation rows the N side.
#include "moe_device.h"
#include "moe_internal.h"

#include <algorithm>

namespace moe {

namespace {

constexpr int kFmtMX = MOE_FMT_MXFP4;
constexpr int kFmtNV = MOE_FMT_NVFP4;
constexpr int kThreads = 256;
constexpr uint32_t kOOB = 0x80000000u;  // buffer offset past every record count

#ifndef MOE_STREAM_LDS_BUDGET
#define MOE_STREAM_LDS_BUDGET 65024  // bytes of activation stage per workgroup
#endif
#ifndef MOE_STREAM_TARGET_ITEMS
#define MOE_STREAM_TARGET_ITEMS 1024  // gate_up splits K until about this many items
#endif

struct StreamJob {
    const uint8_t* w;       // packed E2M1, [E][N][K/2]
    const uint8_t* sc;      // MX: E8M0 [E][N][K/32]; NV: E4M3 [E][N][K/16]
    const float* gscale;    // NV: per-expert fp32 global
    int N, K;               // weight rows per expert, reduction length
    int dense;              // one expert over all M rows
    const int32_t* offsets;
    const int32_t* bucket;
    const int32_t* active;
    const int32_t* num_active;
    int k, M;
    int R;                  // activation rows per pass (16 or 32)
    int span;               // K per split (multiple of 128 * D)
    int splits;
    int nblk;               // row blocks per expert
    int out_rows;           // rows of the partial buffer (gate_up split)
};

struct Tokens {
    int e, base, n;
};

__device__ __forceinline__ bool resolve(const StreamJob& J, int slot, Tokens& t) {
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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// ---- NVFP4 helpers ----------------------------------------------------------

// E4M3 scale code -> (fp32 value whose exponent is used, f16 mantissa factor):
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

// Per-row factor that turns an NVFP4 accumulator into the product value:
// 2^(smax - 127) (activation offset) * global.
__device__ __forceinline__ float nv_row_factor(int smax, float gs) { return ldexpf(gs, smax - 127); }

// ---- activation stage -------------------------------------------------------
// LDS: q[R][span + 16] (E4M3 codes, padded rows), s[R][span / 32] (E8M0).

struct Stage {
    uint8_t* q;
    uint8_t* s;
    int rs;   // q row stride
    int ss;   // s row stride
};

__device__ __forceinline__ Stage stage_layout(uint8_t* lds, int R, int span) {
    Stage S;
    S.rs = span + 16;
    S.ss = span / 32;
    S.q = lds;
    S.s = lds + (size_t)R * S.rs;
    return S;
}

// Copies rows s_arow[0..npass) x K [k0, k0 + len) into the stage and zeroes
// rows [npass, rows_z) (the padding columns of the last MFMA N-block).
__device__ void stage_rows(const Stage& S, const uint8_t* __restrict__ a_q,
                           const uint8_t* __restrict__ a_s, int K, int k0, int len,
                           const int* s_arow, int npass, int rows_z) {
    const int tid = threadIdx.x;
    const int cpr = len / 16;  // 16-byte chunks per row
    for (int idx = tid; idx < rows_z * cpr; idx += kThreads) {
        const int t = idx / cpr, c = idx - t * cpr;
        v4i v = v4i{0, 0, 0, 0};
        if (t < npass) v = load16(a_q + (size_t)s_arow[t] * K + k0 + 16 * c);
        *reinterpret_cast<v4i*>(S.q + t * S.rs + 16 * c) = v;
    }
    const int dpr = len / 128;  // scale dwords per row
    for (int idx = tid; idx < rows_z * dpr; idx += kThreads) {
        const int t = idx / dpr, c = idx - t * dpr;
        uint32_t v = 0;
        if (t < npass)
            v = *reinterpret_cast<const uint32_t*>(a_s + (size_t)s_arow[t] * (K / 32) + k0 / 32 + 4 * c);
        *reinterpret_cast<uint32_t*>(S.s + t * S.ss + 4 * c) = v;
    }
}

// NVFP4: largest E8M0 code of each staged row over the staged K range
// (activations enter the f16 MFMA as E4M3 * 2^(s - smax), inside f16 range);
// zero for padding rows.
__device__ void stage_row_smax(const Stage& S, int len, int npass, int rows_z, int* s_smax) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int dpr = len / 128;
    for (int t = wave; t < rows_z; t += kThreads / 64) {
        uint32_t mx = 0;
        if (t < npass) {
            for (int d = lane; d < dpr; d += 64) {
                const uint32_t v = *reinterpret_cast<const uint32_t*>(S.s + t * S.ss + 4 * d);
                mx = max(mx, max(max(v & 0xffu, (v >> 8) & 0xffu), max((v >> 16) & 0xffu, v >> 24)));
            }
            for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
        }
        if (lane == 0) s_smax[t] = (int)mx;
    }
}

// ---- weight ring ------------------------------------------------------------

template <int MB, int D>
struct Ring {
    v4i a[D][MB];
    uint32_t s[D][MB];
};

// Per-lane weight coordinates of MB blocks of 16 rows.
template <int MB>
struct WCoord {
    __amdgpu_buffer_rsrc_t rw, rs;
    uint32_t vw[MB];  // byte offset of (row, 16g) in the expert's packed matrix
    uint32_t vs[MB];  // byte offset of the lane's scale word in the scale matrix
};

template <int FMT, int MB>
__device__ __forceinline__ WCoord<MB> wcoord(const StreamJob& J, int e, const int (&row)[MB]) {
    const int g = (threadIdx.x & 63) >> 4;
    const uint32_t wbytes = (uint32_t)J.N * (J.K / 2);
    const uint32_t sbytes = (uint32_t)J.N * (J.K / (FMT == kFmtMX ? 32 : 16));
    WCoord<MB> c;
    c.rw = make_rsrc(J.w + (size_t)e * wbytes, wbytes);
    c.rs = make_rsrc(J.sc + (size_t)e * sbytes, sbytes);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        c.vw[mb] = (uint32_t)row[mb] * (J.K / 2) + 16 * g;
        c.vs[mb] = FMT == kFmtMX ? (uint32_t)row[mb] * (J.K / 32) : (uint32_t)row[mb] * (J.K / 16) + 2 * g;
    }
    return c;
}

// Loads absolute K step `st` into ring slot u; ok == false loads zeros.
template <int FMT, int MB, int D>
__device__ __forceinline__ void ring_load(Ring<MB, D>& R, int u, const WCoord<MB>& c, int st, bool ok) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        R.a[u][mb] = __builtin_amdgcn_raw_buffer_load_b128(c.rw, ok ? c.vw[mb] : kOOB, 64 * st, 2);
        if constexpr (FMT == kFmtMX)
            R.s[u][mb] = __builtin_amdgcn_raw_buffer_load_b32(c.rs, ok ? c.vs[mb] : kOOB, 4 * st, 0);
        else
            R.s[u][mb] = __builtin_amdgcn_raw_buffer_load_b16(c.rs, ok ? c.vs[mb] : kOOB, 8 * st, 0);
    }
}

template <int FMT, int MB, int D>
__device__ __forceinline__ void ring_prologue(Ring<MB, D>& R, const WCoord<MB>& c, int s0, int nst) {
#pragma unroll
    for (int u = 0; u < D; ++u) ring_load<FMT, MB, D>(R, u, c, s0 + u, u < nst);
}

// One 128-K step: MB weight blocks x NB activation blocks (staged step ls).
template <int FMT, int MB, int NB>
__device__ __forceinline__ void step_mfma(const v4i (&a)[MB], const uint32_t (&ws)[MB], const Stage& S,
                                          int ls, const int (&sfo)[NB], v4f (&acc)[MB][2]) {
    const int lane = threadIdx.x & 63;
    const int i = lane & 15, g = lane >> 4;
    if constexpr (FMT == kFmtMX) {
        v8i B[NB];
        int sb[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int t = 16 * j + i;
            const uint8_t* rp = S.q + t * S.rs + 128 * ls;
            const v4i b0 = *reinterpret_cast<const v4i*>(rp + 16 * g);
            const v4i b1 = *reinterpret_cast<const v4i*>(rp + 64 + 16 * g);
            B[j] = v8i{b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
            sb[j] = S.s[t * S.ss + 4 * ls + g];
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const v8i A = {a[mb].x, a[mb].y, a[mb].z, a[mb].w, 0, 0, 0, 0};
            const int sa = (int)(ws[mb] >> (8 * g));
#pragma unroll
            for (int j = 0; j < NB; ++j)
                acc[mb][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B[j], acc[mb][j], 4, 0, 0, sa,
                                                                              0, sb[j]);
        }
    } else {
        v8h B[NB][4];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int t = 16 * j + i;
            const uint8_t* rp = S.q + t * S.rs + 128 * ls + 32 * g;
            const v4i b0 = *reinterpret_cast<const v4i*>(rp);
            const v4i b1 = *reinterpret_cast<const v4i*>(rp + 16);
            const int sb = S.s[t * S.ss + 4 * ls + g];
            const float sf = exp2i(max(sb + sfo[j], -126));
            B[j][0] = fp8x8_to_f16((uint32_t)b0.x, (uint32_t)b0.y, sf);
            B[j][1] = fp8x8_to_f16((uint32_t)b0.z, (uint32_t)b0.w, sf);
            B[j][2] = fp8x8_to_f16((uint32_t)b1.x, (uint32_t)b1.y, sf);
            B[j][3] = fp8x8_to_f16((uint32_t)b1.z, (uint32_t)b1.w, sf);
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            float sv0, sv1;
            _Float16 m0, m1;
            nv_scale_split(ws[mb] & 0xffu, sv0, m0);
            nv_scale_split((ws[mb] >> 8) & 0xffu, sv1, m1);
            const v8h A0 = nv_dequant8((uint32_t)a[mb].x, sv0, m0);
            const v8h A1 = nv_dequant8((uint32_t)a[mb].y, sv0, m0);
            const v8h A2 = nv_dequant8((uint32_t)a[mb].z, sv1, m1);
            const v8h A3 = nv_dequant8((uint32_t)a[mb].w, sv1, m1);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, B[j][0], acc[mb][j], 0, 0, 0);
                acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, B[j][1], acc[mb][j], 0, 0, 0);
                acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A2, B[j][2], acc[mb][j], 0, 0, 0);
                acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A3, B[j][3], acc[mb][j], 0, 0, 0);
            }
        }
    }
}

// The K loop of one pass: nst staged steps (a multiple of D) starting at
// absolute step s0; the ring holds the first D steps on entry.  Every slot is
// refilled D steps ahead (zeros past the range).  NB is a compile-time
// constant, so no branch separates an MFMA from the read of its accumulator.
template <int FMT, int MB, int D, int NB>
__device__ __forceinline__ void stream_k(Ring<MB, D>& R, const WCoord<MB>& c, const Stage& S, int s0, int nst,
                                         const int* s_smax, v4f (&acc)[MB][2]) {
    const int i = threadIdx.x & 15;
    int sfo[NB];  // NVFP4: -smax of the lane's activation row
#pragma unroll
    for (int j = 0; j < NB; ++j) sfo[j] = FMT == kFmtNV ? -s_smax[16 * j + i] : 0;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[mb][j] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int l0 = 0; l0 < nst; l0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            step_mfma<FMT, MB, NB>(R.a[u], R.s[u], S, l0 + u, sfo, acc);
            const int ln = l0 + u + D;
            ring_load<FMT, MB, D>(R, u, c, s0 + ln, ln < nst);
        }
    }
}

template <int FMT, int MB, int D>
__device__ __forceinline__ void stream_pass(Ring<MB, D>& R, const WCoord<MB>& c, const Stage& S, int s0, int nst,
                                            int npass, const int* s_smax, v4f (&acc)[MB][2]) {
    if (npass > 16)
        stream_k<FMT, MB, D, 2>(R, c, S, s0, nst, s_smax, acc);
    else
        stream_k<FMT, MB, D, 1>(R, c, S, s0, nst, s_smax, acc);
}

// MXFP8 of 4 consecutive values (part of a 32-value block shared by 8
// consecutive lanes): returns the 4 codes, writes the block's scale code.
__device__ __forceinline__ uint32_t mx_quant4_group8(const float hv[4], uint8_t& scale_out) {
    uint32_t amax = 0;
    int special = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t b = __float_as_uint(hv[c]) & 0x7fffffffu;
        amax = max(amax, b);
        special |= f32_bits_special(b) ? 1 : 0;
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, off, 64));
        special |= __shfl_xor(special, off, 64);
    }
    uint32_t w = 0;
    if (special) {
        scale_out = 0xff;
#pragma unroll
        for (int c = 0; c < 4; ++c) w |= (((__float_as_uint(hv[c]) >> 24) & 0x80u) | 0x7fu) << (8 * c);
    } else {
        const int shared = mx_shared_exp(amax);
        scale_out = (uint8_t)(shared + 127);
        const float f = exp2i(-shared);
        w = e4m3x2_sat(hv[0] * f, hv[1] * f) | (e4m3x2_sat(hv[2] * f, hv[3] * f) << 16);
    }
    return w;
}

__device__ __forceinline__ float silu_mul(float gt, float up) { return gt / (1.0f + __expf(-gt)) * up; }

extern __shared__ __align__(16) uint8_t g_lds[];

// ---- gate_up ----------------------------------------------------------------
// Item = (slot, 32 output columns, K split).  Waves 0/1 stream gate rows
// cb*32 + [0,16) / [16,32), waves 2/3 the matching up rows (rows I + ...).
// FUSED (one split): SwiGLU + MXFP8 requant in the epilogue, h rows are
// bucket positions (routed) or token rows (dense).  Otherwise fp32 partials
// part[split][row][2I] (already multiplied by the NVFP4 row factor).

template <int FMT, int D, bool FUSED>
__global__ __launch_bounds__(kThreads, 2) void k_gate_up(StreamJob J, const uint8_t* __restrict__ a_q,
                                                         const uint8_t* __restrict__ a_s,
                                                         uint8_t* __restrict__ h_q, uint8_t* __restrict__ h_s,
                                                         float* __restrict__ part) {
    const int I = J.N / 2, K = J.K;
    const int ks = blockIdx.x % J.splits;
    const int blk = (blockIdx.x / J.splits) % J.nblk;
    const int slot = blockIdx.x / (J.splits * J.nblk);
    Tokens tk;
    if (!resolve(J, slot, tk)) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int i = lane & 15, g = lane >> 4;
    const int col0 = blk * 32 + (wave & 1) * 16;         // first of the wave's 16 output columns
    const int wrow[1] = {(wave >> 1) * I + col0 + i};     // gate or up row of the lane
    const WCoord<1> wc = wcoord<FMT, 1>(J, tk.e, wrow);
    const int k0 = ks * J.span;
    const int len = min(J.span, K - k0);
    const int s0 = k0 / 128, nst = len / 128;

    Ring<1, D> R;
    ring_prologue<FMT, 1, D>(R, wc, s0, nst);

    const Stage S = stage_layout(g_lds, J.R, J.span);
    __shared__ int s_arow[32];
    __shared__ int s_orow[32];
    __shared__ int s_smax[32];
    const float gs = FMT == kFmtNV ? J.gscale[tk.e] : 1.0f;

    for (int t0 = 0; t0 < tk.n; t0 += J.R) {
        const int npass = min(J.R, tk.n - t0);
        const int rows_z = npass > 16 ? 32 : 16;
        if (t0 > 0) ring_prologue<FMT, 1, D>(R, wc, s0, nst);
        if (threadIdx.x < 32) {
            const int t = threadIdx.x;
            int ar = -1, orow = -1;
            if (t < npass) {
                const int b = tk.base + t0 + t;
                ar = J.dense ? b : J.bucket[b] / J.k;
                orow = b;
            }
            s_arow[t] = ar;
            s_orow[t] = orow;
        }
        __syncthreads();
        stage_rows(S, a_q, a_s, K, k0, len, s_arow, npass, rows_z);
        __syncthreads();
        if (FMT == kFmtNV) {
            stage_row_smax(S, len, npass, rows_z, s_smax);
            __syncthreads();
        }
        v4f acc[1][2];
        stream_pass<FMT, 1, D>(R, wc, S, s0, nst, npass, s_smax, acc);
        if constexpr (FUSED) {
            __syncthreads();  // the stage is reused for the gate/up tile
            float* sG = reinterpret_cast<float*>(g_lds);  // [32][65]
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int t = 16 * j + i;
                if (t < npass) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) sG[t * 65 + wave * 16 + 4 * g + r] = acc[0][j][r];
                }
            }
            __syncthreads();
            // SwiGLU + MXFP8 requant: 8 lanes per row, 4 columns each.
            const int t = threadIdx.x >> 3, q8 = threadIdx.x & 7;
            float hv[4];
            float fac = 1.0f;
            if (FMT == kFmtNV && t < npass) fac = nv_row_factor(s_smax[t], gs);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int col = 4 * q8 + c;
                float gt = 0.f, up = 0.f;
                if (t < npass) {
                    gt = sG[t * 65 + col] * fac;
                    up = sG[t * 65 + 32 + col] * fac;
                }
                hv[c] = silu_mul(gt, up);
            }
            uint8_t sc;
            const uint32_t codes = mx_quant4_group8(hv, sc);
            if (t < npass) {
                const size_t orow = (size_t)s_orow[t];
                *reinterpret_cast<uint32_t*>(h_q + orow * I + blk * 32 + 4 * q8) = codes;
                if (q8 == 0) h_s[orow * (I / 32) + blk] = sc;
            }
        } else {
            const int colw = (wave >> 1) * I + col0 + 4 * g;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int t = 16 * j + i;
                if (t < npass) {
                    v4f v = acc[0][j];
                    if (FMT == kFmtNV) v = v * nv_row_factor(s_smax[t], gs);
                    *reinterpret_cast<v4f*>(part + ((size_t)ks * J.out_rows + s_orow[t]) * (2 * I) + colw) = v;
                }
            }
        }
        __syncthreads();
    }
}

// Sum of the split partials in split order, SwiGLU, MXFP8 requant of h.
// Thread = (row, 4 columns); 8 consecutive threads share a 32-column block.
__global__ __launch_bounds__(kThreads) void k_swiglu_quant(const float* __restrict__ part, int splits, int rows,
                                                           int I, uint8_t* __restrict__ h_q,
                                                           uint8_t* __restrict__ h_s) {
    const int idx = blockIdx.x * kThreads + threadIdx.x;
    const int q8 = idx & 7, blk = idx >> 3;
    const int cbs = I / 32;
    const int row = blk / cbs, cb = blk - row * cbs;
    if (row >= rows) return;  // whole 8-lane groups leave together
    const int col = cb * 32 + 4 * q8;
    v4f gt = v4f{0.f, 0.f, 0.f, 0.f}, up = v4f{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < splits; ++s) {
        const float* pr = part + ((size_t)s * rows + row) * (2 * I);
        gt += *reinterpret_cast<const v4f*>(pr + col);
        up += *reinterpret_cast<const v4f*>(pr + I + col);
    }
    float hv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) hv[c] = silu_mul(gt[c], up[c]);
    uint8_t sc;
    const uint32_t codes = mx_quant4_group8(hv, sc);
    *reinterpret_cast<uint32_t*>(h_q + (size_t)row * I + col) = codes;
    if (q8 == 0) h_s[(size_t)row * cbs + cb] = sc;
}

// ---- down -------------------------------------------------------------------
// Item = (slot, 64*MB output features); wave w owns MB blocks of 16 features.
// Activations are h rows (bucket positions for routed experts); the output
// row of bucket position b is its pair id bucket[b].

template <int FMT, int D, int MB>
__global__ __launch_bounds__(kThreads, 2) void k_down(StreamJob J, const uint8_t* __restrict__ h_q,
                                                      const uint8_t* __restrict__ h_s, float* __restrict__ y) {
    const int H = J.N, I = J.K;
    constexpr int RB = 64 * MB;
    const int blk = blockIdx.x % J.nblk;
    const int slot = blockIdx.x / J.nblk;
    Tokens tk;
    if (!resolve(J, slot, tk)) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int i = lane & 15, g = lane >> 4;
    const int f0 = blk * RB + wave * (16 * MB);
    int wrow[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) wrow[mb] = f0 + 16 * mb + i;
    const WCoord<MB> wc = wcoord<FMT, MB>(J, tk.e, wrow);
    const int nst = I / 128;

    Ring<MB, D> R;
    ring_prologue<FMT, MB, D>(R, wc, 0, nst);

    const Stage S = stage_layout(g_lds, J.R, I);
    __shared__ int s_arow[32];
    __shared__ int s_orow[32];
    __shared__ int s_smax[32];
    const float gs = FMT == kFmtNV ? J.gscale[tk.e] : 1.0f;

    for (int t0 = 0; t0 < tk.n; t0 += J.R) {
        const int npass = min(J.R, tk.n - t0);
        const int rows_z = npass > 16 ? 32 : 16;
        if (t0 > 0) ring_prologue<FMT, MB, D>(R, wc, 0, nst);
        if (threadIdx.x < 32) {
            const int t = threadIdx.x;
            int ar = -1, orow = -1;
            if (t < npass) {
                const int b = tk.base + t0 + t;
                ar = b;
                orow = J.dense ? b : J.bucket[b];
            }
            s_arow[t] = ar;
            s_orow[t] = orow;
        }
        __syncthreads();
        stage_rows(S, h_q, h_s, I, 0, I, s_arow, npass, rows_z);
        __syncthreads();
        if (FMT == kFmtNV) {
            stage_row_smax(S, I, npass, rows_z, s_smax);
            __syncthreads();
        }
        v4f acc[MB][2];
        stream_pass<FMT, MB, D>(R, wc, S, 0, nst, npass, s_smax, acc);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int t = 16 * j + i;
                if (t < npass) {
                    v4f v = acc[mb][j];
                    if (FMT == kFmtNV) v = v * nv_row_factor(s_smax[t], gs);
                    *reinterpret_cast<v4f*>(y + (size_t)s_orow[t] * H + f0 + 16 * mb + 4 * g) = v;
                }
            }
        }
        __syncthreads();
    }
}

// ---- host plans -------------------------------------------------------------

int pow2_divisor(int n, int cap) {
    int d = 1;
    while (d * 2 <= cap && n % (d * 2) == 0) d *= 2;
    return d;
}

// Stage rows: the MFMA N-block is 16 rows, and no expert has more than M rows
// (a row picks an expert once).
int rows_for(int M) { return M <= 16 ? 16 : 32; }

size_t stage_bytes(int R, int span) { return (size_t)R * (span + 16) + (size_t)R * (span / 32); }

// Longest K range (a multiple of unit) whose stage of R rows fits the budget.
int max_span(int R, int unit) {
    int span = unit;
    while (stage_bytes(R, span + unit) <= (size_t)MOE_STREAM_LDS_BUDGET) span += unit;
    return span;
}

struct GatePlan {
    int R, D, span, splits, nblk;
    size_t lds;
};

GatePlan gate_plan(const ExpertJob& j) {
    GatePlan p;
    const int K = j.K, steps = K / 128;
    p.D = pow2_divisor(steps, 8);
    p.R = rows_for(j.M);
    p.nblk = j.N_out / 32;
    const int unit = 128 * p.D;
    const long items = (long)j.slots * p.nblk;
    const int want = (int)std::max<long>(1, (MOE_STREAM_TARGET_ITEMS + items - 1) / items);
    int span = (K + want - 1) / want;
    span = (span + unit - 1) / unit * unit;
    p.span = std::min(std::min(span, max_span(p.R, unit)), K);
    p.splits = (K + p.span - 1) / p.span;
    p.lds = std::max(stage_bytes(p.R, p.span), (size_t)32 * 65 * sizeof(float));
    return p;
}

struct DownPlan {
    int R, D, MB, nblk;
    size_t lds;
};

DownPlan down_plan(const ExpertJob& j) {
    DownPlan p;
    const int I = j.K, steps = I / 128;
    p.D = pow2_divisor(steps, 8);
    // weight loads in flight per lane: MB * D <= 8 (16 bytes each)
    p.MB = p.D == 8 ? 1 : (p.D == 4 || j.N_out % 256 != 0 ? 2 : 4);
    p.R = rows_for(j.M);
    if (p.R == 32 && stage_bytes(32, I) > (size_t)MOE_STREAM_LDS_BUDGET) p.R = 16;
    p.nblk = j.N_out / (64 * p.MB);
    p.lds = stage_bytes(p.R, I);
    return p;
}

StreamJob stream_job(const ExpertJob& j, int N, int R, int span, int splits, int nblk, int out_rows) {
    StreamJob s;
    s.w = static_cast<const uint8_t*>(j.w.w);
    s.sc = j.w.scales;
    s.gscale = j.w.global_scale;
    s.N = N;
    s.K = j.K;
    s.dense = j.dense ? 1 : 0;
    s.offsets = j.offsets;
    s.bucket = j.bucket;
    s.active = j.active;
    s.num_active = j.num_active;
    s.k = j.k;
    s.M = j.M;
    s.R = R;
    s.span = span;
    s.splits = splits;
    s.nblk = nblk;
    s.out_rows = out_rows;
    return s;
}

template <int FMT, int D>
hipError_t launch_gate_up_d(const StreamJob& J, const GatePlan& p, int blocks, const uint8_t* a_q,
                            const uint8_t* a_s, uint8_t* h_q, uint8_t* h_s, float* part, hipStream_t stream) {
    if (p.splits == 1)
        hipLaunchKernelGGL((k_gate_up<FMT, D, true>), dim3(blocks), dim3(kThreads), p.lds, stream, J, a_q, a_s, h_q,
                           h_s, part);
    else
        hipLaunchKernelGGL((k_gate_up<FMT, D, false>), dim3(blocks), dim3(kThreads), p.lds, stream, J, a_q, a_s,
                           h_q, h_s, part);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_gate_up_f(const StreamJob& J, const GatePlan& p, int blocks, const uint8_t* a_q,
                            const uint8_t* a_s, uint8_t* h_q, uint8_t* h_s, float* part, hipStream_t stream) {
    switch (p.D) {
        case 8: return launch_gate_up_d<FMT, 8>(J, p, blocks, a_q, a_s, h_q, h_s, part, stream);
        case 4: return launch_gate_up_d<FMT, 4>(J, p, blocks, a_q, a_s, h_q, h_s, part, stream);
        case 2: return launch_gate_up_d<FMT, 2>(J, p, blocks, a_q, a_s, h_q, h_s, part, stream);
        default: return launch_gate_up_d<FMT, 1>(J, p, blocks, a_q, a_s, h_q, h_s, part, stream);
    }
}

template <int FMT, int D, int MB>
hipError_t launch_down_k(const StreamJob& J, const DownPlan& p, int blocks, const uint8_t* h_q,
                         const uint8_t* h_s, float* y, hipStream_t stream) {
    hipLaunchKernelGGL((k_down<FMT, D, MB>), dim3(blocks), dim3(kThreads), p.lds, stream, J, h_q, h_s, y);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_down_f(const StreamJob& J, const DownPlan& p, int blocks, const uint8_t* h_q,
                         const uint8_t* h_s, float* y, hipStream_t stream) {
    if (p.D == 8) return launch_down_k<FMT, 8, 1>(J, p, blocks, h_q, h_s, y, stream);
    if (p.D == 4) return launch_down_k<FMT, 4, 2>(J, p, blocks, h_q, h_s, y, stream);
    if (p.D == 2)
        return p.MB == 4 ? launch_down_k<FMT, 2, 4>(J, p, blocks, h_q, h_s, y, stream)
                         : launch_down_k<FMT, 2, 2>(J, p, blocks, h_q, h_s, y, stream);
    return p.MB == 4 ? launch_down_k<FMT, 1, 4>(J, p, blocks, h_q, h_s, y, stream)
                     : launch_down_k<FMT, 1, 2>(J, p, blocks, h_q, h_s, y, stream);
}

int out_rows_of(const ExpertJob& j) { return j.dense ? j.M : j.M * j.k; }

}  // namespace

size_t gate_up_fp4_partials_bytes(const ExpertJob& job) {
    const GatePlan p = gate_plan(job);
    if (p.splits == 1) return 0;
    return align_up((size_t)p.splits * out_rows_of(job) * 2 * job.N_out * sizeof(float));
}

hipError_t launch_gate_up_fp4(const ExpertJob& job, const uint8_t* a_q, const uint8_t* a_s, uint8_t* h_q,
                              uint8_t* h_s, float* partials, hipStream_t stream) {
    const GatePlan p = gate_plan(job);
    const int rows = out_rows_of(job);
    const StreamJob J = stream_job(job, 2 * job.N_out, p.R, p.span, p.splits, p.nblk, rows);
    const int blocks = job.slots * p.nblk * p.splits;
    hipError_t e = job.w.fmt == MOE_FMT_MXFP4
                       ? launch_gate_up_f<kFmtMX>(J, p, blocks, a_q, a_s, h_q, h_s, partials, stream)
                       : launch_gate_up_f<kFmtNV>(J, p, blocks, a_q, a_s, h_q, h_s, partials, stream);
    if (e != hipSuccess || p.splits == 1) return e;
    const int threads = rows * (job.N_out / 32) * 8;
    hipLaunchKernelGGL(k_swiglu_quant, dim3((threads + kThreads - 1) / kThreads), dim3(kThreads), 0, stream,
                       partials, p.splits, rows, job.N_out, h_q, h_s);
    return hipGetLastError();
}

hipError_t launch_down_fp4(const ExpertJob& job, const uint8_t* h_q, const uint8_t* h_s, float* y,
                           hipStream_t stream) {
    const DownPlan p = down_plan(job);
    const StreamJob J = stream_job(job, job.N_out, p.R, job.K, 1, p.nblk, out_rows_of(job));
    const int blocks = job.slots * p.nblk;
    return job.w.fmt == MOE_FMT_MXFP4 ? launch_down_f<kFmtMX>(J, p, blocks, h_q, h_s, y, stream)
                                      : launch_down_f<kFmtNV>(J, p, blocks, h_q, h_s, y, stream);
}

}  // namespace moe
