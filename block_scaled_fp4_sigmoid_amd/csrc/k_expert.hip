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

// ---------------------------------------------------------------------------
// Streaming structure shared by gate_up and down (FP4 experts).
//   * A pass covers up to kTP = 32 of the expert's rows (two 16-row N-blocks,
//     i.e. up to four 8-row tiles).
//   * K is consumed in chunks of kKC = 512 (four 128-K MFMA steps).  The
//     pass rows' activation chunk is staged in LDS (double-buffered) by all
//     256 threads; each wave then reads its B operands from LDS.
//   * Each wave keeps the NEXT chunk's weight loads in flight (a second
//     register buffer) while it computes the current chunk, so every wave has
//     several KB of weight reads outstanding at all times.

constexpr int kTP = 32;
constexpr int kKC = 512;
constexpr int kCS = kKC / 128;  // MFMA steps per chunk
constexpr int kRowB = kKC + 16; // padded LDS bytes per staged row
constexpr int kSclB = kKC / 32; // scale bytes per staged row and chunk

struct ActLds {
    uint8_t q[2][kTP * kRowB];
    uint8_t s[2][kTP * kSclB];
};

struct Stage {
    v4i d[4];
    uint32_t s[4];
};

// Global -> registers: thread t stages 64 bytes of row t/8 (part t%8) of the
// chunk starting at kbase, and threads < kTP stage that row's 16 scale bytes.
__device__ __forceinline__ void stage_load(Stage& st, const uint8_t* __restrict__ act_q,
                                           const uint8_t* __restrict__ act_s, int K,
                                           const int* s_row, int npass, int kbase) {
    const int tid = threadIdx.x, tok = tid >> 3, part = tid & 7;
    const int row = tok < npass ? s_row[tok] : -1;
    const int koff = kbase + part * 64;
    if (row >= 0 && koff < K) {
        const uint8_t* p = act_q + (size_t)row * K + koff;
#pragma unroll
        for (int q = 0; q < 4; ++q) st.d[q] = load16(p + 16 * q);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) st.d[q] = v4i{0, 0, 0, 0};
    }
    if (tid < kTP) {
        const int r2 = tid < npass ? s_row[tid] : -1;
        const int nd = min(4, (K - kbase) / 128);
        const uint32_t* sp = reinterpret_cast<const uint32_t*>(act_s + (size_t)(r2 < 0 ? 0 : r2) * (K / 32) + kbase / 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) st.s[q] = (r2 >= 0 && q < nd) ? sp[q] : 0x7f7f7f7fu;
    }
}

__device__ __forceinline__ void stage_store(const Stage& st, ActLds& L, int buf) {
    const int tid = threadIdx.x, tok = tid >> 3, part = tid & 7;
    uint8_t* dst = L.q[buf] + tok * kRowB + part * 64;
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<v4i*>(dst + 16 * q) = st.d[q];
    if (tid < kTP) {
#pragma unroll
        for (int q = 0; q < 4; ++q) *reinterpret_cast<uint32_t*>(L.s[buf] + tid * kSclB + 4 * q) = st.s[q];
    }
}

// Largest E8M0 scale code of each pass row over the whole K (NVFP4 path:
// activations enter the f16 MFMA as E4M3 * 2^(s - smax), inside f16 range).
// Written for all kTP rows of the pass.
__device__ void pass_row_smax(const uint8_t* act_s, int K, const int* s_row, int npass,
                              int* s_smax) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nsd = K / 128;  // scale dwords per row
    for (int tt = 0; tt < kTP / 4; ++tt) {
        const int t = wave * (kTP / 4) + tt;
        if (t >= npass) {  // padding rows: any finite offset (their codes are zero)
            if (lane == 0) s_smax[t] = 0;
            continue;
        }
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

// Weight registers of one chunk: NMB 16-row blocks x kCS steps (16 packed
// bytes per lane and step) with their scale words.
template <int NMB>
struct WChunk {
    v4i a[NMB][kCS];
    uint32_t s[NMB][kCS];
};

template <int FMT, int NMB>
__device__ __forceinline__ void wload(WChunk<NMB>& w, const uint8_t* const* wrow,
                                      const uint8_t* const* srow, int c, int steps) {
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
        for (int i = 0; i < kCS; ++i) {
            const int s = c * kCS + i;
            if (s < steps) {
                w.a[mb][i] = load16_nt(wrow[mb] + 64 * s + 16 * g);
                if constexpr (FMT == kFmtMX)
                    w.s[mb][i] = *reinterpret_cast<const uint32_t*>(srow[mb] + 4 * s) >> (8 * g);
                else
                    w.s[mb][i] = *reinterpret_cast<const uint16_t*>(srow[mb] + 8 * s + 2 * g);
            } else {
                w.a[mb][i] = v4i{0, 0, 0, 0};
                w.s[mb][i] = 0;
            }
        }
    }
}

// All kCS steps of a chunk are computed: past the end of K the weights are
// zero (wload) and so are the staged activations (stage_load), so the padding
// steps add exact zeros.  NB (16-row N-blocks of the pass, 1 or 2) is a
// compile-time constant: no branch separates an MFMA from the code that reads
// its accumulator.
template <int FMT, int NMB, int NB>
__device__ __forceinline__ void compute_chunk(const WChunk<NMB>& w, const ActLds& L, int buf,
                                              const int* s_smax, v4f (&acc)[NMB][2]) {
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, g = lane >> 4;
#pragma unroll
    for (int i = 0; i < kCS; ++i) {
        if constexpr (FMT == kFmtMX) {
            v8i B[NB];
            uint32_t sb[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int t = 16 * j + m;
                const uint8_t* rp = L.q[buf] + t * kRowB + 128 * i;
                const v4i b0 = *reinterpret_cast<const v4i*>(rp + 16 * g);
                const v4i b1 = *reinterpret_cast<const v4i*>(rp + 64 + 16 * g);
                B[j] = v8i{b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
                sb[j] = L.s[buf][t * kSclB + 4 * i + g];
            }
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) {
                const v4i a = w.a[mb][i];
                const v8i A = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[mb][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        A, B[j], acc[mb][j], 4, 0, 0, (int)w.s[mb][i], 0, (int)sb[j]);
            }
        } else {
            v8h B[NB][4];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int t = 16 * j + m;
                const uint8_t* rp = L.q[buf] + t * kRowB + 128 * i + 32 * g;
                const v4i b0 = *reinterpret_cast<const v4i*>(rp);
                const v4i b1 = *reinterpret_cast<const v4i*>(rp + 16);
                const int sb = L.s[buf][t * kSclB + 4 * i + g];
                const float sf = exp2i(max(sb - s_smax[t], -126));
                B[j][0] = fp8x8_to_f16((uint32_t)b0.x, (uint32_t)b0.y, sf);
                B[j][1] = fp8x8_to_f16((uint32_t)b0.z, (uint32_t)b0.w, sf);
                B[j][2] = fp8x8_to_f16((uint32_t)b1.x, (uint32_t)b1.y, sf);
                B[j][3] = fp8x8_to_f16((uint32_t)b1.z, (uint32_t)b1.w, sf);
            }
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) {
                const v4i a = w.a[mb][i];
                float sv0, sv1;
                _Float16 m0, m1;
                nv_scale_split(w.s[mb][i] & 0xffu, sv0, m0);
                nv_scale_split((w.s[mb][i] >> 8) & 0xffu, sv1, m1);
                const v8h A0 = nv_dequant8((uint32_t)a.x, sv0, m0);
                const v8h A1 = nv_dequant8((uint32_t)a.y, sv0, m0);
                const v8h A2 = nv_dequant8((uint32_t)a.z, sv1, m1);
                const v8h A3 = nv_dequant8((uint32_t)a.w, sv1, m1);
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
}

// Weight lookahead: a ring of RING chunk buffers keeps RING-1 chunks of
// weight loads in flight while one is consumed.  RING = 1 is the form for a K
// that fits one chunk (its single chunk is loaded up front).
template <int NMB, int RING>
struct WRing {
    WChunk<NMB> c[RING];
};

template <int RING>
constexpr int lookahead() { return RING > 1 ? RING - 1 : 1; }

// Issue the first chunks of weight loads (done as soon as the expert is
// known, before the row bookkeeping of the pass).
template <int FMT, int NMB, int RING>
__device__ __forceinline__ void ring_prologue(WRing<NMB, RING>& R, const uint8_t* const* wrow,
                                              const uint8_t* const* srow, int K) {
    const int steps = K / 128;
    const int nch = (steps + kCS - 1) / kCS;
#pragma unroll
    for (int d = 0; d < lookahead<RING>(); ++d)
        if (d < nch) wload<FMT, NMB>(R.c[d % RING], wrow, srow, d, steps);
}

// One pass: all of K for the wave's NMB weight blocks against the staged
// rows (NB 16-row N-blocks).  Activation chunks alternate between two LDS
// buffers (staged one chunk ahead by the whole workgroup); weights come from
// the ring (RING-1 chunks ahead).  Every wave of the workgroup runs the same
// chunk sequence.
template <int FMT, int NMB, int RING, int NB>
__device__ __forceinline__ void stream_pass(WRing<NMB, RING>& R, const uint8_t* const* wrow,
                                            const uint8_t* const* srow,
                                            const uint8_t* __restrict__ act_q,
                                            const uint8_t* __restrict__ act_s, int K,
                                            const int* s_row, const int* s_smax, int npass,
                                            ActLds& L, v4f (&acc)[NMB][2]) {
    const int steps = K / 128;
    const int nch = (steps + kCS - 1) / kCS;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[mb][j] = v4f{0.f, 0.f, 0.f, 0.f};
    Stage st;
    stage_load(st, act_q, act_s, K, s_row, npass, 0);
    stage_store(st, L, 0);
    __syncthreads();
    // RING == 1 is only used when nch == 1 (its lookahead load never fires).
    constexpr int LA = lookahead<RING>();
    constexpr int UN = RING > 1 ? RING : 2;  // unroll: ring slot and LDS buffer compile-time
    for (int c0 = 0; c0 < nch; c0 += UN) {
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int c = c0 + u;
            if (c >= nch) break;
            if (RING > 1 && c + LA < nch) wload<FMT, NMB>(R.c[(u + LA) % RING], wrow, srow, c + LA, steps);
            if (c + 1 < nch) stage_load(st, act_q, act_s, K, s_row, npass, (c + 1) * kKC);
            compute_chunk<FMT, NMB, NB>(R.c[u % RING], L, u & 1, s_smax, acc);
            if (c + 1 < nch) stage_store(st, L, (u + 1) & 1);
            __syncthreads();
        }
    }
}

template <int FMT, int NMB, int RING>
__device__ __forceinline__ void stream_pass_rows(WRing<NMB, RING>& R, const uint8_t* const* wrow,
                                                 const uint8_t* const* srow,
                                                 const uint8_t* __restrict__ act_q,
                                                 const uint8_t* __restrict__ act_s, int K,
                                                 const int* s_row, const int* s_smax, int npass,
                                                 ActLds& L, v4f (&acc)[NMB][2]) {
    if (npass > 16)
        stream_pass<FMT, NMB, RING, 2>(R, wrow, srow, act_q, act_s, K, s_row, s_smax, npass, L, acc);
    else
        stream_pass<FMT, NMB, RING, 1>(R, wrow, srow, act_q, act_s, K, s_row, s_smax, npass, L, acc);
}

// Per-row factor that turns an NVFP4 accumulator into the product value:
// 2^(smax - 127) (activation offset) * global.
__device__ __forceinline__ float nv_row_factor(int smax, float gs) { return ldexpf(gs, smax - 127); }

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
    const uint8_t* wrow[1] = {J.w + grow * (H / 2)};
    const uint8_t* srow[1] = {J.scales + grow * (FMT == kFmtMX ? H / 32 : H / 16)};
    const float gs = (FMT == kFmtNV) ? J.gscale[tk.e] : 1.0f;

    __shared__ __align__(16) ActLds L;
    __shared__ int s_row[kTP];
    __shared__ int s_smax[kTP];
    __shared__ float s_G[kTP][65];

    WRing<1, 4> R;
    ring_prologue<FMT, 1, 4>(R, wrow, srow, H);
    for (int t0 = 0; t0 < tk.n; t0 += kTP) {
        const int npass = min(kTP, tk.n - t0);
        const int nb = (npass + 15) / 16;
        if (t0 > 0) ring_prologue<FMT, 1, 4>(R, wrow, srow, H);
        if (threadIdx.x < kTP) {
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
        v4f acc[1][2];
        stream_pass_rows<FMT, 1>(R, wrow, srow, a_q, a_s, H, s_row, s_smax, npass, L, acc);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (j < nb) {
#pragma unroll
                for (int r = 0; r < 4; ++r) s_G[16 * j + m][wave * 16 + 4 * g + r] = acc[0][j][r];
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
                gt = s_G[t][col] * fac;
                up = s_G[t][32 + col] * fac;
            }
            hv[c] = gt / (1.0f + __expf(-gt)) * up;
        }
        uint8_t sc;
        const uint32_t codes = mx_quant4_group8(hv, sc);
        if (t < npass) {
            const size_t orow = (size_t)tk.base + t0 + t;
            *reinterpret_cast<uint32_t*>(h_q + orow * I + cb * 32 + 4 * q8) = codes;
            if (q8 == 0) h_s[orow * (I / 32) + cb] = sc;
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
// down, FP4 experts.  Item = (slot, 64*NMB output features); wave w owns NMB
// blocks of 16 features.  NMB grows as I shrinks so an item stays ~32-64 KB.

static int down_blocks_per_wave(int H, int I) {
    (void)H;
    if (I <= kKC) return 2;  // K fits one chunk: 2 blocks per wave, one load burst
    return 1;
}

template <int FMT, int NMB>
__global__ __launch_bounds__(256) void k_down_fp4(JobDev J, const uint8_t* __restrict__ h_q,
                                                  const uint8_t* __restrict__ h_s,
                                                  float* __restrict__ y) {
    const int H = J.N_out, I = J.K;
    constexpr int RB = 64 * NMB;
    const int NRB = H / RB;
    const int slot = blockIdx.x / NRB, rb = blockIdx.x % NRB;
    Tokens tk;
    if (!resolve(J, slot, tk)) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int m = lane & 15, g = lane >> 4;
    const float gs = (FMT == kFmtNV) ? J.gscale[tk.e] : 1.0f;
    const uint8_t* wrow[NMB];
    const uint8_t* srow[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
        const size_t grow = (size_t)tk.e * H + rb * RB + wave * (16 * NMB) + mb * 16 + m;
        wrow[mb] = J.w + grow * (I / 2);
        srow[mb] = J.scales + grow * (FMT == kFmtMX ? I / 32 : I / 16);
    }

    __shared__ __align__(16) ActLds L;
    __shared__ int s_row[kTP];
    __shared__ int s_out[kTP];
    __shared__ int s_smax[kTP];

    constexpr int RING = NMB > 1 ? 1 : 4;  // NMB > 1 only when K fits one chunk
    WRing<NMB, RING> R;
    ring_prologue<FMT, NMB, RING>(R, wrow, srow, I);
    for (int t0 = 0; t0 < tk.n; t0 += kTP) {
        const int npass = min(kTP, tk.n - t0);
        const int nb = (npass + 15) / 16;
        if (t0 > 0) ring_prologue<FMT, NMB, RING>(R, wrow, srow, I);
        if (threadIdx.x < kTP) {
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
        v4f acc[NMB][2];
        stream_pass_rows<FMT, NMB>(R, wrow, srow, h_q, h_s, I, s_row, s_smax, npass, L, acc);
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
            const int f0 = rb * RB + wave * (16 * NMB) + mb * 16;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int t = 16 * j + m;
                if (j < nb && t < npass) {
                    v4f v = acc[mb][j];
                    if (FMT == kFmtNV) v = v * nv_row_factor(s_smax[t], gs);
                    *reinterpret_cast<v4f*>(y + (size_t)s_out[t] * H + f0 + 4 * g) = v;
                }
            }
        }
        __syncthreads();
    }
}

template <int FMT>
static void launch_down_fmt(int nmb, int blocks, hipStream_t stream, const JobDev& J,
                            const uint8_t* h_q, const uint8_t* h_s, float* y) {
    if (nmb == 2)
        hipLaunchKernelGGL((k_down_fp4<FMT, 2>), dim3(blocks), dim3(256), 0, stream, J, h_q, h_s, y);
    else
        hipLaunchKernelGGL((k_down_fp4<FMT, 1>), dim3(blocks), dim3(256), 0, stream, J, h_q, h_s, y);
}

hipError_t launch_down_fp4(const ExpertJob& job, const uint8_t* h_q, const uint8_t* h_s,
                           float* y, hipStream_t stream) {
    const JobDev J = to_dev(job);
    const int nmb = down_blocks_per_wave(job.N_out, job.K);
    const int blocks = job.slots * (job.N_out / (64 * nmb));
    if (job.w.fmt == MOE_FMT_MXFP4)
        launch_down_fmt<kFmtMX>(nmb, blocks, stream, J, h_q, h_s, y);
    else
        launch_down_fmt<kFmtNV>(nmb, blocks, stream, J, h_q, h_s, y);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bf16 shared expert (dense over all M rows).  gate_up splits K across S
// workgroups per 32-column block; partial sums go to the workspace and a
// second launch adds them in split order (deterministic), applies SwiGLU and
// rounds h to bf16.  (A last-arriver reduction inside one launch would need a
// device-scope release fence per workgroup, which on this GPU writes back the
// L2 and costs far more than the extra launch.)

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

// bf16 A x bf16 B over K range [k0, k1) (multiple of 32), up to 4 N-blocks.
// Loads for 8 K-steps are issued together before their MFMAs.
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
    constexpr int U = 8;
    for (int kb = k0; kb < k1; kb += 32 * U) {
        v4i a[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kk = kb + 32 * u;
            a[u] = (kk < k1) ? load16_nt(wrow + kk + 8 * g) : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < nb) {
                v4i b[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int kk = kb + 32 * u;
                    b[u] = (rowj[j] >= 0 && kk < k1) ? load16(act + (size_t)rowj[j] * K + kk + 8 * g)
                                                     : v4i{0, 0, 0, 0};
                }
#pragma unroll
                for (int u = 0; u < U; ++u)
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[u]),
                                                                     __builtin_bit_cast(v8bf, b[u]),
                                                                     acc[j], 0, 0, 0);
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_gate_up_bf16(JobDev J, int splits,
                                                      const uint16_t* __restrict__ a,
                                                      float* __restrict__ part) {
    const int I = J.N_out, H = J.K, M = J.M;
    const int cb = blockIdx.x / splits, ks = blockIdx.x % splits;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int m = lane & 15, g = lane >> 4;
    const int wr = (wave >> 1) * I + cb * 32 + (wave & 1) * 16 + m;
    const uint16_t* wrow = reinterpret_cast<const uint16_t*>(J.w) + (size_t)wr * H;
    const int kc = H / splits;
    __shared__ int s_row[kPass];
    for (int t0 = 0; t0 < M; t0 += kPass) {
        const int npass = min(kPass, M - t0);
        const int nb = (npass + 15) / 16;
        if (threadIdx.x < kPass) s_row[threadIdx.x] = threadIdx.x < npass ? t0 + threadIdx.x : -1;
        __syncthreads();
        v4f acc[4];
        wave_gemm_bf16(wrow, a, H, ks * kc, (ks + 1) * kc, s_row, nb, acc);
        // partial G: [split][row][2I]; this lane: features wr-block rows 4g+r
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = 16 * j + m;
            if (j < nb && t < npass) {
                const int col = (wave >> 1) * I + cb * 32 + (wave & 1) * 16 + 4 * g;
                *reinterpret_cast<v4f*>(part + ((size_t)ks * M + t0 + t) * (2 * I) + col) = acc[j];
            }
        }
        __syncthreads();
    }
}

// Sum of the split-K partials in split order, SwiGLU, bf16 rounding of h.
// A separate launch, so every partial is visible without a device-scope fence.
__global__ __launch_bounds__(256) void k_bf16_swiglu(const float* __restrict__ part, int splits,
                                                     int M, int I, uint16_t* __restrict__ h) {
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= M * I) return;
    const int t = idx / I, col = idx % I;
    float gt = 0.f, up = 0.f;
    for (int s0 = 0; s0 < splits; s0 += 8) {
        float pg[8], pu[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int sp = s0 + u;
            const float* pr = part + ((size_t)(sp < splits ? sp : 0) * M + t) * (2 * I);
            pg[u] = sp < splits ? pr[col] : 0.f;
            pu[u] = sp < splits ? pr[I + col] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (s0 + u < splits) {
                gt += pg[u];
                up += pu[u];
            }
        }
    }
    const float hv = gt / (1.0f + __expf(-gt)) * up;
    h[(size_t)t * I + col] = (uint16_t)f32_to_bf16_rne(hv);
}

hipError_t launch_gate_up_bf16(const ExpertJob& job, const uint16_t* a, uint16_t* h,
                               float* part, hipStream_t stream) {
    const JobDev J = to_dev(job);
    const Bf16Plan p = bf16_plan(job.K, job.N_out);
    const int blocks = (job.N_out / 32) * p.splits;
    hipLaunchKernelGGL(k_gate_up_bf16, dim3(blocks), dim3(256), 0, stream, J, p.splits, a, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n = job.M * job.N_out;
    hipLaunchKernelGGL(k_bf16_swiglu, dim3((n + 255) / 256), dim3(256), 0, stream, part, p.splits,
                       job.M, job.N_out, h);
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
