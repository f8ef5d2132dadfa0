// quant_dev.h — one 32-value MXFP8 block (device code shared by the quant
// kernels).
//
// Pages: SGLang-NVIDIA-Mega README, DeepSeek-V4.1 slot table, row "Shared
// expert gate_up (shared_ll)" (a one-pass MXFP8 quant of the activations).
// Rule (OCP MX v1.0; the pages state none): shared exponent = floor(log2
// amax) - 8 clamped at -127; elements = E4M3 RNE of x / 2^shared, saturated
// at 448; NaN/Inf blocks get scale 0xFF and NaN codes.
#pragma once
#include "moe_device.h"

namespace moe {

// One 32-value block: src -> 32 codes at q, scale code at *s.
__device__ __forceinline__ void quant_block32(const uint16_t* __restrict__ xsrc, uint8_t* __restrict__ qdst,
                                              uint8_t* __restrict__ sdst) {
    const v4i* src = reinterpret_cast<const v4i*>(xsrc);
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const v4i v = src[i];
        w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
    uint32_t amax = 0;
    bool special = false;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t lo = w[i] & 0x7fffu, hi = (w[i] >> 16) & 0x7fffu;
        amax = max(amax, max(lo, hi));
        special |= (lo & 0x7f80u) == 0x7f80u || (hi & 0x7f80u) == 0x7f80u;
    }
    uint32_t out[8];
    uint8_t scale;
    if (special) {
        scale = 0xff;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t o = 0;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t wd = w[2 * i + h];
                o |= (((wd >> 8) & 0x80u) | 0x7fu) << (16 * h);
                o |= (((wd >> 24) & 0x80u) | 0x7fu) << (16 * h + 8);
            }
            out[i] = o;
        }
    } else {
        const int shared = mx_shared_exp(amax << 16);
        scale = (uint8_t)(shared + 127);
        const float f = exp2i(-shared);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t c0 = e4m3x2_sat(bf16_to_f32(w[2 * i] & 0xffffu) * f, bf16_to_f32(w[2 * i] >> 16) * f);
            const uint32_t c1 = e4m3x2_sat(bf16_to_f32(w[2 * i + 1] & 0xffffu) * f, bf16_to_f32(w[2 * i + 1] >> 16) * f);
            out[i] = c0 | (c1 << 16);
        }
    }
    v4i* dst = reinterpret_cast<v4i*>(qdst);
    dst[0] = v4i{(int)out[0], (int)out[1], (int)out[2], (int)out[3]};
    dst[1] = v4i{(int)out[4], (int)out[5], (int)out[6], (int)out[7]};
    *sdst = scale;
}

}  // namespace moe

namespace moe {

// The same rule over a block spread across four neighbouring lanes (lanes
// 4j..4j+3, eight bf16 values each, packed two per word in w): the amax and
// the special flag are combined over the four lanes.  All four lanes must be
// active.  Returns the lane's eight codes (first value in the low byte of .x);
// *scale is the block's scale code.
__device__ __forceinline__ uint2 quant_bf16x8_lanes4(const uint32_t w[4], uint8_t& scale) {
    uint32_t amax = 0;
    int special = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = w[i] & 0x7fffu, hi = (w[i] >> 16) & 0x7fffu;
        amax = max(amax, max(lo, hi));
        special |= ((lo & 0x7f80u) == 0x7f80u || (hi & 0x7f80u) == 0x7f80u) ? 1 : 0;
    }
#pragma unroll
    for (int off = 1; off < 4; off <<= 1) {
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, off, 64));
        special |= __shfl_xor(special, off, 64);
    }
    uint32_t out[2];
    if (special) {
        scale = 0xff;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            uint32_t o = 0;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t wd = w[2 * i + h];
                o |= (((wd >> 8) & 0x80u) | 0x7fu) << (16 * h);
                o |= (((wd >> 24) & 0x80u) | 0x7fu) << (16 * h + 8);
            }
            out[i] = o;
        }
    } else {
        const int shared = mx_shared_exp(amax << 16);
        scale = (uint8_t)(shared + 127);
        const float f = exp2i(-shared);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t c0 = e4m3x2_sat(bf16_to_f32(w[2 * i] & 0xffffu) * f, bf16_to_f32(w[2 * i] >> 16) * f);
            const uint32_t c1 =
                e4m3x2_sat(bf16_to_f32(w[2 * i + 1] & 0xffffu) * f, bf16_to_f32(w[2 * i + 1] >> 16) * f);
            out[i] = c0 | (c1 << 16);
        }
    }
    return uint2{out[0], out[1]};
}

}  // namespace moe

// ---- NVFP4 activations ---------------------------------------------------------
// Pages: README Qwen3.5 slot table, rows "route" (NVFP4 quant of the MoE input
// in the router launch) and "mkm" (NVFP4 requant of the SwiGLU output before
// FC2).  Rule (the pages state none): the NVFP4 weight encoding applied with a
// static fp32 global g, every step in fp32 —
//   a block of 16 values with a non-finite value: scale 0x7F, codes 0;
//   else s = amax / (6 g) (the product rounded, then the quotient), scale =
//   E4M3 RNE of s saturating at 448, sd its value; sd == 0: codes 0; else
//   code = E2M1 RNE of v / (sd g) (product, then quotient) saturating at 6,
//   with the quotient's sign bit.
// Codes pack two per byte, the even element in the low nibble.
namespace moe {

// E2M1 code of q: magnitude by threshold (ties go to the even code: > at the
// midpoints below an odd code, >= below an even one), saturating at 6.
__device__ __forceinline__ uint32_t e2m1_rne_sat(float q) {
    const float a = fabsf(q);
    const uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
    return m | ((__float_as_uint(q) >> 28) & 8u);
}

// Scale code and the divisor sd * g of a finite block with largest magnitude amax.
__device__ __forceinline__ uint32_t nvfp4_scale(float amax, float g, float& d) {
    const float t = 6.0f * g;
    const float s = fminf(amax / t, 448.0f);
    const uint32_t sc = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(s, s, 0, false) & 0xffu;
    d = __builtin_amdgcn_cvt_f32_fp8((int)sc, 0) * g;
    return sc;
}

__device__ __forceinline__ bool f32_nonfinite(float v) { return (__float_as_uint(v) & 0x7f800000u) == 0x7f800000u; }

// One block of 16 values held by one thread: returns the 8 code bytes (first
// value in the low nibble of .x), the scale code in *sc.
__device__ __forceinline__ uint2 nvfp4_quant16(const float (&v)[16], float g, uint8_t& sc) {
    float amax = 0.0f;
    bool special = false;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        special |= f32_nonfinite(v[i]);
        amax = fmaxf(amax, fabsf(v[i]));
    }
    if (special) {
        sc = 0x7F;
        return uint2{0u, 0u};
    }
    float d;
    sc = (uint8_t)nvfp4_scale(amax, g, d);
    uint32_t w[2] = {0u, 0u};
    if (d != 0.0f) {
#pragma unroll
        for (int i = 0; i < 16; ++i) w[i >> 3] |= e2m1_rne_sat(v[i] / d) << (4 * (i & 7));
    }
    return uint2{w[0], w[1]};
}

// A block spread over four neighbouring lanes (lanes 4j..4j+3, four values
// each): amax and the special flag are combined over the four lanes; returns
// the lane's four codes (16 bits, first value lowest); *sc is the block's
// scale code.  All four lanes must be active.
__device__ __forceinline__ uint32_t nvfp4_quant4_lanes4(const float (&v)[4], float g, uint8_t& sc) {
    float amax = 0.0f;
    int special = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        special |= f32_nonfinite(v[i]) ? 1 : 0;
        amax = fmaxf(amax, fabsf(v[i]));
    }
#pragma unroll
    for (int off = 1; off < 4; off <<= 1) {
        amax = fmaxf(amax, __shfl_xor(amax, off, 64));
        special |= __shfl_xor(special, off, 64);
    }
    if (special) {
        sc = 0x7F;
        return 0u;
    }
    float d;
    sc = (uint8_t)nvfp4_scale(amax, g, d);
    uint32_t w = 0u;
    if (d != 0.0f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) w |= e2m1_rne_sat(v[i] / d) << (4 * i);
    }
    return w;
}

// One block of 16 bf16 values (32 bytes at src) -> 8 code bytes at q, scale at *s.
__device__ __forceinline__ void quant_nvfp4_bf16x16(const uint16_t* __restrict__ src, float g, uint8_t* __restrict__ q,
                                                    uint8_t* __restrict__ s) {
    const v4i* p = reinterpret_cast<const v4i*>(src);
    const v4i a = p[0], b = p[1];
    const uint32_t w[8] = {(uint32_t)a.x, (uint32_t)a.y, (uint32_t)a.z, (uint32_t)a.w,
                           (uint32_t)b.x, (uint32_t)b.y, (uint32_t)b.z, (uint32_t)b.w};
    float v[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = bf16_to_f32(w[i] & 0xffffu);
        v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
    uint8_t sc;
    const uint2 c = nvfp4_quant16(v, g, sc);
    *reinterpret_cast<uint2*>(q) = c;
    *s = sc;
}

}  // namespace moe
