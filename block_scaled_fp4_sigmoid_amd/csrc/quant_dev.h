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
