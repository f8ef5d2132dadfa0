// moe_device.h — device helpers shared by the layer's gfx950 kernels
// (private to this library; not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v2s __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// SwiGLU of one gate/up pair: silu(g) * u with silu(g) = g / (1 + e^-g).
// limit > 0 is the clamped form (README DeepSeek-V4.1 slot table, row
// "Shared expert gate_up (shared_ll)"): the gate capped from above at limit
// and up clamped to [-limit, limit] before the product; NaN passes through.
__device__ __forceinline__ float swiglu(float g, float u, float limit) {
    if (limit > 0.0f) {
        g = g > limit ? limit : g;
        u = u > limit ? limit : (u < -limit ? -limit : u);
    }
    return g / (1.0f + __expf(-g)) * u;
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet, sign kept).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// 2^e as fp32 for e in [-126, 127].
__device__ __forceinline__ float exp2i(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// Two fp32 values (already divided by the block scale, |v| < 512, finite)
// -> two E4M3 codes, round to nearest even, saturating at +-448.  The
// hardware conversion rounds to nearest even below 448 and overflows to NaN
// from 464 up, so clamping first gives the saturating rule.
__device__ __forceinline__ uint32_t e4m3x2_sat(float a, float b) {
    a = fminf(fmaxf(a, -448.0f), 448.0f);
    b = fminf(fmaxf(b, -448.0f), 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// Shared MXFP8 exponent from the largest |value| of a block, given as the
// fp32 bit pattern with the sign cleared: floor(log2 amax) - 8, clamped at
// -127 (amax = 0 and subnormal amax land on the clamp).
__device__ __forceinline__ int mx_shared_exp(uint32_t amax_bits) {
    int e = (int)((amax_bits >> 23) & 0xff) - 127 - 8;
    return e < -127 ? -127 : e;
}

__device__ __forceinline__ bool f32_bits_special(uint32_t bits) { return (bits & 0x7f800000u) == 0x7f800000u; }

template <typename T>
__device__ __forceinline__ T wave_shfl_xor(T v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

// Relaxed device-scope load (bypasses a possibly stale per-CU cache line).
template <typename T>
__device__ __forceinline__ T load_agent(const T* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Raw buffer resource over [p, p + bytes): loads at offsets at or past `bytes`
// return zeros and stores there are dropped, without a memory access.  Every
// buffer the kernels address this way holds fewer than 2^31 bytes (the C ABI
// refuses larger shapes), so kOOB is past every record count.
constexpr uint32_t kOOB = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ v4i load16(const void* p) { return *reinterpret_cast<const v4i*>(p); }
__device__ __forceinline__ v4i load16_nt(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
}

}  // namespace moe
