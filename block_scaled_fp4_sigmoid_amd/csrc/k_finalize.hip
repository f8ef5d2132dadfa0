// k_finalize.hip — top-k weighted finalize fused with the shared-expert add,
// the residual add and RMSNorm (gfx950).
//
// Pages: SGLang-NVIDIA-Mega README, DeepSeek-V4.1 slot table, rows "hop_b"
// and "two_shot" (the finalize folded with the shared-expert add before the
// next norm); README Qwen3.5 slot table, row "hop" (fused residual add +
// RMSNorm).  t = residual + y_sh + sum_j w_j y_j (fp32, slot order);
// residual_out = bf16_rne(t); out = bf16_rne(r' * rsqrt(mean(r'^2) + eps) * gamma).
//
// One workgroup per row; each thread owns 8 consecutive columns per 2048.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kFinThreads = 256;

__global__ __launch_bounds__(kFinThreads) void k_finalize(const float* __restrict__ y,
                                                          const float* __restrict__ topk_w,
                                                          const float* __restrict__ y_sh,
                                                          const uint16_t* residual,
                                                          const uint16_t* __restrict__ gamma,
                                                          float eps, int H, int k,
                                                          uint16_t* out, uint16_t* residual_out) {
    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    constexpr int kMaxChunks = 8;  // H <= 16384 = 8 * 2048
    float rv[kMaxChunks][8];
    float ss = 0.f;
    const float* wr = topk_w + (size_t)r * k;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        const int col = c * 2048 + tid * 8;
        if (col < H) {
            const v4i rb = load16(residual + (size_t)r * H + col);
            uint32_t rw[4] = {(uint32_t)rb.x, (uint32_t)rb.y, (uint32_t)rb.z, (uint32_t)rb.w};
            float t[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                t[2 * i] = bf16_to_f32(rw[i] & 0xffffu);
                t[2 * i + 1] = bf16_to_f32(rw[i] >> 16);
            }
            if (y_sh) {
                const float4 a = *reinterpret_cast<const float4*>(y_sh + (size_t)r * H + col);
                const float4 b = *reinterpret_cast<const float4*>(y_sh + (size_t)r * H + col + 4);
                t[0] += a.x; t[1] += a.y; t[2] += a.z; t[3] += a.w;
                t[4] += b.x; t[5] += b.y; t[6] += b.z; t[7] += b.w;
            }
            for (int j = 0; j < k; ++j) {
                const float wj = wr[j];
                const float* yr = y + ((size_t)r * k + j) * H + col;
                const float4 a = *reinterpret_cast<const float4*>(yr);
                const float4 b = *reinterpret_cast<const float4*>(yr + 4);
                t[0] = fmaf(wj, a.x, t[0]); t[1] = fmaf(wj, a.y, t[1]);
                t[2] = fmaf(wj, a.z, t[2]); t[3] = fmaf(wj, a.w, t[3]);
                t[4] = fmaf(wj, b.x, t[4]); t[5] = fmaf(wj, b.y, t[5]);
                t[6] = fmaf(wj, b.z, t[6]); t[7] = fmaf(wj, b.w, t[7]);
            }
            uint32_t ob[4];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t bits = f32_to_bf16_rne(t[i]);
                rv[c][i] = bf16_to_f32(bits);
                ss = fmaf(rv[c][i], rv[c][i], ss);
                if (i & 1) ob[i >> 1] |= bits << 16;
                else ob[i >> 1] = bits;
            }
            if (residual_out)
                *reinterpret_cast<v4i*>(residual_out + (size_t)r * H + col) =
                    v4i{(int)ob[0], (int)ob[1], (int)ob[2], (int)ob[3]};
        }
    }
    // fixed-order reduction: wave butterfly, then the 4 wave sums in order
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    __shared__ float s_part[kFinThreads / 64];
    if ((tid & 63) == 0) s_part[tid >> 6] = ss;
    __syncthreads();
    const float tot = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
    const float inv = rsqrtf(tot / (float)H + eps);
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        const int col = c * 2048 + tid * 8;
        if (col < H) {
            const v4i gb = load16(gamma + col);
            uint32_t gw[4] = {(uint32_t)gb.x, (uint32_t)gb.y, (uint32_t)gb.z, (uint32_t)gb.w};
            uint32_t ob[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float o0 = rv[c][2 * i] * inv * bf16_to_f32(gw[i] & 0xffffu);
                const float o1 = rv[c][2 * i + 1] * inv * bf16_to_f32(gw[i] >> 16);
                ob[i] = f32_to_bf16_rne(o0) | (f32_to_bf16_rne(o1) << 16);
            }
            *reinterpret_cast<v4i*>(out + (size_t)r * H + col) = v4i{(int)ob[0], (int)ob[1], (int)ob[2], (int)ob[3]};
        }
    }
}

hipError_t launch_finalize(const float* y, const float* topk_w, const float* y_sh,
                           const uint16_t* residual, const uint16_t* gamma, float eps, int M,
                           int H, int k, uint16_t* out, uint16_t* residual_out,
                           hipStream_t stream) {
    hipLaunchKernelGGL(k_finalize, dim3(M), dim3(kFinThreads), 0, stream, y, topk_w, y_sh,
                       residual, gamma, eps, H, k, out, residual_out);
    return hipGetLastError();
}

}  // namespace moe
