// k_finalize.hip — top-k weighted finalize fused with the shared-expert add,
// the residual add and RMSNorm (gfx950).
//
// Pages: SGLang-NVIDIA-Mega README, DeepSeek-V4.1 slot table, rows "hop_b"
// and "two_shot" (the finalize folded with the shared-expert add before the
// next norm); README Qwen3.5 slot table, row "hop" (fused residual add +
// RMSNorm).  t = residual + y_sh + sum_j w_j y_j (fp32, slot order);
// residual_out = bf16_rne(t); out = bf16_rne(r' * rsqrt(mean(r'^2) + eps) * gamma).
// Optionally also the next layer's input as MXFP8 (same slot table, row
// "hop_b": the next input's MXFP8 scales written by the norm's consumer):
// the one-pass quant rule applied to the bf16 out, codes [M][H] and scales
// [M][H/32] as the activation quant lays them out.
//
// One workgroup per row; each thread owns 8 consecutive columns per NT * 8
// (four neighbouring lanes hold one 32-value block).  Up to H = 4096 a row
// takes 512 threads, whose registers hold 16 pairs' loads at once (k <= 16 in
// one round of loads); above, 1024 threads and rounds of 8 pairs.  y is [M*k][H] by pair,
// or grouped as the fused layer's down writes it (pair p's row at yrec[p]:
// its first 128-column block at yrec[p].x floats, the next ones yrec[p].y * 128
// floats further each); y_sh likewise [M][H] or grouped (rows 0..M-1 taken as
// one expert's).
#include "moe_device.h"
#include "moe_internal.h"
#include "quant_dev.h"

namespace moe {

// NT threads per row, KB pairs per round of loads, NC passes of NT * 8 columns
template <int NT, int KB, int NC>
__global__ __launch_bounds__(NT) void k_finalize(const float* __restrict__ y,
                                                          const float* __restrict__ topk_w,
                                                          const float* __restrict__ y_sh,
                                                          const uint16_t* residual,
                                                          const uint16_t* __restrict__ gamma,
                                                          float eps, int H, int k,
                                                          uint16_t* out, uint16_t* residual_out,
                                                          uint8_t* __restrict__ out_q,
                                                          uint8_t* __restrict__ out_s,
                                                          const int2* __restrict__ yrec, int ysh_grp,
                                                          int M) {
    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    constexpr int kFinChunk = NT * 8;  // columns per pass of the workgroup
    constexpr int kMaxChunks = NC;     // H <= NC * NT * 8
    constexpr int kBatch = KB;         // slots whose loads are in flight together
    float rv[kMaxChunks][8];
    uint32_t gw[kMaxChunks][4];
    float ss = 0.f;
    const float* wr = topk_w + (size_t)r * k;
    // the row of y_sh: grouped, its group of min(16, M - g0) rows from row g0
    const int g0 = r & ~(kYGroupRows - 1);
    const size_t sh_row = ysh_grp ? (size_t)g0 * H + (r - g0) * kYBlockCols : (size_t)r * H;
    const int sh_blk = ysh_grp ? min(kYGroupRows, M - g0) * kYBlockCols : kYBlockCols;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        const int col = c * kFinChunk + tid * 8;
        if (col < H) {
            // every operand of the column group is requested before the first add
            const v4i rb = load16(residual + (size_t)r * H + col);
            const v4i gb = load16(gamma + col);
            float4 sa = {0.f, 0.f, 0.f, 0.f}, sb = sa;
            if (y_sh) {
                const float* ys = y_sh + sh_row + (size_t)(col / kYBlockCols) * sh_blk + col % kYBlockCols;
                sa = *reinterpret_cast<const float4*>(ys);
                sb = *reinterpret_cast<const float4*>(ys + 4);
            }
            gw[c][0] = (uint32_t)gb.x; gw[c][1] = (uint32_t)gb.y; gw[c][2] = (uint32_t)gb.z; gw[c][3] = (uint32_t)gb.w;
            float t[8];
            const uint32_t rw[4] = {(uint32_t)rb.x, (uint32_t)rb.y, (uint32_t)rb.z, (uint32_t)rb.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                t[2 * i] = bf16_to_f32(rw[i] & 0xffffu);
                t[2 * i + 1] = bf16_to_f32(rw[i] >> 16);
            }
            t[0] += sa.x; t[1] += sa.y; t[2] += sa.z; t[3] += sa.w;
            t[4] += sb.x; t[5] += sb.y; t[6] += sb.z; t[7] += sb.w;
            // slot order
            for (int j0 = 0; j0 < k; j0 += kBatch) {
                float4 ya[kBatch], yb[kBatch];
                float wj[kBatch];
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int j = j0 + u;
                    if (j < k) {
                        const size_t p = (size_t)r * k + j;
                        int2 yp = {(int)(p * H), 1};  // by pair: one row per "group"
                        if (yrec) yp = yrec[p];
                        const float* yr = y + (size_t)yp.x + (size_t)(col / kYBlockCols) * (yp.y * kYBlockCols) +
                                          col % kYBlockCols;
                        ya[u] = *reinterpret_cast<const float4*>(yr);
                        yb[u] = *reinterpret_cast<const float4*>(yr + 4);
                        wj[u] = wr[j];
                    }
                }
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    if (j0 + u < k) {
                        t[0] = fmaf(wj[u], ya[u].x, t[0]); t[1] = fmaf(wj[u], ya[u].y, t[1]);
                        t[2] = fmaf(wj[u], ya[u].z, t[2]); t[3] = fmaf(wj[u], ya[u].w, t[3]);
                        t[4] = fmaf(wj[u], yb[u].x, t[4]); t[5] = fmaf(wj[u], yb[u].y, t[5]);
                        t[6] = fmaf(wj[u], yb[u].z, t[6]); t[7] = fmaf(wj[u], yb[u].w, t[7]);
                    }
                }
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
    // fixed-order reduction: wave butterfly, then the wave sums in order
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    __shared__ float s_part[NT / 64];
    if ((tid & 63) == 0) s_part[tid >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) tot += s_part[w];
    const float inv = rsqrtf(tot / (float)H + eps);
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        const int col = c * kFinChunk + tid * 8;
        if (col < H) {
            uint32_t ob[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float o0 = rv[c][2 * i] * inv * bf16_to_f32(gw[c][i] & 0xffffu);
                const float o1 = rv[c][2 * i + 1] * inv * bf16_to_f32(gw[c][i] >> 16);
                ob[i] = f32_to_bf16_rne(o0) | (f32_to_bf16_rne(o1) << 16);
            }
            *reinterpret_cast<v4i*>(out + (size_t)r * H + col) = v4i{(int)ob[0], (int)ob[1], (int)ob[2], (int)ob[3]};
            if (out_q) {
                // H % 32 == 0: the four lanes of a block are all in range
                uint8_t sc;
                const uint2 codes = quant_bf16x8_lanes4(ob, sc);
                *reinterpret_cast<uint2*>(out_q + (size_t)r * H + col) = codes;
                if ((tid & 3) == 0) out_s[(size_t)r * (H / 32) + col / 32] = sc;
            }
        }
    }
}

hipError_t launch_finalize(const float* y, const float* topk_w, const float* y_sh,
                           const uint16_t* residual, const uint16_t* gamma, float eps, int M,
                           int H, int k, uint16_t* out, uint16_t* residual_out, uint8_t* out_q,
                           uint8_t* out_s, hipStream_t stream, const int2* yrec, bool ysh_grouped) {
    if (H <= 512 * 8)
        hipLaunchKernelGGL((k_finalize<512, 16, 1>), dim3(M), dim3(512), 0, stream, y, topk_w, y_sh, residual, gamma,
                           eps, H, k, out, residual_out, out_q, out_s, yrec, ysh_grouped ? 1 : 0, M);
    else
        hipLaunchKernelGGL((k_finalize<1024, 8, 2>), dim3(M), dim3(1024), 0, stream, y, topk_w, y_sh, residual, gamma,
                           eps, H, k, out, residual_out, out_q, out_s, yrec, ysh_grouped ? 1 : 0, M);
    return hipGetLastError();
}

}  // namespace moe
