// k_quant.hip — one-pass MXFP8 quantization of bf16 activation rows (gfx950).
//
// Pages: SGLang-NVIDIA-Mega README, DeepSeek-V4.1 slot table, row "Shared
// expert gate_up (shared_ll)" (a one-pass MXFP8 quant of the activations).
// Rule (OCP MX v1.0, the pages state none): per 32 values, shared exponent =
// floor(log2 amax) - 8 clamped at -127; elements = E4M3 RNE of x / 2^shared,
// saturated at 448; NaN/Inf blocks get scale 0xFF and NaN codes.
//
// One thread per 32-value block: 64 bytes in (four 16-byte loads), 32 bytes +
// one scale byte out.  amax comes from the bf16 bit patterns (integer max of
// the magnitudes, exact for subnormals too).
//
// With a routing the rows are written in bucket order (row of bucket position
// b = the token of pair bucket[b]), so the expert GEMMs find an expert's rows
// contiguous.
#include "moe_device.h"
#include "moe_internal.h"
#include "quant_dev.h"

namespace moe {

__global__ __launch_bounds__(256) void k_quant_mxfp8(const uint16_t* __restrict__ x, int nblocks,
                                                     uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
    const int b = blockIdx.x * 256 + threadIdx.x;
    if (b >= nblocks) return;
    quant_block32(x + (size_t)b * 32, q + (size_t)b * 32, s + b);
}

// Rows [0, P): bucket order (row b = token bucket[b] / k); rows [P, P + Mt):
// token order into qt/st (Mt = M, or 0 when no token-ordered copy is wanted).
__global__ __launch_bounds__(256) void k_quant_pairs(const uint16_t* __restrict__ x,
                                                     const int32_t* __restrict__ bucket, int k, int P, int Mt,
                                                     int K, uint8_t* __restrict__ qp, uint8_t* __restrict__ sp,
                                                     uint8_t* __restrict__ qt, uint8_t* __restrict__ st) {
    const int bpr = K / 32;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    const int row = idx / bpr, blk = idx - row * bpr;
    if (row >= P + Mt) return;
    if (row < P) {
        const int tok = bucket[row] / k;
        quant_block32(x + (size_t)tok * K + 32 * blk, qp + (size_t)row * K + 32 * blk, sp + (size_t)row * bpr + blk);
    } else {
        const int tok = row - P;
        quant_block32(x + (size_t)tok * K + 32 * blk, qt + (size_t)tok * K + 32 * blk, st + (size_t)tok * bpr + blk);
    }
}

// NVFP4 activations (rule in quant_dev.h): one thread per 16-value block, 32
// bytes in, 8 code bytes + one scale byte out.  With a bucket, rows in bucket
// order (row b = token bucket[b] / k); without, row order.
__global__ __launch_bounds__(256) void k_quant_nvfp4(const uint16_t* __restrict__ x, const int32_t* __restrict__ bucket,
                                                     int k, int rows, int K, float g, uint8_t* __restrict__ q,
                                                     uint8_t* __restrict__ s) {
    const int bpr = K / 16;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    const int row = idx / bpr, blk = idx - row * bpr;
    if (row >= rows) return;
    const int tok = bucket ? bucket[row] / k : row;
    quant_nvfp4_bf16x16(x + (size_t)tok * K + 16 * blk, g, q + (size_t)row * (K / 2) + 8 * blk,
                        s + (size_t)row * bpr + blk);
}

hipError_t launch_quant_nvfp4(const uint16_t* x, const int32_t* bucket, int k, int rows, int K, float g, uint8_t* q,
                              uint8_t* s, hipStream_t stream) {
    const long n = (long)rows * (K / 16);
    hipLaunchKernelGGL(k_quant_nvfp4, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, x, bucket, k, rows, K, g,
                       q, s);
    return hipGetLastError();
}

hipError_t launch_quant_mxfp8(const uint16_t* x, int M, int K, uint8_t* q, uint8_t* s,
                              hipStream_t stream) {
    const int nblocks = M * (K / 32);
    hipLaunchKernelGGL(k_quant_mxfp8, dim3((nblocks + 255) / 256), dim3(256), 0, stream, x, nblocks, q, s);
    return hipGetLastError();
}

hipError_t launch_quant_pairs(const uint16_t* x, const int32_t* bucket, int k, int M, int K, uint8_t* qp,
                              uint8_t* sp, uint8_t* qt, uint8_t* st, hipStream_t stream) {
    const int P = M * k, Mt = qt ? M : 0;
    const long n = (long)(P + Mt) * (K / 32);
    hipLaunchKernelGGL(k_quant_pairs, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, x, bucket, k, P, Mt, K,
                       qp, sp, qt, st);
    return hipGetLastError();
}

}  // namespace moe
