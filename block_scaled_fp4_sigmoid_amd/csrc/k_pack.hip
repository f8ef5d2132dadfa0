// k_pack.hip — rearrangement of FP4 expert weights into the order in which
// the gfx950 expert GEMMs load them (done once, when the weights are loaded).
//
// Pages: SGLang Spark GB10 Optimizations, section 1 (NVFP4 weights with FP8
// scale rows, one scale per 16 values along K); SGLang-NVIDIA-Mega README,
// DeepSeek-V4.1 slot table, row "Routed experts (moe)" (block-scaled expert
// GEMMs; the weight order inside a matrix is the kernel's business).  The
// values are unchanged: only their places move.
//
// Standard layout (input): w [E][N][K/2] (two E2M1 per byte, low nibble =
// lower K), MX scales [E][N][K/32], NV scales [E][N][K/16].
// Packed layout (output); S = K/128 steps, Q = ceil(S/4) quads, rb = 16-row
// block, lane l = 16g + i (the MFMA operand lane of row 16rb + i, K group g):
//   w   [E][N/16][S][64 lanes][16 B]: lane l's bytes of step s are the row's
//       bytes [64s + 16g, +16)  (one 1 KB load per block and step);
//   MX  [E][N/16][Q][64 lanes][4 B]: byte u = E8M0 of K block 4(4q+u) + g;
//   NV  [E][N/16][Q][64 lanes][8 B]: bytes 2u, 2u+1 = E4M3 of K blocks
//       8(4q+u) + 2g and + 1;
// scale entries of steps past S are zero.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

// One thread per 16 output weight bytes.
__global__ __launch_bounds__(256) void k_pack_w(const uint8_t* __restrict__ w, int E, int N, int K,
                                                uint8_t* __restrict__ out) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    const int S = K / 128;
    const long total = (long)E * (N / 16) * S * 64;
    if (idx >= total) return;
    const int l = (int)(idx % 64);
    const long r1 = idx / 64;
    const int s = (int)(r1 % S);
    const long blk = r1 / S;  // e * (N/16) + rb
    const int i = l & 15, g = l >> 4;
    const long row = blk * 16 + i;  // e * N + 16 rb + i
    *reinterpret_cast<v4i*>(out + idx * 16) = load16(w + row * (K / 2) + 64 * s + 16 * g);
}

// One thread per lane entry of a quad: 4 (MX) or 8 (NV) output scale bytes.
template <int NV>
__global__ __launch_bounds__(256) void k_pack_s(const uint8_t* __restrict__ sc, int E, int N, int K,
                                                uint8_t* __restrict__ out) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    const int S = K / 128, Q = (S + 3) / 4;
    const long total = (long)E * (N / 16) * Q * 64;
    if (idx >= total) return;
    const int l = (int)(idx % 64);
    const long r1 = idx / 64;
    const int q = (int)(r1 % Q);
    const long blk = r1 / Q;
    const int i = l & 15, g = l >> 4;
    const long row = blk * 16 + i;
    if (!NV) {
        const uint8_t* src = sc + row * (K / 32);
        uint32_t v = 0;
        for (int u = 0; u < 4; ++u)
            if (4 * q + u < S) v |= (uint32_t)src[4 * (4 * q + u) + g] << (8 * u);
        *reinterpret_cast<uint32_t*>(out + idx * 4) = v;
    } else {
        const uint8_t* src = sc + row * (K / 16);
        uint32_t v[2] = {0, 0};
        for (int u = 0; u < 4; ++u)
            if (4 * q + u < S)
                for (int h = 0; h < 2; ++h)
                    v[u >> 1] |= (uint32_t)src[8 * (4 * q + u) + 2 * g + h] << (16 * (u & 1) + 8 * h);
        *reinterpret_cast<uint32_t*>(out + idx * 8) = v[0];
        *reinterpret_cast<uint32_t*>(out + idx * 8 + 4) = v[1];
    }
}

}  // namespace

size_t packed_scale_bytes(int fmt, int E, int N, int K) {
    const int S = K / 128, Q = (S + 3) / 4;
    return (size_t)E * (N / 16) * Q * 64 * (fmt == MOE_FMT_NVFP4 ? 8 : 4);
}

hipError_t launch_pack_fp4(int fmt, int E, int N, int K, const uint8_t* w, const uint8_t* sc, uint8_t* w_out,
                           uint8_t* sc_out, hipStream_t stream) {
    const long nw = (long)E * (N / 16) * (K / 128) * 64;
    hipLaunchKernelGGL(k_pack_w, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, stream, w, E, N, K, w_out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long ns = (long)E * (N / 16) * ((K / 128 + 3) / 4) * 64;
    if (fmt == MOE_FMT_NVFP4)
        hipLaunchKernelGGL(k_pack_s<1>, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, stream, sc, E, N, K, sc_out);
    else
        hipLaunchKernelGGL(k_pack_s<0>, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, stream, sc, E, N, K, sc_out);
    return hipGetLastError();
}

}  // namespace moe
