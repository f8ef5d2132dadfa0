// k_dense_bf16.hip — the bf16 shared expert (dense over all M rows) on gfx950
// matrix cores: gate_up + SwiGLU (bf16 h) and down.
//
// Pages: sgl-nvidia-mega PR #24, "Modifications / Target spec" (NVFP4 routed
// experts beside a BF16 shared expert); SGLang-NVIDIA-Mega README,
// DeepSeek-V4.1 slot table, rows "hop_b" / "two_shot" (the shared expert's
// output is added in the finalize).
//
// Operand layout (checked on the hardware): v_mfma_f32_16x16x32_bf16, lane
// (i, g) holds K [8g, 8g+8) of row/column i; output lane l holds
// D[4(l/16)+r][l%16], r = 0..3.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

struct JobDev {
    const uint8_t* w;
    int N_out, K;
    int M;
};

static JobDev to_dev(const ExpertJob& j) {
    JobDev d;
    d.w = static_cast<const uint8_t*>(j.w.w);
    d.N_out = j.N_out;
    d.K = j.K;
    d.M = j.M;
    return d;
}

constexpr int kPass = 64;  // rows per pass: 4 N-blocks of 16

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
