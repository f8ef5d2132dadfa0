// k_probe.hip — streaming-read calibration for the measurements (gfx950).
//
// One launch reads a device buffer once in the access pattern of the weight
// streaming GEMMs: the buffer is rows of row_bytes; a wave owns 16 rows and
// lane (i, g) reads 16 bytes of row i at 64 s + 16 g for steps s, eight steps
// in flight.  The XOR of everything read keeps the loads live; it is stored
// only if it equals a fixed constant (the sink is written at most once).  The
// rate reached is the practical HBM read rate the weight-streaming kernels
// are compared against, beside the published peak.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 8;

typedef int v4i_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void k_stream_read(const uint8_t* __restrict__ buf, size_t rows, int row_bytes,
                                                           uint32_t* __restrict__ sink) {
    const size_t wave = (size_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
    const size_t row = wave * 16 + i;
    if (wave * 16 >= rows) return;
    const bool live = row < rows;  // the last wave may hold fewer than 16 rows
    const uint8_t* rp = buf + (live ? row : 0) * (size_t)row_bytes + 16 * g;
    const int steps = row_bytes / 64;
    v4i_t acc = {0, 0, 0, 0};
    int s = 0;
    for (; s + kInFlight <= steps; s += kInFlight) {
        v4i_t v[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) v[u] = *reinterpret_cast<const v4i_t*>(rp + 64 * (s + u));
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) acc ^= v[u];
    }
    for (; s < steps; ++s) acc ^= *reinterpret_cast<const v4i_t*>(rp + 64 * s);
    const uint32_t x = (uint32_t)(acc.x ^ acc.y ^ acc.z ^ acc.w);
    if (live && x == 0x9E3779B9u) sink[0] = x;
}

}  // namespace

extern "C" {

int moe_probe_stream_read(const void* buf, size_t bytes, int row_bytes, uint32_t* sink, hipStream_t stream) {
    if (!buf || !sink || bytes == 0 || row_bytes < 64 || row_bytes % 64 != 0) return 1;
    if (bytes % (size_t)row_bytes != 0 || (uintptr_t)buf % 16 != 0) return 1;
    const size_t rows = bytes / (size_t)row_bytes;
    const size_t waves = (rows + 15) / 16;
    const size_t blocks = (waves + kThreads / 64 - 1) / (kThreads / 64);
    if (blocks > 0x7fffffffu) return 1;
    hipLaunchKernelGGL(k_stream_read, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       static_cast<const uint8_t*>(buf), rows, row_bytes, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
