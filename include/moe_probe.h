/* moe_probe.h — measurement helper library (libmoe_probe_mi355.so), separate
 * from the MoE layer's ABI: it calibrates what the weight-streaming kernels
 * are compared against.  Not part of the layer.
 *
 * The weight-streaming kernels are HBM-bound; their bandwidth is reported as
 * a fraction of the published HBM peak and of the read rate this probe
 * reaches on the same device in the same run. */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* moe_probe_stream_read — read `bytes` bytes of device memory at `buf` once,
 * asynchronously on `stream`, in the access pattern of the weight-streaming
 * GEMMs: the buffer is bytes / row_bytes rows; each wave of 64 lanes owns 16
 * rows and reads 64 bytes of each per step (16 per lane), eight steps in
 * flight.  sink: one uint32 of device memory (caller-owned), written only if
 * the XOR of the data equals a fixed constant (its value carries no meaning).
 * buf must be 16-byte aligned; row_bytes a positive multiple of 64; bytes a
 * non-zero multiple of row_bytes.  Returns 0 on success, 1 for invalid
 * arguments (nothing enqueued), 2 if the launch failed. */
int moe_probe_stream_read(const void *buf, size_t bytes, int row_bytes, uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif
