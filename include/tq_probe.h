/*
 * tq_probe.h -- C ABI of libtqprobe.so: HBM streaming probes used to measure
 * what the memory system delivers on this GPU, next to the decode kernels.
 * Not part of the decode computation.  All pointers are DEVICE pointers owned
 * by the caller; calls are asynchronous on `stream` (a hipStream_t, NULL =
 * null stream) and return 0 on success or the hipError_t of a failed launch.
 *
 * tq_probe_read: reads every 16-byte word of src[0, n_bytes) once (n_bytes a
 *   multiple of 16, src 16-byte aligned) and writes one XOR digest per
 *   workgroup to sink[0, num_workgroups) (uint32), so the reads cannot be
 *   elided.  num_workgroups <= 65536.
 * tq_probe_copy: dst[i] = src[i] for the 16-byte words of [0, n_bytes):
 *   a plain copy of known size, for scaling hardware byte counters.
 */
#ifndef TQ_PROBE_H
#define TQ_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int32_t tq_probe_read(const void* src, size_t n_bytes, uint32_t* sink, int32_t num_workgroups,
                      void* stream);
int32_t tq_probe_copy(void* dst, const void* src, size_t n_bytes, int32_t num_workgroups,
                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_PROBE_H */
