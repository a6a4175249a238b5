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
 * tq_probe_pattern: the byte pattern of the fp8 decode stream with no
 *   arithmetic, as a ceiling for kernels that move those bytes that way.
 *   num_workgroups workgroups of 8 waves; wave w reads chunks_per_wave chunks,
 *   each 4096 bytes of k (into registers) and 4096 bytes of v plus 256 bytes of
 *   scales (into LDS by LDS-direct loads), from k/v + (w * chunks_per_wave + c)
 *   * 4096 and scales + (w * chunks_per_wave + c) * 256, one chunk in flight
 *   ahead, and writes one digest per workgroup to sink.  kv_bytes and
 *   scale_bytes are the buffer sizes (checked); all 16-byte aligned.
 * tq_probe_pattern4: the same for the 4-bit format's stream: wave w reads
 *   chunks_per_wave chunks, each 4096 bytes of rows from rows + (w *
 *   chunks_per_wave + c) * 4096 (four 1 KiB LDS-direct loads) and 192 bytes of
 *   metadata from meta + (w * chunks_per_wave + c) * 256, into LDS, one chunk
 *   in flight ahead; rows_bytes and meta_bytes are the buffer sizes (checked);
 *   16-byte aligned.
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
int32_t tq_probe_pattern(const void* k, const void* v, const void* scales, size_t kv_bytes,
                         size_t scale_bytes, int32_t chunks_per_wave, int32_t num_workgroups,
                         uint32_t* sink, void* stream);
int32_t tq_probe_pattern4(const void* rows, const void* meta, size_t rows_bytes, size_t meta_bytes,
                          int32_t chunks_per_wave, int32_t num_workgroups, uint32_t* sink,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_PROBE_H */
