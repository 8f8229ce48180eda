/*
 * da_probe.h -- measurement probes used by the benchmark beside the decode-attention
 * library (libda_probe.so, a library of its own: nothing here is part of attention).
 *
 *  - da_read_probe streams n_bytes (a positive multiple of 16) from device memory src with
 *    16-byte loads and writes at most one fp32 per workgroup (at most 4096) into the device
 *    buffer sink, so the reads cannot be elided. Its rate is the plain streaming-read rate of
 *    the chip, against which a kernel's HBM rate is also quoted.
 *  - da_copy_probe copies n_bytes (a positive multiple of 16) from device src to device dst
 *    (non-overlapping): a transfer of known size against which hardware traffic counters
 *    (FETCH_SIZE, WRITE_SIZE) are calibrated.
 * Both enqueue on `stream` (a hipStream_t; NULL = the default stream), never synchronise,
 * and return 0, -1 for a bad argument (nothing enqueued) or -4 when the launch failed.
 */
#ifndef DA_PROBE_H
#define DA_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

int da_read_probe(const void* src, size_t n_bytes, float* sink, void* stream);
int da_copy_probe(const void* src, void* dst, size_t n_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DA_PROBE_H */
