/*
 * qmm_probe.h -- C ABI of libqmm_probe.so, a measurement tool built beside
 * the product library (libqmm.so) and not part of it.
 *
 * qmm_read_probe: a plain streaming read of `bytes` (a multiple of 16; buf
 * 16-byte aligned, device memory) over `workgroups` workgroups of 256
 * threads, each lane keeping `loads_per_lane` (1, 2, 4 or 8) independent
 * 16-byte loads in flight.  Every 16-byte chunk is read exactly once:
 * workgroup w reads blocks w, w + workgroups, ... of 256 * loads_per_lane
 * chunks and writes the XOR of its chunks' four int32 words to sink[w]
 * (device int32 [workgroups]), so the loads are not removed.  It computes
 * nothing else: it measures the time the memory system takes to deliver a
 * buffer of that size, the floor a bandwidth-bound call is compared
 * against, and gives a read of known size to calibrate traffic counters.
 * Returns 0, 1 for an invalid argument (nothing is enqueued) or 4 when the
 * launch failed.  Asynchronous on `stream` (a hipStream_t, NULL = default).
 */
#ifndef QMM_PROBE_H
#define QMM_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int qmm_read_probe(const void *buf, size_t bytes, int32_t *sink, int64_t workgroups, int loads_per_lane,
                   void *stream);

#ifdef __cplusplus
}
#endif
#endif /* QMM_PROBE_H */
