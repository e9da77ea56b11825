/*
 * qmv_probe.h -- measurement probes exported by libqmv.so.  Not steps of the
 * method: they give the hardware ceilings that the bandwidth-bound kernels of
 * qmv.h are read against (the quest page "PyTorch MPS", section "Where It Is
 * Fast: Big Ops", reads its matvec against the streaming bandwidth it
 * measured on the same machine).
 */
#ifndef QMV_PROBE_H
#define QMV_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * stream_read: reads every byte of p once with 128-bit loads (a grid-stride
 * pass over the whole buffer) and XORs all of its 32-bit words into *sink, so
 * the reads cannot be elided; timed over a buffer much larger than the
 * caches it gives the streaming-read ceiling.
 *   p       device, 16-byte aligned (QMV_ERR_ALIGNMENT), bytes > 0 and a
 *           multiple of 16 (QMV_ERR_INVALID_ARG)
 *   sink    device uint32, 4-byte aligned; XORed into, not cleared: the
 *           caller zeroes it to read the checksum.  Concurrent calls on one
 *           sink race.
 *   stream  hipStream_t; the call only enqueues.
 * Returns QMV_OK or an error status of qmv.h.
 */
int qmv_stream_read(const void *p, int64_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* QMV_PROBE_H */
