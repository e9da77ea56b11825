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
 * stream_read: reads every byte of p once with 128-bit loads and XORs the
 * 32-bit words each workgroup read into its own word of sink, so the reads
 * cannot be elided and no two workgroups touch one address.  Up to 32 MB
 * every thread reads one 16-byte chunk (all loads in flight at once, up to
 * 8192 workgroups); a larger buffer is read in a grid-stride pass by at most
 * 1024 workgroups.  Timed over a buffer much larger than the caches it gives
 * the streaming-read ceiling, over a smaller one the time a plain read of
 * that many bytes takes.  The XOR of the 8192 sink words is the XOR of every
 * word of p.
 *   p       device, 16-byte aligned (QMV_ERR_ALIGNMENT), bytes > 0 and a
 *           multiple of 16 (QMV_ERR_INVALID_ARG)
 *   sink    device uint32 [8192], 4-byte aligned; XORed into, not cleared:
 *           the caller zeroes it to read the checksum.  Concurrent calls on
 *           one sink race.
 *   stream  hipStream_t; the call only enqueues.
 * Returns QMV_OK or an error status of qmv.h.
 */
int qmv_stream_read(const void *p, int64_t bytes, uint32_t *sink, void *stream);

/*
 * gemm_4bit_plan: host-side introspection of qmv_gemm_4bit with 16-bit
 * activations, computed by the same code that picks the kernel and maps
 * workgroups to tiles at launch.  No device is touched.
 *   M, N, K, blocksize  as for qmv_gemm_4bit (same argument checks)
 *   tiles   host [4 * cap] int64 out: for workgroup w, the rectangle of C it
 *           writes, {row0, col0, rows, cols} (it reads the same rows of A
 *           and the same rows of the weight); NULL with cap = 0 to count
 *   kernel  host out: 0 narrow (M <= 16), 1 split-K (M <= 64), 2 tile,
 *           3 large-M (128 x 256 tiles, weights decoded in registers)
 * Returns the number of workgroups (>= 0), or a negative qmv.h status.
 */
int64_t qmv_gemm_4bit_plan(int64_t M, int64_t N, int64_t K, int32_t blocksize, int64_t *tiles,
                           int64_t cap, int32_t *kernel);

#ifdef __cplusplus
}
#endif
#endif /* QMV_PROBE_H */
