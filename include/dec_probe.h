/* Measured ceilings for the roofline figures (libdec_probe.so).
 *
 * Measurement aids beside the forward library: what one GPU sustains for a
 * streaming read of device memory, a device-to-device copy, and back-to-back
 * bf16 MFMAs with no memory traffic.  The published peaks (8 TB/s HBM, 2.5
 * PFLOP/s dense bf16) stay the roofline denominators; these give the measured
 * ceilings beside them.  Nothing on the forward path calls them.
 *
 * Every call launches its kernel once untimed, then `reps` times between two
 * HIP events on `stream` (a hipStream_t; null is the default stream), waits
 * for the second event and writes the mean milliseconds per launch to *ms.
 * Pointers are device pointers the caller owns; nothing is allocated.
 * Returns 0, -2 for an invalid argument (nothing launched), -1 for a HIP
 * error.
 */
#ifndef DEC_PROBE_H
#define DEC_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DECP_RUN_BYTES 16384   /* the read and copy probes' unit: one block of 256 threads each */
#define DECP_GRID_BLOCKS 2048  /* blocks of 256 threads of the MFMA probe */

/* Reads every 16-byte word of buf[0, bytes) once (non-temporal loads), one
 * block of 256 threads per DECP_RUN_BYTES run, and stores the XOR of run b's
 * 32-bit words into sink[b] (bytes / DECP_RUN_BYTES 32-bit words).  bytes: a
 * positive multiple of DECP_RUN_BYTES; buf 16-byte aligned.  Read rate =
 * bytes / *ms. */
int decp_stream_read(const void *buf, size_t bytes, void *sink, int reps, void *stream, double *ms);

/* dst[0, bytes) = src[0, bytes) in 16-byte words, one block per
 * DECP_RUN_BYTES run (the ranges must not overlap; both 16-byte aligned;
 * bytes a positive multiple of DECP_RUN_BYTES).  Traffic = 2 x bytes / *ms. */
int decp_copy(const void *src, void *dst, size_t bytes, int reps, void *stream, double *ms);

/* Floats the MFMA probe's `sink` must hold: one per thread. */
int decp_mfma_sink_floats(void);

/* Every wave of DECP_GRID_BLOCKS x 4 issues iters x 4 independent
 * 32x32x16 bf16 MFMAs (no loads); *flops = the launch's flops (2 a
 * multiply-add), so the rate is *flops / *ms; sink holds one float a thread. */
int decp_mfma_bf16(int iters, void *sink, int reps, void *stream, double *ms, double *flops);

#ifdef __cplusplus
}
#endif

#endif
