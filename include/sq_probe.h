/* sq_probe.h -- attainable-ceiling probes (libsqprobe.so).
 *
 * Measurement helpers for the benchmark's roofline report; they are not part
 * of the SmoothQuant path and libsq.so does not depend on them.  The published
 * peaks (int8 MFMA 5.0 POP/s, HBM3E 8 TB/s) are what the roofline fractions
 * are quoted against; these probes report what this machine attains for the
 * same operations, so a kernel's distance from the attainable value can be
 * told apart from the distance between the attainable value and the spec.
 *
 * All pointers are device pointers owned by the caller; every call enqueues
 * on `stream` (0 = null stream) and returns immediately.  Return value:
 * 0 = launched, 1 = invalid argument (nothing launched), 2 = HIP launch error.
 */
#ifndef SQ_PROBE_H
#define SQ_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* sqp_stream_t;

/* int8 MFMA loop: `blocks` workgroups of 256 threads; every thread loads 16
 * 16-byte operand vectors from `src` (size blocks * 256 * 256 bytes, 16-byte
 * aligned) and issues `iters` (a multiple of 8) x 4 v_mfma_i32_32x32x32_i8.
 * Work = blocks * 4 waves * iters * 4 * 2 * 32^3 int8 operations.  `out`
 * receives one int per thread (blocks * 256 ints) so nothing is elided. */
int sqp_mfma_i8(const void* src, int blocks, int iters, int* out, sqp_stream_t stream);

/* Streaming read of `bytes` (a multiple of 16) from the 16-byte aligned
 * `src`, grid-stride with `blocks` workgroups of 256 threads; `out` receives
 * blocks * 256 ints. */
int sqp_read(const void* src, int64_t bytes, int blocks, int* out, sqp_stream_t stream);

/* Plain copy of `bytes` (a multiple of 16) from `src` to `dst` (16-byte
 * aligned, not overlapping), grid-stride with `blocks` workgroups of 256
 * threads.  A profiled run uses it as the reference of known size that
 * scales the hardware's fetched / written byte counters. */
int sqp_copy(const void* src, void* dst, int64_t bytes, int blocks, sqp_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SQ_PROBE_H */
