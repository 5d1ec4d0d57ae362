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

/* Exactness checks of the quantizer's short division sequences (the device
 * functions rcp_rn, div_rn_narrow and div_rn of the library, compiled into this
 * probe library from the same source).  Each kernel adds to counts[0] the
 * number of results that are not the correctly rounded IEEE quotient RN(a/b)
 * -- decided exactly from the fp64 residual a - b q, with no division
 * instruction -- and to counts[1] the number that differ from the compiler's
 * own IEEE division; first_bad is lowered to the smallest failing key.  The
 * caller initialises counts (two uint64) to 0 and *first_bad to 0xffffffff.
 * raw != 0 checks a deliberately short form instead (the negative control
 * that shows the checker detects wrong roundings).
 *
 * sqp_check_rcp: every float bit pattern b in [lo, hi), 0x00800000 <= lo <
 *   hi <= 0x7f800000; q = rcp_rn(b) (raw: the hardware estimate v_rcp_f32
 *   alone).  Key = the bit pattern of b.
 * sqp_check_div_narrow: all 2^30 pairs of a bf16 significand a in [1, 2) and
 *   an fp32 significand b in [1, 2), key = a_index << 23 | b_index;
 *   q = div_rn_narrow(a, b, rcp_rn(b)) (raw: RN(a * rcp_rn(b))).  Scaling a
 *   or b by a power of two scales q exactly, so this covers every exponent
 *   whose quotient stays normal.
 * sqp_check_div: `count` pairs, b = the fp32 significand in [1, 2) with index
 *   key mod 2^23, a an fp32 significand in [1, 2) hashed from (seed, key);
 *   q = div_rn(a, b, rcp_rn(b)) (raw: RN(a * rcp_rn(b))). */
int sqp_check_rcp(uint32_t lo, uint32_t hi, int raw, unsigned long long* counts,
                  uint32_t* first_bad, sqp_stream_t stream);
int sqp_check_div_narrow(int raw, unsigned long long* counts, uint32_t* first_bad,
                         sqp_stream_t stream);
int sqp_check_div(uint32_t seed, uint32_t count, int raw, unsigned long long* counts,
                  uint32_t* first_bad, sqp_stream_t stream);

/* sqp_check_codes: the quantizers' code step (chunk_codes, eight values at a
 * time: rne of the correctly rounded quotient by the step, taken from the
 * exact product with RN(1/step) unless a half-integer lies within its error
 * bound) on `count` chunks hashed from (seed, key): per chunk a step formed
 * from a maximum in [2^-30, 2^30) as the kernels form it, values (k + f) times
 * the step with f uniform or within 4 ulps of 1/2 (ties); clamp != 0 the
 * static quantizer's form (|k| up to 140, dividends limited to +-128 steps,
 * codes clamped to +-127).  counts[0] += codes that differ from those of the
 * compiler's IEEE quotient; counts[1] is unused.  raw != 0: the short form
 * without its fallback (the negative control).  Key = chunk index. */
int sqp_check_codes(uint32_t seed, uint32_t count, int clamp, int raw, unsigned long long* counts,
                    uint32_t* first_bad, sqp_stream_t stream);

/* q[i] = a[i] / b[i] with the compiler's fp32 division (n elements), so the
 * host can confirm that division is the correctly rounded one. */
int sqp_div_ref(const float* a, const float* b, float* q, int64_t n, sqp_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SQ_PROBE_H */
