/*
 * esdg_probe.h -- C ABI of libesdg_probe.so: HBM streaming probes used to
 * measure the bandwidth roof on the device the volume kernel runs on.  Not
 * part of the volume-term path; the benchmark and the profiling runs use it.
 *
 * The node-log entries expose the volume kernel's per-node logarithm for
 * accuracy tests; the timeline entries run the volume kernel with phase
 * marks (when each workgroup loads, computes and stores).
 *
 * The 8-read:1-write fp64 stream is the empirical streaming roofline of
 * "hipBone: A performance-portable GPU-accelerated C++ version of the
 * NekBone benchmark" (its bandwidth section: a kernel reading eight arrays
 * and writing one, timed on resident data); the plain copy is the reference
 * kernel of known traffic used to calibrate the FETCH_SIZE / WRITE_SIZE
 * hardware counters.
 *
 * All pointers are device pointers owned by the caller; calls are
 * asynchronous on `stream`, allocate nothing and return a status:
 * 0 ok, -1 NULL pointer (n > 0), -2 misaligned (wide form only), -3 n < 0
 * or too large, -4 launch failure.
 * n == 0 is a no-op.
 */
#ifndef ESDG_PROBE_H
#define ESDG_PROBE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dst[i] = sum_{j<8} src[j*n + i], i < n: reads 64 n bytes, writes 8 n bytes. */
int esdg_probe_stream81_f64(const double *src, double *dst, int64_t n, hipStream_t stream);

/* The same stream with 32 bytes per lane per array (16-byte loads); src and
 * dst 16-byte aligned and n even, else -2. */
int esdg_probe_stream81_wide_f64(const double *src, double *dst, int64_t n, hipStream_t stream);

/* y[i] = natural log of x[i] as the volume kernel computes its per-node logs
 * (fp64: the library's own series; fp32: hardware log2 times ln 2), i < n.
 * A test hook for the accuracy of that log; x must be positive and normal. */
int esdg_probe_node_log_f64(const double *x, double *y, int64_t n, hipStream_t stream);
int esdg_probe_node_log_f32(const float *x, float *y, int64_t n, hipStream_t stream);

/* dst[i] = src[i], i < n: reads and writes 8 n bytes. */
int esdg_probe_copy_f64(const double *src, double *dst, int64_t n, hipStream_t stream);

/* Phase timeline of the library's volume kernel ([ESDG-GPU §3, Eq. 2], the
 * volume term, as esdg_volume_rhs_* computes it; nbr == NULL) or of its whole
 * right-hand side (nbr given, as esdg_rhs_* without Coriolis): the same
 * kernel, launch shape and result, with lane 0 of every workgroup writing
 * marks[w * 6 + i] (uint64) for workgroup w: the device wall clock on entry
 * (i = 0), once its nodes are staged in LDS (1), once its line pairs are
 * done (2) and once its last wave has issued its stores (3, the latest of
 * its waves' clocks; no barrier is added for it); the hardware id of its
 * compute unit (4) and the batch of elements it took (5).  The call clears
 * marks on the stream before the launch.  Arguments and layouts as
 * for esdg_volume_rhs_* / esdg_rhs_*; marks holds at least
 * 6 * esdg_probe_timeline_workgroups(N, nelem, fp64) values.  Inputs are
 * not checked for aliasing.  Returns 0, -1 NULL pointer, -3 N outside 1..8
 * or nelem out of range, -4 launch failure; nelem == 0 is a no-op. */
int64_t esdg_probe_timeline_workgroups(int N, int64_t nelem, int fp64);
int esdg_probe_timeline_f64(const double *q, const double *phi, const double *geom,
                            const double *D, const int32_t *nbr, int N, int64_t nelem,
                            double *rhs, uint64_t *marks, hipStream_t stream);
int esdg_probe_timeline_f32(const float *q, const float *phi, const float *geom, const float *D,
                            const int32_t *nbr, int N, int64_t nelem, float *rhs,
                            uint64_t *marks, hipStream_t stream);

/* Frequency of the device wall clock the timeline reads, in kHz (< 0 on error). */
int esdg_probe_wall_clock_khz(void);

#ifdef __cplusplus
}
#endif
#endif /* ESDG_PROBE_H */
