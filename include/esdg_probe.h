/*
 * esdg_probe.h -- C ABI of libesdg_probe.so: HBM streaming probes used to
 * measure the bandwidth roof on the device the volume kernel runs on.  Not
 * part of the volume-term path; the benchmark and the profiling runs use it.
 *
 * The node-log entries expose the volume kernel's per-node logarithm for
 * accuracy tests.
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

#ifdef __cplusplus
}
#endif
#endif /* ESDG_PROBE_H */
