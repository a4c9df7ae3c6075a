// stream_probe.hip -- HBM streaming probes (libesdg_probe.so): the
// 8-read:1-write fp64 stream that gives the empirical bandwidth roof, and a
// plain copy of known traffic for counter calibration.  Consecutive lanes
// touch consecutive doubles (each wave load covers 512 contiguous bytes); a
// grid-stride loop keeps the grid at 16 workgroups per CU.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "esdg_probe.h"

namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads)
stream81(const double *__restrict__ src, double *__restrict__ dst, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
        double s = 0.0;
#pragma unroll
        for (int j = 0; j < 8; ++j) s += src[j * n + i];
        dst[i] = s;
    }
}

__global__ void __launch_bounds__(kThreads)
copy(const double *__restrict__ src, double *__restrict__ dst, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

unsigned grid_for(int64_t n)
{
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int64_t want = (n + kThreads - 1) / kThreads;
    const int64_t cap = (int64_t)cus * 16;
    const int64_t g = want < cap ? want : cap;
    return (unsigned)(g > 0 ? g : 1);
}

int check(const void *src, const void *dst, int64_t n, int64_t arrays)
{
    if (n < 0 || n > INT64_MAX / (8 * arrays)) return -3;
    if (n > 0 && (!src || !dst)) return -1;
    return 0;
}

}  // namespace

extern "C" {

int esdg_probe_stream81_f64(const double *src, double *dst, int64_t n, hipStream_t stream)
{
    const int st = check(src, dst, n, 9);
    if (st || n == 0) return st;
    hipLaunchKernelGGL(stream81, dim3(grid_for(n)), dim3(kThreads), 0, stream, src, dst, n);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int esdg_probe_copy_f64(const double *src, double *dst, int64_t n, hipStream_t stream)
{
    const int st = check(src, dst, n, 2);
    if (st || n == 0) return st;
    hipLaunchKernelGGL(copy, dim3(grid_for(n)), dim3(kThreads), 0, stream, src, dst, n);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
