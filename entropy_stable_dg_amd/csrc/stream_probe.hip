// stream_probe.hip -- HBM streaming probes (libesdg_probe.so): the
// 8-read:1-write fp64 stream that gives the empirical bandwidth roof, and a
// plain copy of known traffic for counter calibration.  Consecutive lanes
// touch consecutive doubles (each wave load covers 512 contiguous bytes); a
// grid-stride loop keeps the grid at 16 workgroups per CU.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "esdg_probe.h"
#include "volume_kernel.hpp"
#include "launch_table.hpp"

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

// The same 8:1 stream with 32 bytes per lane per array (two 16-byte loads):
// wider requests reach a few percent more bandwidth on this part.  Lane i
// covers doubles 4i .. 4i+3 of each array; a scalar loop finishes n % 4.
__global__ void __launch_bounds__(kThreads)
stream81_wide(const double *__restrict__ src, double *__restrict__ dst, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int64_t nv = n / 4;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nv; i += stride) {
        double2 s0 = make_double2(0.0, 0.0), s1 = make_double2(0.0, 0.0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const double2 *p = reinterpret_cast<const double2 *>(src + j * n + 4 * i);
            const double2 a = p[0], b = p[1];
            s0.x += a.x; s0.y += a.y; s1.x += b.x; s1.y += b.y;
        }
        double2 *o = reinterpret_cast<double2 *>(dst + 4 * i);
        o[0] = s0;
        o[1] = s1;
    }
    for (int64_t i = 4 * nv + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
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

// The per-node natural log of the volume kernel, element by element (a test
// hook for its accuracy: the fp64 form is the library's own series, the fp32
// form the hardware log2 scaled by ln 2, exactly as the pairs use them).
template <typename T>
__global__ void __launch_bounds__(kThreads)
node_log(const T *__restrict__ x, T *__restrict__ y, int64_t n)
{
    using A = esdg::Arith<T>;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
        y[i] = T(A::kLogToLn) * A::node_log(x[i]);
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

// Phase timeline of the library's volume kernel (or whole right-hand side
// when nbr is given): the same kernel instance with WallMarks.
template <typename T, int N>
int64_t timeline_workgroups(int64_t nelem)
{
    using C = typename esdg::Launch<T, N>::C;
    return (nelem + C::EPB - 1) / C::EPB;
}

template <typename T>
int64_t workgroups_of(int N, int64_t nelem)
{
    switch (N) {
        case 1: return timeline_workgroups<T, 1>(nelem);
        case 2: return timeline_workgroups<T, 2>(nelem);
        case 3: return timeline_workgroups<T, 3>(nelem);
        case 4: return timeline_workgroups<T, 4>(nelem);
        case 5: return timeline_workgroups<T, 5>(nelem);
        case 6: return timeline_workgroups<T, 6>(nelem);
        case 7: return timeline_workgroups<T, 7>(nelem);
        case 8: return timeline_workgroups<T, 8>(nelem);
    }
    return -3;
}

template <typename T, int N>
int timeline_launch(const T *q, const T *phi, const T *geom, const T *D, const int32_t *nbr,
                    int64_t nelem, T *rhs, uint64_t *marks, hipStream_t stream)
{
    using C = typename esdg::Launch<T, N>::C;
    const int64_t blocks = timeline_workgroups<T, N>(nelem);
    const esdg::Rotation<T> rot{T(0), T(0), T(0), false};
    const esdg::Sink<T, false> sink{rhs, nullptr, T(0), T(0), T(0)};
    const esdg::WallMarks wm{(unsigned long long *)marks};
    if (nbr)
        hipLaunchKernelGGL((esdg::volume_rhs_kernel<T, N, C, true, false, false, esdg::WallMarks>),
                           dim3((unsigned)blocks), dim3(C::NT), 0, stream, q, (const T *)nullptr,
                           phi, geom, D, nbr, rot, nelem, sink, wm);
    else
        hipLaunchKernelGGL((esdg::volume_rhs_kernel<T, N, C, false, false, false, esdg::WallMarks>),
                           dim3((unsigned)blocks), dim3(C::NT), 0, stream, q, (const T *)nullptr,
                           phi, geom, D, (const int32_t *)nullptr, rot, nelem, sink, wm);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

template <typename T>
int timeline(const T *q, const T *phi, const T *geom, const T *D, const int32_t *nbr, int N,
             int64_t nelem, T *rhs, uint64_t *marks, hipStream_t stream)
{
    if (N < 1 || N > 8 || nelem < 0) return -3;
    const int64_t Np = (int64_t)(N + 1) * (N + 1) * (N + 1);
    if (nelem > INT64_MAX / (10 * Np * (int64_t)sizeof(T)) || workgroups_of<T>(N, nelem) > INT32_MAX)
        return -3;
    if (nelem == 0) return 0;
    if (!q || !phi || !geom || !D || !rhs || !marks) return -1;
    // slot 3 of every workgroup is raised by each of its waves: start at zero
    if (hipMemsetAsync(marks, 0, (size_t)workgroups_of<T>(N, nelem) * esdg::kMarkValues * 8,
                       stream) != hipSuccess)
        return -4;
    switch (N) {
        case 1: return timeline_launch<T, 1>(q, phi, geom, D, nbr, nelem, rhs, marks, stream);
        case 2: return timeline_launch<T, 2>(q, phi, geom, D, nbr, nelem, rhs, marks, stream);
        case 3: return timeline_launch<T, 3>(q, phi, geom, D, nbr, nelem, rhs, marks, stream);
        case 4: return timeline_launch<T, 4>(q, phi, geom, D, nbr, nelem, rhs, marks, stream);
        case 5: return timeline_launch<T, 5>(q, phi, geom, D, nbr, nelem, rhs, marks, stream);
        case 6: return timeline_launch<T, 6>(q, phi, geom, D, nbr, nelem, rhs, marks, stream);
        case 7: return timeline_launch<T, 7>(q, phi, geom, D, nbr, nelem, rhs, marks, stream);
        case 8: return timeline_launch<T, 8>(q, phi, geom, D, nbr, nelem, rhs, marks, stream);
    }
    return -3;
}

}  // namespace

extern "C" {

int64_t esdg_probe_timeline_workgroups(int N, int64_t nelem, int fp64)
{
    if (N < 1 || N > 8 || nelem < 0 || nelem > INT64_MAX / 2) return -3;
    return fp64 ? workgroups_of<double>(N, nelem) : workgroups_of<float>(N, nelem);
}

int esdg_probe_timeline_f64(const double *q, const double *phi, const double *geom,
                            const double *D, const int32_t *nbr, int N, int64_t nelem,
                            double *rhs, uint64_t *marks, hipStream_t stream)
{
    return timeline<double>(q, phi, geom, D, nbr, N, nelem, rhs, marks, stream);
}

int esdg_probe_timeline_f32(const float *q, const float *phi, const float *geom, const float *D,
                            const int32_t *nbr, int N, int64_t nelem, float *rhs,
                            uint64_t *marks, hipStream_t stream)
{
    return timeline<float>(q, phi, geom, D, nbr, N, nelem, rhs, marks, stream);
}

int esdg_probe_wall_clock_khz(void)
{
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, 0) != hipSuccess) return -4;
    return khz;
}

int esdg_probe_stream81_f64(const double *src, double *dst, int64_t n, hipStream_t stream)
{
    const int st = check(src, dst, n, 9);
    if (st || n == 0) return st;
    hipLaunchKernelGGL(stream81, dim3(grid_for(n)), dim3(kThreads), 0, stream, src, dst, n);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int esdg_probe_stream81_wide_f64(const double *src, double *dst, int64_t n, hipStream_t stream)
{
    const int st = check(src, dst, n, 9);
    if (st || n == 0) return st;
    // 16-byte loads need 16-byte aligned array starts: src, dst and n even
    if (((uintptr_t)src | (uintptr_t)dst) % 16 != 0 || n % 2 != 0) return -2;
    hipLaunchKernelGGL(stream81_wide, dim3(grid_for((n + 3) / 4)), dim3(kThreads), 0, stream, src,
                       dst, n);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int esdg_probe_node_log_f64(const double *x, double *y, int64_t n, hipStream_t stream)
{
    const int st = check(x, y, n, 2);
    if (st || n == 0) return st;
    hipLaunchKernelGGL(node_log<double>, dim3(grid_for(n)), dim3(kThreads), 0, stream, x, y, n);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int esdg_probe_node_log_f32(const float *x, float *y, int64_t n, hipStream_t stream)
{
    const int st = check(x, y, n, 1);
    if (st || n == 0) return st;
    hipLaunchKernelGGL(node_log<float>, dim3(grid_for(n)), dim3(kThreads), 0, stream, x, y, n);
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
