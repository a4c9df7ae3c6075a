// esdg_api.hip -- C ABI of libesdg: argument checks, launch configuration per
// polynomial order, and the fp64 / fp32 entry points declared in esdg.h.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "esdg.h"
#include "volume_kernel.hpp"

namespace esdg {
namespace {

constexpr int kMinOrder = 1;
constexpr int kMaxOrder = 8;

// Launch shape per precision and order: EPB elements x NT threads per
// workgroup (the 3 (N+1)^2 line tasks of EPB elements fill whole waves as far
// as possible), whether the metric terms are staged in LDS, and whether the
// pair loop carries its series-only second form (volume term / with the
// surface term).  Chosen by timing on MI355X at the bubble, baroclinic and
// N=4 L=6 mesh sizes; the series form where it measured faster at the
// 4096- and 32,768-element sizes (it adds registers: at N <= 2 it gains
// nothing, and the fp64 N = 8 kernel would spill).
//
// At N = 3 and N = 7 (N+1 a power of two) the unpadded LDS node grid puts
// the lanes of a direction-1 or direction-2 line read on a few banks (up to
// 16 lanes per bank at N = 7); one pad value per row (N = 7) or three per
// plane (N = 3; fp32 with four per element and direction-major lines) spread
// them.  Waves whose lanes hold lines of two directions conflict too: at
// fp64 N = 6 and at N = 2 the 49 or 63 lines of each direction start on a
// 64-lane boundary (order 2), at the same 192 threads.  Other pads and orders were neutral
// to slower.  At fp64 N = 5 a 3-wave register cap on the volume kernel (168
// registers, a 36-byte spill) lets three workgroups share a CU instead of
// two; at fp32 N = 4 and 5 a 5-wave cap on the kernel with the surface term
// (96 and 89 registers) does the same for five workgroups instead of four,
// and at fp32 N = 7 and 8 direction-3 lines that finish their nodes (25 and
// 32 KB of LDS) with 4-wave caps (128 registers) give five and four
// workgroups per CU instead of four and three.
template <typename T, int N> struct Launch;
// LaunchCfg<EPB, NT, waves hint, metric staged in LDS, line cached in
// registers, line order (0 element-major, 1 direction-major, 2 direction-major
// with each direction on a 32-lane boundary), direction-3 lines finish the
// nodes, series form (volume term), series form (with the surface term), LDS
// pad per row, per plane, per element, waves hint with the surface term>
template <> struct Launch<double, 1> { using C = LaunchCfg<16, 192>; };                       // 192/192 lines
template <> struct Launch<double, 2> { using C = LaunchCfg<7, 192, 0, true, false, 2>; };     // 189/192
template <> struct Launch<double, 3> { using C = LaunchCfg<4, 192, 0, false, false, false, false, true, false, 0, 3>; };          // 192/192
template <> struct Launch<double, 4> { using C = LaunchCfg<3, 256, 0, false, false, true, false, true>; };           // 225/256
template <> struct Launch<double, 5> { using C = LaunchCfg<2, 256, 3, false, false, true, false, true, true>; };    // 216/256
template <> struct Launch<double, 6> { using C = LaunchCfg<1, 192, 0, true, false, 2, false, true>; };          // 147/192
template <> struct Launch<double, 7> { using C = LaunchCfg<1, 192, 0, false, false, true, true, true, true, 1>; };      // 192/192
template <> struct Launch<double, 8> { using C = LaunchCfg<1, 256, 0, false, false, true, true>; };                 // 243/256
template <> struct Launch<float, 1> { using C = LaunchCfg<16, 192>; };
template <> struct Launch<float, 2> { using C = LaunchCfg<7, 192, 0, true, false, 2>; };
template <> struct Launch<float, 3> { using C = LaunchCfg<4, 192, 0, true, false, 1, false, true, true, 0, 3, 4>; };
template <> struct Launch<float, 4> { using C = LaunchCfg<3, 256, 0, false, false, true, false, true, true, 0, 0, 0, 5>; };
template <> struct Launch<float, 5> { using C = LaunchCfg<2, 256, 0, false, false, true, false, true, false, 0, 0, 0, 5>; };
template <> struct Launch<float, 6> { using C = LaunchCfg<1, 192, 0, false, false, false, false, true, true>; };
template <> struct Launch<float, 7> { using C = LaunchCfg<1, 192, 4, false, false, 1, true, true, true, 1, 0, 0, 4>; };
template <> struct Launch<float, 8> { using C = LaunchCfg<1, 256, 0, false, false, true, true, true, true, 0, 0, 0, 4>; };

template <typename T, int N, bool SURF>
int launch(const T *q, const T *phi, const T *geom, const T *D, const int32_t *nbr,
           Rotation<T> rot, int64_t nelem, T *rhs, hipStream_t stream)
{
    using C = typename Launch<T, N>::C;
    const int64_t blocks = (nelem + C::EPB - 1) / C::EPB;
    if (blocks > INT32_MAX) return ESDG_ERR_NELEM;
    hipLaunchKernelGGL((volume_rhs_kernel<T, N, C, SURF>), dim3((unsigned)blocks), dim3(C::NT),
                       0, stream, q, phi, geom, D, nbr, rot, nelem, rhs);
    return hipGetLastError() == hipSuccess ? ESDG_OK : ESDG_ERR_LAUNCH;
}

bool overlaps(const void *a, int64_t abytes, const void *b, int64_t bbytes)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

// Both entry points: SURF = false gives the volume term, SURF = true the
// volume term plus the surface term (nbr must then be given) and, with omega
// given (host pointer, 3 values read during the call), the Coriolis source.
template <typename T, bool SURF>
int evaluate(const T *q, const T *phi, const T *geom, const T *D, const int32_t *nbr,
             const T *omega, int N, int64_t nelem, T *rhs, hipStream_t stream)
{
    if (N < kMinOrder || N > kMaxOrder) return ESDG_ERR_ORDER;
    if (nelem < 0) return ESDG_ERR_NELEM;
    if (nelem == 0) return ESDG_OK;
    if (!q || !phi || !geom || !D || !rhs || (SURF && !nbr)) return ESDG_ERR_NULL;
    const int64_t Nq = N + 1, Np = Nq * Nq * Nq;
    // the largest array has 10 * nelem * Np elements of T
    if (nelem > INT64_MAX / (10 * Np * (int64_t)sizeof(T))) return ESDG_ERR_NELEM;
    const int64_t field = nelem * Np * (int64_t)sizeof(T);
    const int64_t rbytes = 5 * field;
    if (overlaps(rhs, rbytes, q, 5 * field) || overlaps(rhs, rbytes, phi, field) ||
        overlaps(rhs, rbytes, geom, 10 * field) ||
        overlaps(rhs, rbytes, D, Nq * Nq * (int64_t)sizeof(T)) ||
        (SURF && overlaps(rhs, rbytes, nbr, 6 * nelem * (int64_t)sizeof(int32_t))))
        return ESDG_ERR_ALIAS;
    Rotation<T> rot{T(0), T(0), T(0), false};
    if (SURF && omega) rot = Rotation<T>{omega[0], omega[1], omega[2], true};
    switch (N) {
        case 1: return launch<T, 1, SURF>(q, phi, geom, D, nbr, rot, nelem, rhs, stream);
        case 2: return launch<T, 2, SURF>(q, phi, geom, D, nbr, rot, nelem, rhs, stream);
        case 3: return launch<T, 3, SURF>(q, phi, geom, D, nbr, rot, nelem, rhs, stream);
        case 4: return launch<T, 4, SURF>(q, phi, geom, D, nbr, rot, nelem, rhs, stream);
        case 5: return launch<T, 5, SURF>(q, phi, geom, D, nbr, rot, nelem, rhs, stream);
        case 6: return launch<T, 6, SURF>(q, phi, geom, D, nbr, rot, nelem, rhs, stream);
        case 7: return launch<T, 7, SURF>(q, phi, geom, D, nbr, rot, nelem, rhs, stream);
        case 8: return launch<T, 8, SURF>(q, phi, geom, D, nbr, rot, nelem, rhs, stream);
    }
    return ESDG_ERR_ORDER;
}

}  // namespace
}  // namespace esdg

extern "C" {

int esdg_volume_rhs_f64(const double *q, const double *phi, const double *geom, const double *D,
                        int N, int64_t nelem, double *rhs, hipStream_t stream)
{
    return esdg::evaluate<double, false>(q, phi, geom, D, nullptr, nullptr, N, nelem, rhs, stream);
}

int esdg_volume_rhs_f32(const float *q, const float *phi, const float *geom, const float *D,
                        int N, int64_t nelem, float *rhs, hipStream_t stream)
{
    return esdg::evaluate<float, false>(q, phi, geom, D, nullptr, nullptr, N, nelem, rhs, stream);
}

int esdg_rhs_f64(const double *q, const double *phi, const double *geom, const double *D,
                 const int32_t *nbr, const double *omega, int N, int64_t nelem, double *rhs,
                 hipStream_t stream)
{
    return esdg::evaluate<double, true>(q, phi, geom, D, nbr, omega, N, nelem, rhs, stream);
}

int esdg_rhs_f32(const float *q, const float *phi, const float *geom, const float *D,
                 const int32_t *nbr, const float *omega, int N, int64_t nelem, float *rhs,
                 hipStream_t stream)
{
    return esdg::evaluate<float, true>(q, phi, geom, D, nbr, omega, N, nelem, rhs, stream);
}

const char *esdg_status_string(int status)
{
    switch (status) {
        case ESDG_OK: return "ok";
        case ESDG_ERR_NULL: return "a required pointer is NULL";
        case ESDG_ERR_ORDER: return "polynomial order N outside the compiled range";
        case ESDG_ERR_NELEM: return "nelem is negative or too large";
        case ESDG_ERR_LAUNCH: return "kernel launch failed";
        case ESDG_ERR_ALIAS: return "rhs overlaps an input array";
    }
    return "unknown status";
}

int esdg_min_order(void) { return esdg::kMinOrder; }
int esdg_max_order(void) { return esdg::kMaxOrder; }

}  // extern "C"
