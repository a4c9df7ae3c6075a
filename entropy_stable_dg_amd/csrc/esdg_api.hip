// esdg_api.hip -- C ABI of libesdg: argument checks, the launch per
// polynomial order (shapes in launch_table.hpp), and the fp64 / fp32 entry
// points declared in esdg.h.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <mutex>

#include "esdg.h"
#include "volume_kernel.hpp"
#include "launch_table.hpp"
#include "integrals_kernel.hpp"

namespace esdg {
namespace {

constexpr int kMinOrder = 1;
constexpr int kMaxOrder = 8;

template <typename T, int N, bool SURF, bool STAGE, bool PERT>
int launch(const T *q, const T *ref, const T *phi, const T *geom, const T *D, const int32_t *nbr,
           Rotation<T> rot, int64_t nelem, Sink<T, STAGE> sink, hipStream_t stream)
{
    using C = typename Launch<T, N>::C;
    const int64_t blocks = (nelem + C::EPB - 1) / C::EPB;
    if (blocks > INT32_MAX) return ESDG_ERR_NELEM;
    hipLaunchKernelGGL((volume_rhs_kernel<T, N, C, SURF, STAGE, PERT>), dim3((unsigned)blocks),
                       dim3(C::NT), 0, stream, q, ref, phi, geom, D, nbr, rot, nelem, sink);
    return hipGetLastError() == hipSuccess ? ESDG_OK : ESDG_ERR_LAUNCH;
}

template <typename T, bool SURF, bool STAGE, bool PERT>
int launch_order(int N, const T *q, const T *ref, const T *phi, const T *geom, const T *D,
                 const int32_t *nbr, Rotation<T> rot, int64_t nelem, Sink<T, STAGE> sink,
                 hipStream_t stream)
{
    switch (N) {
        case 1: return launch<T, 1, SURF, STAGE, PERT>(q, ref, phi, geom, D, nbr, rot, nelem, sink, stream);
        case 2: return launch<T, 2, SURF, STAGE, PERT>(q, ref, phi, geom, D, nbr, rot, nelem, sink, stream);
        case 3: return launch<T, 3, SURF, STAGE, PERT>(q, ref, phi, geom, D, nbr, rot, nelem, sink, stream);
        case 4: return launch<T, 4, SURF, STAGE, PERT>(q, ref, phi, geom, D, nbr, rot, nelem, sink, stream);
        case 5: return launch<T, 5, SURF, STAGE, PERT>(q, ref, phi, geom, D, nbr, rot, nelem, sink, stream);
        case 6: return launch<T, 6, SURF, STAGE, PERT>(q, ref, phi, geom, D, nbr, rot, nelem, sink, stream);
        case 7: return launch<T, 7, SURF, STAGE, PERT>(q, ref, phi, geom, D, nbr, rot, nelem, sink, stream);
        case 8: return launch<T, 8, SURF, STAGE, PERT>(q, ref, phi, geom, D, nbr, rot, nelem, sink, stream);
    }
    return ESDG_ERR_ORDER;
}

bool overlaps(const void *a, int64_t abytes, const void *b, int64_t bbytes)
{
    if (!a || !b) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

// Sizes shared by the entry points.  N and nelem are checked first; `field`
// is the bytes of one [nelem][Np] field.
struct Sizes {
    int64_t Nq, Np, field, nelem;
};

template <typename T>
int check_sizes(int N, int64_t nelem, Sizes &z)
{
    if (N < kMinOrder || N > kMaxOrder) return ESDG_ERR_ORDER;
    if (nelem < 0) return ESDG_ERR_NELEM;
    z.Nq = N + 1;
    z.Np = z.Nq * z.Nq * z.Nq;
    // the largest array has 10 * nelem * Np elements of T
    if (nelem > INT64_MAX / (10 * z.Np * (int64_t)sizeof(T))) return ESDG_ERR_NELEM;
    z.field = nelem * z.Np * (int64_t)sizeof(T);
    z.nelem = nelem;
    return ESDG_OK;
}

// True when the output range [out, out + obytes) overlaps one of the inputs
// (q: 5 fields, ref: 2 fields when given, phi, geom, D, nbr when given).
template <typename T>
bool output_overlaps_inputs(const void *out, int64_t obytes, const Sizes &z, const T *q,
                            const T *ref, const T *phi, const T *geom, const T *D,
                            const int32_t *nbr)
{
    return overlaps(out, obytes, q, 5 * z.field) || overlaps(out, obytes, ref, 2 * z.field) ||
           overlaps(out, obytes, phi, z.field) || overlaps(out, obytes, geom, 10 * z.field) ||
           overlaps(out, obytes, D, z.Nq * z.Nq * (int64_t)sizeof(T)) ||
           overlaps(out, obytes, nbr, 6 * z.nelem * (int64_t)sizeof(int32_t));
}

template <typename T>
Rotation<T> rotation(const T *omega)
{
    Rotation<T> rot{T(0), T(0), T(0), false};
    if (omega) rot = Rotation<T>{omega[0], omega[1], omega[2], true};
    return rot;
}

// The volume term (SURF = false) or the whole right-hand side (SURF = true:
// nbr must be given; omega, a host pointer to 3 values read during the call,
// adds the Coriolis source), of the full state (ref NULL) or of perturbation
// variables about the reference ref (whole right-hand side only).
template <typename T, bool SURF>
int evaluate(const T *q, const T *ref, const T *phi, const T *geom, const T *D,
             const int32_t *nbr, const T *omega, int N, int64_t nelem, T *rhs, hipStream_t stream,
             bool pert)
{
    Sizes z;
    if (int st = check_sizes<T>(N, nelem, z)) return st;
    if (nelem == 0) return ESDG_OK;
    if (!q || !phi || !geom || !D || !rhs || (SURF && !nbr) || (pert && !ref)) return ESDG_ERR_NULL;
    if (output_overlaps_inputs(rhs, 5 * z.field, z, q, pert ? ref : nullptr, phi, geom, D,
                               SURF ? nbr : nullptr))
        return ESDG_ERR_ALIAS;
    const Rotation<T> rot = SURF ? rotation(omega) : Rotation<T>{T(0), T(0), T(0), false};
    const Sink<T, false> sink{rhs, nullptr, T(0), T(0), T(0)};
    if (!SURF) return launch_order<T, false, false, false>(N, q, nullptr, phi, geom, D, nullptr, rot,
                                                           nelem, sink, stream);
    if (pert) return launch_order<T, true, false, true>(N, q, ref, phi, geom, D, nbr, rot, nelem,
                                                        sink, stream);
    return launch_order<T, true, false, false>(N, q, nullptr, phi, geom, D, nbr, rot, nelem, sink,
                                               stream);
}

// One low-storage Runge-Kutta stage: dq <- a dq + dt rhs(q_in), q_out <- q_in + b dq,
// rhs the whole right-hand side.
template <typename T>
int stage(const T *q_in, const T *ref, const T *phi, const T *geom, const T *D, const int32_t *nbr,
          const T *omega, T a, T b, T dt, int N, int64_t nelem, T *dq, T *q_out,
          hipStream_t stream)
{
    Sizes z;
    if (int st = check_sizes<T>(N, nelem, z)) return st;
    if (nelem == 0) return ESDG_OK;
    if (!q_in || !phi || !geom || !D || !nbr || !dq || !q_out) return ESDG_ERR_NULL;
    if (output_overlaps_inputs(dq, 5 * z.field, z, q_in, ref, phi, geom, D, nbr) ||
        output_overlaps_inputs(q_out, 5 * z.field, z, q_in, ref, phi, geom, D, nbr) ||
        overlaps(dq, 5 * z.field, q_out, 5 * z.field))
        return ESDG_ERR_ALIAS;
    const Sink<T, true> sink{dq, q_out, a, b, dt};
    const Rotation<T> rot = rotation(omega);
    if (ref) return launch_order<T, true, true, true>(N, q_in, ref, phi, geom, D, nbr, rot, nelem,
                                                      sink, stream);
    return launch_order<T, true, true, false>(N, q_in, nullptr, phi, geom, D, nbr, rot, nelem, sink,
                                              stream);
}

// The five-stage fourth-order 2N-storage scheme of Carpenter and Kennedy
// (NASA TM-109112, 1994), as the ratios of integers it is published as:
// stage s updates dq <- A_s dq + dt L(q), q <- q + B_s dq.
constexpr int kStages = 5;
constexpr double kLsrkA[kStages] = {
    0.0,
    -567301805773.0 / 1357537059087.0,
    -2404267990393.0 / 2016746695238.0,
    -3550918686646.0 / 2091501179385.0,
    -1275806237668.0 / 842570457699.0,
};
constexpr double kLsrkB[kStages] = {
    1432997174477.0 / 9575080441755.0,
    5161836677717.0 / 13612068292357.0,
    1720146321549.0 / 2090206949498.0,
    3134564353537.0 / 4481467310338.0,
    2277821191437.0 / 14882151754819.0,
};

template <typename T>
int copy(const T *src, T *dst, int64_t n, hipStream_t stream)
{
    if (n == 0) return ESDG_OK;
    const int64_t want = (n + 255) / 256;
    const unsigned blocks = (unsigned)(want < 4096 ? want : 4096);
    hipLaunchKernelGGL((copy_kernel<T>), dim3(blocks), dim3(256), 0, stream, src, dst, n);
    return hipGetLastError() == hipSuccess ? ESDG_OK : ESDG_ERR_LAUNCH;
}

// nsteps steps: the stages alternate between q and q_tmp; after an odd number
// of stages in total the state is copied back into q.
template <typename T>
int steps(T *q, T *q_tmp, T *dq, const T *ref, const T *phi, const T *geom, const T *D,
          const int32_t *nbr, const T *omega, T dt, int nsteps, int N, int64_t nelem,
          hipStream_t stream)
{
    Sizes z;
    if (int st = check_sizes<T>(N, nelem, z)) return st;
    if (nsteps < 0) return ESDG_ERR_NELEM;
    if (nelem == 0 || nsteps == 0) return ESDG_OK;
    if (!q || !q_tmp || !dq || !phi || !geom || !D || !nbr) return ESDG_ERR_NULL;
    if (overlaps(q, 5 * z.field, q_tmp, 5 * z.field) ||
        output_overlaps_inputs(q_tmp, 5 * z.field, z, (const T *)nullptr, ref, phi, geom, D, nbr) ||
        output_overlaps_inputs(q, 5 * z.field, z, (const T *)nullptr, ref, phi, geom, D, nbr))
        return ESDG_ERR_ALIAS;
    // stage() checks dq against everything else
    T *src = q, *dst = q_tmp;
    for (int n = 0; n < nsteps; ++n) {
        for (int s = 0; s < kStages; ++s) {
            const int st = stage<T>(src, ref, phi, geom, D, nbr, omega, T(kLsrkA[s]), T(kLsrkB[s]),
                                    dt, N, nelem, dq, dst, stream);
            if (st != ESDG_OK) return st;
            T *t = src;
            src = dst;
            dst = t;
        }
    }
    return src == q ? ESDG_OK : copy<T>(src, q, 5 * z.field / (int64_t)sizeof(T), stream);
}

// Partial sums over the grid of integrals_partial_kernel: one per 256 nodes,
// at most kIntegralBlocks.
int integral_blocks(int64_t nnodes)
{
    const int64_t want = (nnodes + kIntegralThreads - 1) / kIntegralThreads;
    return (int)(want < kIntegralBlocks ? want : kIntegralBlocks);
}

// The three integrals into out (device, 3 doubles), with `part` (device) of
// at least 3 * kIntegralBlocks doubles for the partial sums.
template <typename T>
int integrals(const T *q, const T *ref, const T *phi, const T *geom, const T *w, int N,
              int64_t nelem, double *part, double *out, hipStream_t stream)
{
    Sizes z;
    if (int st = check_sizes<T>(N, nelem, z)) return st;
    if (!out || !part) return ESDG_ERR_NULL;
    if (overlaps(out, 3 * sizeof(double), part, 3 * kIntegralBlocks * sizeof(double)))
        return ESDG_ERR_ALIAS;
    if (nelem > 0 && (!q || !phi || !geom || !w)) return ESDG_ERR_NULL;
    const int64_t nnodes = nelem * z.Np;
    if (nelem > 0 && (output_overlaps_inputs(out, 3 * sizeof(double), z, q, ref, phi, geom,
                                             (const T *)nullptr, nullptr) ||
                      output_overlaps_inputs(part, 3 * kIntegralBlocks * sizeof(double), z, q, ref,
                                             phi, geom, (const T *)nullptr, nullptr) ||
                      overlaps(out, 3 * sizeof(double), w, z.Nq * (int64_t)sizeof(T)) ||
                      overlaps(part, 3 * kIntegralBlocks * sizeof(double), w,
                               z.Nq * (int64_t)sizeof(T))))
        return ESDG_ERR_ALIAS;
    const int nb = integral_blocks(nnodes);
    if (nb > 0) {
        if (ref)
            hipLaunchKernelGGL((integrals_partial_kernel<T, true>), dim3(nb), dim3(kIntegralThreads),
                               0, stream, q, ref, phi, geom, w, (int)z.Nq, nnodes, part);
        else
            hipLaunchKernelGGL((integrals_partial_kernel<T, false>), dim3(nb),
                               dim3(kIntegralThreads), 0, stream, q, ref, phi, geom, w, (int)z.Nq,
                               nnodes, part);
    }
    hipLaunchKernelGGL(integrals_final_kernel, dim3(1), dim3(kIntegralThreads), 0, stream, part, nb,
                       out);
    return hipGetLastError() == hipSuccess ? ESDG_OK : ESDG_ERR_LAUNCH;
}

// The allocation-free variant of the integrals keeps its partial sums in
// this file-scope device array (one copy per device, held until the process
// ends) instead of a caller's workspace.  Host code never uses the array's
// name as an address: each device's address comes from hipGetSymbolAddress,
// taken once per device with that device current, and is kept below.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
double *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) double scratch[3 * kIntegralBlocks];

namespace {

// The current device's address of `scratch` (looked up on the first call on
// that device); NULL with *status set when the device cannot be queried.
double *scratch_on_current_device(int *status)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *status = ESDG_ERR_DEVICE;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            *status = ESDG_ERR_DEVICE;
            return nullptr;
        }
        g_scratch_ptr[dev] = static_cast<double *>(p);
    }
    *status = ESDG_OK;
    return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace esdg

extern "C" {

int esdg_volume_rhs_f64(const double *q, const double *phi, const double *geom, const double *D,
                        int N, int64_t nelem, double *rhs, hipStream_t stream)
{
    return esdg::evaluate<double, false>(q, nullptr, phi, geom, D, nullptr, nullptr, N, nelem, rhs,
                                         stream, false);
}

int esdg_volume_rhs_f32(const float *q, const float *phi, const float *geom, const float *D,
                        int N, int64_t nelem, float *rhs, hipStream_t stream)
{
    return esdg::evaluate<float, false>(q, nullptr, phi, geom, D, nullptr, nullptr, N, nelem, rhs,
                                        stream, false);
}

int esdg_rhs_f64(const double *q, const double *phi, const double *geom, const double *D,
                 const int32_t *nbr, const double *omega, int N, int64_t nelem, double *rhs,
                 hipStream_t stream)
{
    return esdg::evaluate<double, true>(q, nullptr, phi, geom, D, nbr, omega, N, nelem, rhs, stream,
                                        false);
}

int esdg_rhs_f32(const float *q, const float *phi, const float *geom, const float *D,
                 const int32_t *nbr, const float *omega, int N, int64_t nelem, float *rhs,
                 hipStream_t stream)
{
    return esdg::evaluate<float, true>(q, nullptr, phi, geom, D, nbr, omega, N, nelem, rhs, stream,
                                       false);
}

int esdg_rhs_pert_f64(const double *qp, const double *ref, const double *phi, const double *geom,
                      const double *D, const int32_t *nbr, const double *omega, int N,
                      int64_t nelem, double *rhs, hipStream_t stream)
{
    return esdg::evaluate<double, true>(qp, ref, phi, geom, D, nbr, omega, N, nelem, rhs, stream,
                                        true);
}

int esdg_rhs_pert_f32(const float *qp, const float *ref, const float *phi, const float *geom,
                      const float *D, const int32_t *nbr, const float *omega, int N,
                      int64_t nelem, float *rhs, hipStream_t stream)
{
    return esdg::evaluate<float, true>(qp, ref, phi, geom, D, nbr, omega, N, nelem, rhs, stream,
                                       true);
}

int esdg_lsrk_stage_f64(const double *q_in, const double *ref, const double *phi,
                        const double *geom, const double *D, const int32_t *nbr,
                        const double *omega, double a, double b, double dt, int N, int64_t nelem,
                        double *dq, double *q_out, hipStream_t stream)
{
    return esdg::stage<double>(q_in, ref, phi, geom, D, nbr, omega, a, b, dt, N, nelem, dq, q_out,
                               stream);
}

int esdg_lsrk_stage_f32(const float *q_in, const float *ref, const float *phi, const float *geom,
                        const float *D, const int32_t *nbr, const float *omega, float a, float b,
                        float dt, int N, int64_t nelem, float *dq, float *q_out,
                        hipStream_t stream)
{
    return esdg::stage<float>(q_in, ref, phi, geom, D, nbr, omega, a, b, dt, N, nelem, dq, q_out,
                              stream);
}

int esdg_lsrk_steps_f64(double *q, double *q_tmp, double *dq, const double *ref,
                        const double *phi, const double *geom, const double *D,
                        const int32_t *nbr, const double *omega, double dt, int nsteps, int N,
                        int64_t nelem, hipStream_t stream)
{
    return esdg::steps<double>(q, q_tmp, dq, ref, phi, geom, D, nbr, omega, dt, nsteps, N, nelem,
                               stream);
}

int esdg_lsrk_steps_f32(float *q, float *q_tmp, float *dq, const float *ref, const float *phi,
                        const float *geom, const float *D, const int32_t *nbr,
                        const float *omega, float dt, int nsteps, int N, int64_t nelem,
                        hipStream_t stream)
{
    return esdg::steps<float>(q, q_tmp, dq, ref, phi, geom, D, nbr, omega, dt, nsteps, N, nelem,
                              stream);
}

int esdg_lsrk_stages(void) { return esdg::kStages; }

int esdg_lsrk_coefficients(double *A, double *B)
{
    if (!A || !B) return ESDG_ERR_NULL;
    for (int s = 0; s < esdg::kStages; ++s) {
        A[s] = esdg::kLsrkA[s];
        B[s] = esdg::kLsrkB[s];
    }
    return ESDG_OK;
}

int64_t esdg_integrals_workspace_bytes(void)
{
    return 3 * (int64_t)esdg::kIntegralBlocks * (int64_t)sizeof(double);
}

int esdg_integrals_f64(const double *q, const double *ref, const double *phi, const double *geom,
                       const double *w, int N, int64_t nelem, double *work, double *out,
                       hipStream_t stream)
{
    return esdg::integrals<double>(q, ref, phi, geom, w, N, nelem, work, out, stream);
}

int esdg_integrals_f32(const float *q, const float *ref, const float *phi, const float *geom,
                       const float *w, int N, int64_t nelem, double *work, double *out,
                       hipStream_t stream)
{
    return esdg::integrals<float>(q, ref, phi, geom, w, N, nelem, work, out, stream);
}

int esdg_integrals_noalloc_f64(const double *q, const double *ref, const double *phi,
                               const double *geom, const double *w, int N, int64_t nelem,
                               double *out, hipStream_t stream)
{
    esdg::Sizes z;
    if (int st = esdg::check_sizes<double>(N, nelem, z)) return st;
    // the partial sums never exceed the array: at most kIntegralBlocks per call
    if (esdg::integral_blocks(nelem * z.Np) > esdg::kIntegralBlocks) return ESDG_ERR_NELEM;
    int st = ESDG_OK;
    double *part = esdg::scratch_on_current_device(&st);
    if (!part) return st;
    return esdg::integrals<double>(q, ref, phi, geom, w, N, nelem, part, out, stream);
}

const char *esdg_status_string(int status)
{
    switch (status) {
        case ESDG_OK: return "ok";
        case ESDG_ERR_NULL: return "a required pointer is NULL";
        case ESDG_ERR_ORDER: return "polynomial order N outside the compiled range";
        case ESDG_ERR_NELEM: return "nelem is negative or too large";
        case ESDG_ERR_LAUNCH: return "kernel launch failed";
        case ESDG_ERR_ALIAS: return "an output overlaps an input or another output";
        case ESDG_ERR_DEVICE: return "the current device or its scratch array could not be located";
    }
    return "unknown status";
}

int esdg_min_order(void) { return esdg::kMinOrder; }
int esdg_max_order(void) { return esdg::kMaxOrder; }

}  // extern "C"
