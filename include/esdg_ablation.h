/*
 * esdg_ablation.h -- C ABI of libesdg_ablation.so: the volume term of
 * esdg.h computed by a ladder of kernel variants that replays, on MI355X, the
 * cumulative optimisation study of "GPU Performance of an Entropy-Stable
 * Discontinuous Galerkin Euler Solver with Non-Conservative Terms"
 * (arXiv 2605.16684v2), §4.1 and Fig. 2.  Every variant maps one thread to one
 * node, as the page does, and computes the same result as
 * esdg_volume_rhs_f64 (same layouts, same contract, fp64 only); the ladder
 * measures which of the page's steps pay off on CDNA4.
 *
 * Variants (cumulative):
 *   ESDG_ABL_BASELINE     one launch per direction (node data staged in LDS
 *                         each time, rhs accumulated in HBM), every ordered
 *                         pair, primitives recomputed per pair, log means
 *                         from a per-pair log, the 3 x 5 flux matrix formed
 *                         and contracted with the metric
 *   ESDG_ABL_HOIST        + primitives computed once per node
 *   ESDG_ABL_LOGMEAN      + logs once per node and the series log mean
 *   ESDG_ABL_CONTRA       + contravariant flux and inverse log mean directly
 *   ESDG_ABL_SYM_UPPER    + half-sweep (each unordered pair once, partner's
 *                         gravity term rescaled, §4.1) with the upper-
 *                         triangular assignment (Fig. 1a)
 *   ESDG_ABL_SYM_INDEXED  half-sweep with the cyclic indexing schedule (Eq. 6)
 *   ESDG_ABL_SYM_WEIGHTED half-sweep with the weighted cyclic schedule
 *                         (constant trip count, antipodal pairs twice at
 *                         weight 1/2, Fig. 1b)
 *   ESDG_ABL_FUSED        weighted half-sweep, three directions in one launch
 *
 * ESDG_ABL_FUSE_FLAG or-ed into any variant runs that variant's three
 * directions in one launch (node data staged once, rhs written once), so the
 * arithmetic steps can also be compared without the per-direction HBM
 * traffic; ESDG_ABL_FUSED | ESDG_ABL_FUSE_FLAG is ESDG_ABL_FUSED.
 *
 * Status codes as in esdg.h; N must be 3, 4 or 7 (ESDG_ERR_ORDER otherwise),
 * nelem at most INT32_MAX (one workgroup per element; ESDG_ERR_NELEM otherwise),
 * variant outside the list gives ESDG_ERR_VARIANT.  Device pointers, caller
 * owned, asynchronous on `stream`, rhs overwritten, nelem == 0 a no-op.
 */
#ifndef ESDG_ABLATION_H
#define ESDG_ABLATION_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ESDG_ABL_BASELINE 0
#define ESDG_ABL_HOIST 1
#define ESDG_ABL_LOGMEAN 2
#define ESDG_ABL_CONTRA 3
#define ESDG_ABL_SYM_UPPER 4
#define ESDG_ABL_SYM_INDEXED 5
#define ESDG_ABL_SYM_WEIGHTED 6
#define ESDG_ABL_FUSED 7
#define ESDG_ABL_COUNT 8
#define ESDG_ABL_FUSE_FLAG 0x100

#define ESDG_ERR_VARIANT (-6)

/* Volume term (fp64) by ablation variant `variant`; see the list above. */
int esdg_ablation_volume_rhs_f64(int variant, const double *q, const double *phi,
                                 const double *geom, const double *D, int N, int64_t nelem,
                                 double *rhs, hipStream_t stream);

/*
 * The production kernel of esdg_volume_rhs_f64 with two lanes per grid line
 * instead of one, at N = 5 and N = 7 (ESDG_ERR_ORDER otherwise): adjacent
 * lanes each own half of a line's nodes, evaluate the pairs within their
 * half and half of the pairs across the halves, and hand the partner's
 * contributions to the other lane by a cross-lane (DPP) swap, so a lane holds
 * half the accumulators and metric of a line and the kernel fits three waves
 * per SIMD instead of two.  It is kept for measurement against the
 * one-lane-per-line production shape (same result up to rounding, same
 * contract as esdg_volume_rhs_f64); the page's register-pressure remark
 * ([ESDG-GPU §4.1], temporary local copies and occupancy) is what it tests.
 */
int esdg_ablation_two_lane_volume_rhs_f64(const double *q, const double *phi, const double *geom,
                                          const double *D, int N, int64_t nelem, double *rhs,
                                          hipStream_t stream);

/* Short name of a variant, with or without ESDG_ABL_FUSE_FLAG (static
 * string, "unknown" outside the list). */
const char *esdg_ablation_name(int variant);

#ifdef __cplusplus
}
#endif
#endif /* ESDG_ABLATION_H */
