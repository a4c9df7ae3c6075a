/*
 * esdg.h -- C ABI of the ESDG flux-differencing volume-term library
 * (libesdg.so, HIP for AMD gfx950): the volume term alone
 * (esdg_volume_rhs_*), the whole right-hand side with the
 * entropy-conservative surface term fused into the same kernel (esdg_rhs_*,
 * esdg_rhs_pert_* for perturbation variables), low-storage Runge-Kutta
 * stages and steps with the right-hand side fused in (esdg_lsrk_*), and the
 * global conservation integrals (esdg_integrals_*).
 *
 * The operation is the volume term of the semi-discrete entropy-stable DG
 * form of "GPU Performance of an Entropy-Stable Discontinuous Galerkin Euler
 * Solver with Non-Conservative Terms" (arXiv 2605.16684v2): §3, Eq. 2 (the
 * volume part, source h = 0), with the two-point entropy-conservative flux of
 * §4.1, Eq. 3-5 and the non-conservative gravity term split as in §4.1.
 * Per node i of element e, with i_k its index along reference direction k and
 * l running over the other nodes of the k-line through i:
 *
 *   rhs_i = -(1/J_i) sum_{k=1..3} sum_{l != i_k} D[i_k][l]
 *                    sum_{j=1..3} (Ja^k_j(i) + Ja^k_j(l)) F_j(q_i, q_l)
 *
 * where F_j(q_i, q_l) is the two-point flux in physical direction j with the
 * receiving node i as the "-" state (Eq. 4-5) and gamma = 1.4.
 *
 * Layouts (all arrays contiguous, Nq = N+1, Np = Nq^3, node index
 * n = a + Nq*(b + Nq*c) with a, b, c the indices along xi_1, xi_2, xi_3):
 *   q     [5][nelem][Np]   rho, rho*u1, rho*u2, rho*u3, E (E includes rho*phi)
 *   phi   [nelem][Np]      geopotential
 *   geom  [10][nelem][Np]  Ja^1_1, Ja^1_2, Ja^1_3, Ja^2_1, ..., Ja^3_3, J,
 *                          Ja^k_j = J * d(xi_k)/d(x_j), J > 0
 *   D     [Nq][Nq]         row-major, D[a][l] = l_l'(xi_a) on the LGL nodes
 *                          (must satisfy the SBP property of an LGL
 *                          collocation operator; only D[a][l], l != a, is read)
 *   rhs   [5][nelem][Np]   OUTPUT, overwritten
 *
 * Ownership and semantics:
 *   - Every pointer is a DEVICE pointer to memory owned by the caller; the
 *     library allocates nothing and keeps no state between calls.
 *   - rhs must not overlap any input (checked: ESDG_ERR_ALIAS).
 *   - The call is asynchronous on `stream` (0 = the null stream) and never
 *     synchronises; it is thread-safe and re-entrant.
 *   - nelem == 0 returns ESDG_OK without launching (pointers are not read).
 *   - Argument errors are returned synchronously, before any HIP call.
 *   - Not checked (preconditions): rho > 0, p > 0, J > 0, finite values.
 *     Violations give NaN/Inf in rhs; they never cause out-of-bounds access.
 *   - Pointers must be aligned to the element type.
 */
#ifndef ESDG_H
#define ESDG_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ESDG_OK          0
#define ESDG_ERR_NULL   (-1)  /* a required pointer is NULL (nelem > 0)             */
#define ESDG_ERR_ORDER  (-2)  /* N outside [esdg_min_order(), esdg_max_order()]     */
#define ESDG_ERR_NELEM  (-3)  /* nelem < 0, or the arrays would not be addressable  */
#define ESDG_ERR_LAUNCH (-4)  /* the kernel launch failed (hipGetLastError)         */
#define ESDG_ERR_ALIAS  (-5)  /* an output overlaps an input or another output      */
#define ESDG_ERR_DEVICE (-7)  /* the current device (or its scratch array) could not
                                 be located: esdg_integrals_noalloc_f64 only          */

/* Volume term in fp64 arithmetic. Returns a status code above. */
int esdg_volume_rhs_f64(const double *q, const double *phi, const double *geom,
                        const double *D, int N, int64_t nelem, double *rhs,
                        hipStream_t stream);

/* Volume term in fp32 arithmetic (fp32 inputs and output); same contract. */
int esdg_volume_rhs_f32(const float *q, const float *phi, const float *geom,
                        const float *D, int N, int64_t nelem, float *rhs,
                        hipStream_t stream);

/*
 * Whole semi-discrete right-hand side of Eq. 2 of the same page (its volume
 * term, its surface term and the source h), with the entropy-conservative
 * two-point flux also on the faces: the face dissipation the page adds to it
 * ([ESDG-GPU §3], from its reference [56]) is not part of this call.  At a
 * node on the xi_k = +-1 face of an element the surface term is
 *     -(+-1) sum_j Ja^k_j(i) F*_j(q_i, q_partner) / (w_end J_i),
 * w_end = 2/(N(N+1)) the LGL end weight, F* the same two-point flux as in
 * the volume (gravity term included).
 *
 *   omega  HOST pointer to 3 values (read during the call, not kept), or NULL:
 *        the rotation vector of the Coriolis term of Eq. 1b; the source is
 *        h = -omega x U on the momentum (U = rho u), added at every node;
 *        NULL means h = 0.  For a planet rotating at Omega, omega = 2 Omega.
 *   nbr  [nelem][6] int32, device: the element across each face, faces in the
 *        order -xi1, +xi1, -xi2, +xi2, -xi3, +xi3.  A neighbour index e' in
 *        [0, nelem) means the faces are conforming with the same orientation:
 *        the partner of node (.., i_k = N, ..) across the +xi_k face is node
 *        (.., i_k = 0, ..) of e' (same tangential indices), and vice versa;
 *        periodic meshes simply name the wrapped element.  -1 is a slip wall:
 *        the partner is the mirror state of the own node (same density,
 *        pressure and phi, velocity reflected in the face normal Ja^k).  Any
 *        other value makes the rhs of that face's nodes NaN (the kernel reads
 *        nothing through it); the library does not check nbr on the host.
 *
 * Everything else (layouts, ownership, streams, status codes, rhs
 * overwritten, nelem == 0 a no-op) as for esdg_volume_rhs_f64; rhs must not
 * overlap nbr either (ESDG_ERR_ALIAS), and nbr == NULL gives ESDG_ERR_NULL.
 */
int esdg_rhs_f64(const double *q, const double *phi, const double *geom,
                 const double *D, const int32_t *nbr, const double *omega, int N,
                 int64_t nelem, double *rhs, hipStream_t stream);

/* The same in fp32 arithmetic (omega as 3 floats). */
int esdg_rhs_f32(const float *q, const float *phi, const float *geom,
                 const float *D, const int32_t *nbr, const float *omega, int N,
                 int64_t nelem, float *rhs, hipStream_t stream);

/*
 * Whole right-hand side (as esdg_rhs_*) of a state carried in perturbation
 * variables about a reference state at rest, the cure the page names for the
 * noise of 32-bit runs on full state variables ([ESDG-GPU §5.2], the last
 * paragraph of the baroclinic test).  With the reference's density rbar and
 * pressure pbar (its total energy Ebar = pbar/(gamma-1) + rbar phi):
 *
 *   qp   [5][nelem][Np]  rho - rbar, rho u1, rho u2, rho u3, E - Ebar
 *   ref  [2][nelem][Np]  rbar, pbar (> 0)
 *
 * and the result is the right-hand side of the full state
 * (rbar + qp0, qp1, qp2, qp3, Ebar + qp4).  The kernel forms the pressure as
 * pbar + (gamma-1)(qp4 - |U|^2/(2 rho) - qp0 phi), so the reference's share
 * never enters the subtraction.  The fp32 entry also forms the momentum
 * flux's pressure mean relative to each element's reference pressure (pbar
 * at its node (N/2, N/2, N/2)) and adds that constant's share per node in
 * fp64: the same result in exact arithmetic, with the rounding of O(p)
 * pair fluxes taken out of near-balanced states.  rhs must not overlap ref
 * either; ref == NULL gives ESDG_ERR_NULL.  Everything else as esdg_rhs_f64.
 */
int esdg_rhs_pert_f64(const double *qp, const double *ref, const double *phi, const double *geom,
                      const double *D, const int32_t *nbr, const double *omega, int N,
                      int64_t nelem, double *rhs, hipStream_t stream);
int esdg_rhs_pert_f32(const float *qp, const float *ref, const float *phi, const float *geom,
                      const float *D, const int32_t *nbr, const float *omega, int N,
                      int64_t nelem, float *rhs, hipStream_t stream);

/*
 * One stage of a 2N-storage low-storage Runge-Kutta scheme on the whole
 * right-hand side L (as esdg_rhs_*, or esdg_rhs_pert_* when ref is given),
 * fused into the same kernel ([ESDG-GPU §3]: the solver advances with a
 * low-storage Runge-Kutta scheme and recomputes the fluxes at every stage;
 * [ESDG-GPU §4.2, Fig. 4] times the update as a kernel of its own):
 *
 *   dq    <- a dq + dt L(q_in)          (a == 0: dq is not read)
 *   q_out <- q_in + b dq
 *
 *   q_in   [5][nelem][Np]  the stage's state (perturbation variables with ref)
 *   ref    [2][nelem][Np]  or NULL: reference density and pressure, as above
 *   dq     [5][nelem][Np]  the scheme's register, read (a != 0) and written
 *   q_out  [5][nelem][Np]  OUTPUT: the next stage's state
 *
 * q_out and dq must not overlap each other or any input (q_out cannot be
 * q_in: neighbouring elements read q_in's face nodes during the launch);
 * ESDG_ERR_ALIAS otherwise.  nbr, omega and the rest as esdg_rhs_f64.
 */
int esdg_lsrk_stage_f64(const double *q_in, const double *ref, const double *phi,
                        const double *geom, const double *D, const int32_t *nbr,
                        const double *omega, double a, double b, double dt, int N, int64_t nelem,
                        double *dq, double *q_out, hipStream_t stream);
int esdg_lsrk_stage_f32(const float *q_in, const float *ref, const float *phi, const float *geom,
                        const float *D, const int32_t *nbr, const float *omega, float a, float b,
                        float dt, int N, int64_t nelem, float *dq, float *q_out,
                        hipStream_t stream);

/*
 * nsteps >= 0 steps of size dt of dq/dt = L(q) (the whole right-hand side,
 * in perturbation variables when ref is given) with the five-stage
 * fourth-order 2N-storage scheme of Carpenter and Kennedy (1994), which
 * stands in for the page's fourteen-stage scheme (its coefficients are not
 * on the page; the page's solver used a five-stage fourth-order scheme
 * before).  The stages ping-pong between q and q_tmp; the result is left in
 * q (one device copy at the end when the stage count is odd).
 *
 *   q      [5][nelem][Np]  in: the state; out: the state after nsteps steps
 *   q_tmp  [5][nelem][Np]  workspace, overwritten
 *   dq     [5][nelem][Np]  workspace (the register), overwritten
 *
 * q, q_tmp and dq must be pairwise disjoint and disjoint from the inputs
 * (ESDG_ERR_ALIAS); nsteps < 0 gives ESDG_ERR_NELEM; nsteps == 0 or
 * nelem == 0 is a no-op.  Launches 5 nsteps kernels (+1 copy) on `stream`
 * and returns at once; an error from a later launch stops the sequence and
 * is returned.
 */
int esdg_lsrk_steps_f64(double *q, double *q_tmp, double *dq, const double *ref,
                        const double *phi, const double *geom, const double *D,
                        const int32_t *nbr, const double *omega, double dt, int nsteps, int N,
                        int64_t nelem, hipStream_t stream);
int esdg_lsrk_steps_f32(float *q, float *q_tmp, float *dq, const float *ref, const float *phi,
                        const float *geom, const float *D, const int32_t *nbr,
                        const float *omega, float dt, int nsteps, int N, int64_t nelem,
                        hipStream_t stream);

/* Stage count of the scheme esdg_lsrk_steps_* uses (5), and its coefficients:
 * stage s updates dq <- A[s] dq + dt L(q), q <- q + B[s] dq.  A and B are HOST
 * arrays of esdg_lsrk_stages() doubles; returns ESDG_ERR_NULL if either is
 * NULL. */
int esdg_lsrk_stages(void);
int esdg_lsrk_coefficients(double *A, double *B);

/*
 * Global conservation diagnostics of [ESDG-GPU §5.2]: the sums over the
 * elements of the integrals of rho, of E (= rho e, e including phi) and of
 * the entropy eta = -rho s/(gamma-1), s = ln p - gamma ln rho, by the LGL
 * quadrature of the collocation nodes (weight w[a] w[b] w[c] J at node
 * a + Nq (b + Nq c)).
 *
 *   q, ref, phi, geom  as above (ref NULL: q is the full state)
 *   w      [Nq]        device: the LGL quadrature weights on [-1, 1]
 *   work   device workspace of esdg_integrals_workspace_bytes() bytes
 *   out    device, 3 doubles: OUTPUT (integral of rho, of E, of eta)
 *
 * Every node's terms are formed and summed in fp64 (also for the fp32 entry);
 * the sum is deterministic (fixed partition and reduction order for a given
 * nelem and N).  nelem == 0 writes zeros.  work and out must not overlap each
 * other or an input (ESDG_ERR_ALIAS).
 */
int64_t esdg_integrals_workspace_bytes(void);
int esdg_integrals_f64(const double *q, const double *ref, const double *phi, const double *geom,
                       const double *w, int N, int64_t nelem, double *work, double *out,
                       hipStream_t stream);
int esdg_integrals_f32(const float *q, const float *ref, const float *phi, const float *geom,
                       const float *w, int N, int64_t nelem, double *work, double *out,
                       hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * integrals as esdg_integrals_f64, without the `work` argument.  The partial
 * sums go to a file-scope device array of the library instead, 3 * 1024
 * doubles (24 KiB) on every device the library runs on, held until the
 * process ends; its address on the current device is looked up on the first
 * call on that device (ESDG_ERR_DEVICE if that fails).  The call allocates
 * nothing.  Any nelem fits: a call writes at most 1024 partial sums (the
 * nodes are split over at most 1024 workgroups); a size needing more would
 * be rejected with ESDG_ERR_NELEM.  Every partial sum a call reads is written
 * earlier in the same call, so nothing needs clearing between calls.
 * Calls on one device share its array: calls that overlap in time on one
 * device (other streams, other host threads) race and give wrong sums; order
 * them on one stream.  Everything else as esdg_integrals_f64.
 */
int esdg_integrals_noalloc_f64(const double *q, const double *ref, const double *phi,
                               const double *geom, const double *w, int N, int64_t nelem,
                               double *out, hipStream_t stream);

/* Static description of a status code (never NULL). */
const char *esdg_status_string(int status);

/* Range of polynomial orders N compiled into the library. */
int esdg_min_order(void);
int esdg_max_order(void);

#ifdef __cplusplus
}
#endif
#endif /* ESDG_H */
