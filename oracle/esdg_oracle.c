/*
 * esdg_oracle.c -- plain, slow CPU oracle of the ESDG flux-differencing
 * volume term, the whole right-hand side, its low-storage Runge-Kutta time
 * stepping and the global conservation integrals.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file: only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header, table or constant with the HIP
 * library; it receives the same seeded input arrays and nothing else.
 *
 * Precision.  The arithmetic type `real` is long double (x86-64: 64-bit
 * significand) when compiled with -DORACLE_LONG_DOUBLE -- the reference the
 * GPU results are compared with -- and double otherwise, the variant that is
 * timed as the CPU baseline.  Inputs and outputs are double arrays in both
 * builds; states are promoted to `real` on entry and results rounded to
 * double once, on exit.
 *
 * Page followed: "GPU Performance of an Entropy-Stable Discontinuous Galerkin
 * Euler Solver with Non-Conservative Terms" (arXiv 2605.16684v2), written
 * [ESDG-GPU] below.
 *
 *   pressure law ........................ [ESDG-GPU §2, the equation after Eq. 1]
 *   semi-discrete volume term ............ [ESDG-GPU §3, Eq. 2 and the text after it]
 *   mean / log mean / jump ............... [ESDG-GPU §4.1, Eq. 3]
 *   momentum flux with gravity ........... [ESDG-GPU §4.1, Eq. 4 and Eq. 5]
 *   diagonal pairs omitted ............... [ESDG-GPU §4.1, Fig. 1 caption]
 *   surface term ......................... [ESDG-GPU §3, Eq. 2 (second brace) and the text
 *                                           after it: minus side = own element, plus side =
 *                                           the neighbour]
 *   Coriolis source h = -omega x U ....... [ESDG-GPU §2, Eq. 1b; §3, h in Eq. 2]
 *   low-storage Runge-Kutta stepping ..... [ESDG-GPU §3, the paragraph after Eq. 2: a
 *                                           five-stage fourth-order low-storage scheme,
 *                                           the fluxes recomputed at every stage]
 *   sum of integrals of rho, rho e and
 *   entropy over the elements ............ [ESDG-GPU §5.2, the conservation paragraph]
 *
 * Readings of the pages that this file takes (the pages print the momentum
 * component only; the other components are fixed by entropy conservation,
 * and the tests pin them by the pairwise entropy condition):
 *   - density flux   F^rho_j = {{rho}}_log {{u_j}}
 *   - energy flux    F^E_j = ( 1/(2(gamma-1){{b}}_log) - 1/2 {{|u|^2}} + {{phi}} ) F^rho_j
 *                            + sum_m {{u_m}} ( F^rho_j {{u_m}} + delta_jm {{rho}}/(2{{b}}) )
 *     where {{|u|^2}} is the mean of |u|^2 (not |{{u}}|^2);
 *   - the "-" state of Eq. 5 is the node that receives the contribution
 *     (own node i), the "+" state its partner l, and [[a]] = a_l - a_i;
 *   - Eq. 2's volume term is read in skew form with M = diag(w J); by the SBP
 *     property it collapses, node by node, to
 *         rhs_i = -(1/J_i) sum_k sum_{l != i_k} D[i_k][l]
 *                          sum_j (Ja^k_j(i) + Ja^k_j(l)) F_j(q_i, q_l)
 *     (l runs over the nodes of the k-line through i); the source h is zero;
 *   - gamma = 7/5.
 *
 * Readings for the surface term (oracle_surface_rhs):
 *   - F* is the same two-point flux as in the volume (entropy conservative,
 *     with its gravity term); the matrix dissipation the pages add to it is
 *     not printed on the pages and is left out;
 *   - M^{-1} M^s G^s_jk F*_j at a node i on the xi_k = +-1 face of an element
 *     is (+-1) Ja^k_j(i) F*_j / (w_end J_i): the surface quadrature weights
 *     cancel against the tangential part of the tensor-product volume
 *     weights, leaving the 1D LGL end weight w_end = 2/(N(N+1)), and the
 *     area-weighted outward normal is +-Ja^k at that face;
 *   - neighbours share the face node for node (conforming, same orientation):
 *     the partner of node (.., i_k = N, ..) across the +xi_k face is node
 *     (.., i_k = 0, ..) of the neighbour, and the other way round;
 *   - a slip wall takes as partner the mirror state of the own node: the same
 *     density, pressure and geopotential, velocity reflected in the face
 *     normal Ja^k(i).
 *
 * Readings for the time stepping (oracle_lsrk_*):
 *   - the pages' fourteen-stage coefficients come from a reference that is not
 *     on the pages; the five-stage fourth-order 2N-storage scheme of Carpenter
 *     and Kennedy (NASA TM-109112, 1994), the kind of scheme the page says the
 *     solver used before, stands in for it.  Per stage s = 1..5, with the
 *     register k starting at zero:
 *         k <- A_s k + dt L(q),   q <- q + B_s k
 *     (the right-hand side is autonomous, so the stage times C_s are unused);
 * Readings for the conservation integrals (oracle_integrals):
 *   - sum over elements of the LGL quadrature of rho, of total energy E
 *     (rho e with e including phi, [ESDG-GPU §2]) and of the entropy
 *     eta = -rho s/(gamma-1), s = ln p - gamma ln rho, with weights
 *     w_a w_b w_c J at node (a, b, c).
 *
 * Every ordered pair is evaluated on its own: no symmetry, no hoisting, no
 * reuse.  That is the plain definition of what the volume term computes.
 */
#include <float.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifdef ORACLE_LONG_DOUBLE
typedef long double real;
#define RLOG1P log1pl
#define RLOG logl
#define RFABS fabsl
#define REAL_MANT_DIG LDBL_MANT_DIG
#else
typedef double real;
#define RLOG1P log1p
#define RLOG log
#define RFABS fabs
#define REAL_MANT_DIG DBL_MANT_DIG
#endif

#define ORACLE_GAMMA ((real)7 / (real)5)

/* State at one node, read off the conserved variables. */
typedef struct {
    real rho;
    real u[3];
    real usq;  /* |u|^2 */
    real p;
    real b;    /* rho / (2 p) */
    real phi;
} node_state;

/* Pressure law of [ESDG-GPU §2]: P = (gamma-1)(E - U.U/(2 rho) - rho phi). */
static node_state read_node(const real q[5], real phi)
{
    node_state s;
    s.rho = q[0];
    s.u[0] = q[1] / q[0];
    s.u[1] = q[2] / q[0];
    s.u[2] = q[3] / q[0];
    s.usq = s.u[0] * s.u[0] + s.u[1] * s.u[1] + s.u[2] * s.u[2];
    real UU = q[1] * q[1] + q[2] * q[2] + q[3] * q[3];
    s.p = (ORACLE_GAMMA - 1) * (q[4] - UU / (2 * q[0]) - q[0] * phi);
    s.b = q[0] / (2 * s.p);
    s.phi = phi;
    return s;
}

/* {{a}} of [ESDG-GPU §4.1, Eq. 3]. */
static real avg(real am, real ap) { return (am + ap) / 2; }

/* {{a}}_log of [ESDG-GPU §4.1, Eq. 3]: (a+ - a-)/(log a+ - log a-), with the
 * limit a- when the two are equal.  Written as d / log1p(d/a-), d = a+ - a-,
 * which is the same quotient and is accurate for nearby arguments. */
static real logmean(real am, real ap)
{
    real d = ap - am;
    if (d == 0) return am;
    return d / RLOG1P(d / am);
}

/* Two-point flux F_j(q_i, q_l) in physical direction j (0, 1, 2), with the
 * own node i as the "-" state and the partner l as the "+" state. */
static void ec_flux(const node_state *si, const node_state *sl, int j, real F[5])
{
    real rho_avg = avg(si->rho, sl->rho);
    real rho_log = logmean(si->rho, sl->rho);
    real b_avg = avg(si->b, sl->b);
    real b_log = logmean(si->b, sl->b);
    real u_avg[3];
    for (int m = 0; m < 3; ++m) u_avg[m] = avg(si->u[m], sl->u[m]);
    real usq_avg = avg(si->usq, sl->usq);
    real phi_avg = avg(si->phi, sl->phi);
    real phi_jump = sl->phi - si->phi;

    real p_tilde = rho_avg / (2 * b_avg);          /* {{rho}}/(2{{b}}), Eq. 4 */
    real rho_hat = b_avg * rho_log / si->b;        /* Eq. 5 */

    real Frho = rho_log * u_avg[j];
    F[0] = Frho;
    for (int m = 0; m < 3; ++m) {
        real Fm = Frho * u_avg[m];
        if (m == j) Fm += p_tilde + rho_hat * phi_jump / 2;   /* Eq. 4 */
        F[1 + m] = Fm;
    }
    real FE = (1 / (2 * (ORACLE_GAMMA - 1) * b_log) - usq_avg / 2 + phi_avg) * Frho;
    for (int m = 0; m < 3; ++m) {
        real sym = Frho * u_avg[m];
        if (m == j) sym += p_tilde;
        FE += u_avg[m] * sym;
    }
    F[4] = FE;
}

/* Batch entry for the flux tests: F[n][5] = F_j(q_i[n], q_l[n]), with the
 * conserved states qi[n][5], ql[n][5] and geopotentials phii[n], phil[n]. */
void oracle_ec_flux(const double *qi, const double *phii, const double *ql,
                    const double *phil, int j, int64_t npair, double *F)
{
    for (int64_t n = 0; n < npair; ++n) {
        real a[5], c[5], out[5];
        for (int f = 0; f < 5; ++f) {
            a[f] = qi[5 * n + f];
            c[f] = ql[5 * n + f];
        }
        node_state si = read_node(a, phii[n]);
        node_state sl = read_node(c, phil[n]);
        ec_flux(&si, &sl, j, out);
        for (int f = 0; f < 5; ++f) F[5 * n + f] = (double)out[f];
    }
}

/*
 * Volume term of Eq. 2 (reading above) on every element, in `real`:
 *
 *   q    [5][nelem][Np]   conserved variables
 *   phi  [nelem][Np]      geopotential
 *   geom [10][nelem][Np]  Ja^1_1..Ja^1_3, Ja^2_1..Ja^2_3, Ja^3_1..Ja^3_3, J
 *   D    [Nq][Nq]         D[a][l] = l_l'(xi_a)
 *   rhs  [5][nelem][Np]   overwritten with the volume term
 *   mag  [5][nelem][Np]   optional (may be NULL): sum over the node's summands
 *                         |(1/J_i) D[i_k][l] sum_j (Ja^k_j(i)+Ja^k_j(l)) F_j|,
 *                         the magnitude against which round-off is measured
 *   nthreads              OpenMP threads (<= 0: the runtime default)
 *
 * Node index n = a + Nq (b + Nq c).
 */
static void volume_rhs_r(const real *q, const double *phi, const double *geom, const double *D,
                         int N, int64_t nelem, real *rhs, double *mag, int nthreads)
{
    const int Nq = N + 1;
    const int64_t Np = (int64_t)Nq * Nq * Nq;
    const int64_t stride = nelem * Np; /* distance between fields */
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads)
#else
    (void)nthreads;
#endif
    for (int64_t e = 0; e < nelem; ++e) {
        node_state *st = (node_state *)malloc((size_t)Np * sizeof(node_state));
        for (int64_t n = 0; n < Np; ++n) {
            real qn[5];
            for (int f = 0; f < 5; ++f) qn[f] = q[f * stride + e * Np + n];
            st[n] = read_node(qn, phi[e * Np + n]);
        }
        for (int c = 0; c < Nq; ++c)
        for (int b = 0; b < Nq; ++b)
        for (int a = 0; a < Nq; ++a) {
            const int64_t i = a + Nq * (b + Nq * c);
            const real Ji = geom[9 * stride + e * Np + i];
            real acc[5] = {0, 0, 0, 0, 0};
            real absacc[5] = {0, 0, 0, 0, 0};
            for (int k = 0; k < 3; ++k) {
                const int ik = (k == 0) ? a : (k == 1) ? b : c;
                for (int l = 0; l < Nq; ++l) {
                    if (l == ik) continue; /* diagonal pairs omitted */
                    const int64_t il = (k == 0) ? l + Nq * (b + Nq * c)
                                     : (k == 1) ? a + Nq * (l + Nq * c)
                                                : a + Nq * (b + Nq * l);
                    real term[5] = {0, 0, 0, 0, 0};
                    for (int j = 0; j < 3; ++j) {
                        const real nj = (real)geom[(3 * k + j) * stride + e * Np + i]
                                      + (real)geom[(3 * k + j) * stride + e * Np + il];
                        real F[5];
                        ec_flux(&st[i], &st[il], j, F);
                        for (int f = 0; f < 5; ++f) term[f] += nj * F[f];
                    }
                    const real d = D[ik * Nq + l];
                    for (int f = 0; f < 5; ++f) {
                        acc[f] += d * term[f];
                        absacc[f] += RFABS(d * term[f]);
                    }
                }
            }
            for (int f = 0; f < 5; ++f) {
                rhs[f * stride + e * Np + i] = -acc[f] / Ji;
                if (mag) mag[f * stride + e * Np + i] = (double)(absacc[f] / RFABS(Ji));
            }
        }
        free(st);
    }
}

/*
 * Surface term of Eq. 2 with the entropy-conservative flux (readings above),
 * ADDED to rhs (and, if mag is not NULL, its absolute value to mag).
 *
 *   nbr [nelem][6]  neighbour across faces -xi1, +xi1, -xi2, +xi2, -xi3,
 *                   +xi3; -1 = slip wall (checked by the caller)
 */
static void surface_rhs_r(const real *q, const double *phi, const double *geom,
                          const int32_t *nbr, int N, int64_t nelem, real *rhs, double *mag,
                          int nthreads)
{
    const int Nq = N + 1;
    const int64_t Np = (int64_t)Nq * Nq * Nq;
    const int64_t stride = nelem * Np;
    const real w_end = (real)2 / ((real)N * (real)(N + 1));  /* LGL weight of xi = +-1 */
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads)
#else
    (void)nthreads;
#endif
    for (int64_t e = 0; e < nelem; ++e) {
        for (int c = 0; c < Nq; ++c)
        for (int b = 0; b < Nq; ++b)
        for (int a = 0; a < Nq; ++a) {
            const int64_t i = a + Nq * (b + Nq * c);
            real qi[5];
            for (int f = 0; f < 5; ++f) qi[f] = q[f * stride + e * Np + i];
            const node_state si = read_node(qi, phi[e * Np + i]);
            const real Ji = geom[9 * stride + e * Np + i];
            for (int k = 0; k < 3; ++k) {
                const int ik = (k == 0) ? a : (k == 1) ? b : c;
                if (ik != 0 && ik != N) continue;  /* not on a xi_k face */
                const int side = (ik == N) ? 1 : -1;
                const int32_t nb = nbr[6 * e + 2 * k + (side > 0 ? 1 : 0)];
                real n[3];
                for (int j = 0; j < 3; ++j) n[j] = geom[(3 * k + j) * stride + e * Np + i];
                node_state sp;
                if (nb < 0) {
                    /* mirror state across the face */
                    sp = si;
                    const real un = (si.u[0] * n[0] + si.u[1] * n[1] + si.u[2] * n[2])
                                  / (n[0] * n[0] + n[1] * n[1] + n[2] * n[2]);
                    for (int j = 0; j < 3; ++j) sp.u[j] = si.u[j] - 2 * un * n[j];
                    sp.usq = sp.u[0] * sp.u[0] + sp.u[1] * sp.u[1] + sp.u[2] * sp.u[2];
                } else {
                    const int jk = N - ik;  /* matching node on the neighbour's opposite face */
                    const int64_t ip = (k == 0) ? jk + Nq * (b + Nq * c)
                                     : (k == 1) ? a + Nq * (jk + Nq * c)
                                                : a + Nq * (b + Nq * jk);
                    real qp[5];
                    for (int f = 0; f < 5; ++f) qp[f] = q[f * stride + (int64_t)nb * Np + ip];
                    sp = read_node(qp, phi[(int64_t)nb * Np + ip]);
                }
                real term[5] = {0, 0, 0, 0, 0};
                for (int j = 0; j < 3; ++j) {
                    real F[5];
                    ec_flux(&si, &sp, j, F);
                    for (int f = 0; f < 5; ++f) term[f] += n[j] * F[f];
                }
                for (int f = 0; f < 5; ++f) {
                    const real v = (real)side * term[f] / (w_end * Ji);
                    rhs[f * stride + e * Np + i] -= v;
                    if (mag) mag[f * stride + e * Np + i] += (double)RFABS(v);
                }
            }
        }
    }
}

/*
 * Source term h of Eq. 2 from the Coriolis term of Eq. 1b: h = -omega x U on
 * the momentum components, U = (q1, q2, q3) the momentum, omega the rotation
 * vector as Eq. 1b writes it (for a planet rotating at Omega it is 2 Omega).
 * ADDED to rhs at every node; density and energy get nothing.
 */
static void add_coriolis_r(const real *q, const double omega[3], int64_t nnodes, real *rhs)
{
    const int64_t stride = nnodes;
    for (int64_t n = 0; n < nnodes; ++n) {
        const real U[3] = {q[1 * stride + n], q[2 * stride + n], q[3 * stride + n]};
        const real wxU[3] = {omega[1] * U[2] - omega[2] * U[1],
                             omega[2] * U[0] - omega[0] * U[2],
                             omega[0] * U[1] - omega[1] * U[0]};
        for (int m = 0; m < 3; ++m) rhs[(1 + m) * stride + n] -= wxU[m];
    }
}

/* double <-> real copies of whole arrays (split over the OpenMP threads, so
 * that the copies of the long double build do not serialise a call) */
static real *promote(const double *x, int64_t n)
{
    real *r = (real *)calloc((size_t)(n > 0 ? n : 1), sizeof(real));
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t i = 0; i < n; ++i) r[i] = x[i];
    return r;
}

static void demote(const real *r, int64_t n, double *x)
{
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t i = 0; i < n; ++i) x[i] = (double)r[i];
}

static int bad_neighbour(const int32_t *nbr, int64_t nelem)
{
    for (int64_t i = 0; i < 6 * nelem; ++i)
        if (nbr[i] < -1 || nbr[i] >= nelem) return 1;
    return 0;
}

/* Volume term (double arrays; see volume_rhs_r).  Returns 0, or -1 on bad sizes. */
int oracle_volume_rhs(const double *q, const double *phi, const double *geom,
                      const double *D, int N, int64_t nelem, double *rhs, double *mag,
                      int nthreads)
{
    if (N < 1 || nelem < 0) return -1;
    const int64_t n = 5 * nelem * (int64_t)(N + 1) * (N + 1) * (N + 1);
    real *qr = promote(q, n);
    real *rr = (real *)malloc((size_t)(n > 0 ? n : 1) * sizeof(real));
    volume_rhs_r(qr, phi, geom, D, N, nelem, rr, mag, nthreads);
    demote(rr, n, rhs);
    free(qr);
    free(rr);
    return 0;
}

/* Surface term ADDED to rhs (double arrays; see surface_rhs_r).
 * Returns 0, -1 on bad sizes, -2 if a neighbour index is outside [-1, nelem). */
int oracle_surface_rhs(const double *q, const double *phi, const double *geom,
                       const int32_t *nbr, int N, int64_t nelem, double *rhs, double *mag,
                       int nthreads)
{
    if (N < 1 || nelem < 0) return -1;
    if (bad_neighbour(nbr, nelem)) return -2;
    const int64_t n = 5 * nelem * (int64_t)(N + 1) * (N + 1) * (N + 1);
    real *qr = promote(q, n);
    real *rr = promote(rhs, n);
    surface_rhs_r(qr, phi, geom, nbr, N, nelem, rr, mag, nthreads);
    demote(rr, n, rhs);
    free(qr);
    free(rr);
    return 0;
}

/* Coriolis source ADDED to rhs (double arrays; see add_coriolis_r). */
void oracle_add_coriolis(const double *q, const double omega[3], int64_t nnodes, double *rhs)
{
    real *qr = promote(q, 5 * nnodes);
    real *rr = promote(rhs, 5 * nnodes);
    add_coriolis_r(qr, omega, nnodes, rr);
    demote(rr, 5 * nnodes, rhs);
    free(qr);
    free(rr);
}

/* ---------------------------------------------------------------------------
 * Low-storage Runge-Kutta time stepping (reading above).
 *
 * The five-stage fourth-order 2N-storage coefficients of Carpenter and
 * Kennedy (1994), as the ratios of integers they are published as. */
static void lsrk_coefficients(real A[5], real B[5])
{
    A[0] = 0;
    A[1] = -(real)567301805773 / (real)1357537059087;
    A[2] = -(real)2404267990393 / (real)2016746695238;
    A[3] = -(real)3550918686646 / (real)2091501179385;
    A[4] = -(real)1275806237668 / (real)842570457699;
    B[0] = (real)1432997174477 / (real)9575080441755;
    B[1] = (real)5161836677717 / (real)13612068292357;
    B[2] = (real)1720146321549 / (real)2090206949498;
    B[3] = (real)3134564353537 / (real)4481467310338;
    B[4] = (real)2277821191437 / (real)14882151754819;
}

/* A right-hand side L(q) of n values, with its context. */
typedef void (*rhs_fn)(const real *q, real *L, void *ctx);

/* nsteps steps of size dt of dq/dt = L(q), in place on q[n]. */
static void lsrk_advance(real *q, int64_t n, real dt, int nsteps, rhs_fn L, void *ctx)
{
    real A[5], B[5];
    lsrk_coefficients(A, B);
    real *k = (real *)calloc((size_t)(n > 0 ? n : 1), sizeof(real));
    real *Lq = (real *)malloc((size_t)(n > 0 ? n : 1) * sizeof(real));
    for (int step = 0; step < nsteps; ++step) {
        for (int s = 0; s < 5; ++s) {
            L(q, Lq, ctx);
            for (int64_t i = 0; i < n; ++i) {
                k[i] = A[s] * k[i] + dt * Lq[i];
                q[i] = q[i] + B[s] * k[i];
            }
        }
    }
    free(k);
    free(Lq);
}

/* The published coefficients, rounded to double (for the tests). */
void oracle_lsrk_coefficients(double A[5], double B[5])
{
    real a[5], b[5];
    lsrk_coefficients(a, b);
    for (int s = 0; s < 5; ++s) {
        A[s] = (double)a[s];
        B[s] = (double)b[s];
    }
}

/* The stepper on a user ODE dy/dt = f(y) (double callback), for the tests
 * that pin the scheme's order on problems with known solutions. */
typedef void (*oracle_ode_fn)(const double *y, double *dydt, int64_t n);

typedef struct {
    oracle_ode_fn f;
    int64_t n;
    double *y, *dy;
} ode_ctx;

static void ode_rhs(const real *q, real *L, void *vctx)
{
    ode_ctx *c = (ode_ctx *)vctx;
    demote(q, c->n, c->y);
    c->f(c->y, c->dy, c->n);
    for (int64_t i = 0; i < c->n; ++i) L[i] = c->dy[i];
}

int oracle_lsrk_ode(double *y, int64_t n, double dt, int nsteps, oracle_ode_fn f)
{
    if (n < 1 || nsteps < 0 || !f) return -1;
    ode_ctx c = {f, n, (double *)malloc((size_t)n * sizeof(double)),
                 (double *)malloc((size_t)n * sizeof(double))};
    real *q = promote(y, n);
    lsrk_advance(q, n, dt, nsteps, ode_rhs, &c);
    demote(q, n, y);
    free(q);
    free(c.y);
    free(c.dy);
    return 0;
}

/* The whole right-hand side of Eq. 2 as the stepped operator. */
typedef struct {
    const double *phi, *geom, *D, *omega;
    const int32_t *nbr;
    int N, nthreads;
    int64_t nelem;
} esdg_ctx;

static void esdg_rhs(const real *q, real *L, void *vctx)
{
    const esdg_ctx *c = (const esdg_ctx *)vctx;
    volume_rhs_r(q, c->phi, c->geom, c->D, c->N, c->nelem, L, NULL, c->nthreads);
    surface_rhs_r(q, c->phi, c->geom, c->nbr, c->N, c->nelem, L, NULL, c->nthreads);
    if (c->omega) {
        const int64_t Np = (int64_t)(c->N + 1) * (c->N + 1) * (c->N + 1);
        add_coriolis_r(q, c->omega, c->nelem * Np, L);
    }
}

/* nsteps steps of size dt of dq/dt = rhs(q) (volume + surface + Coriolis,
 * omega NULL for none), in place on q [5][nelem][Np].
 * Returns 0, -1 on bad sizes, -2 on a bad neighbour index. */
int oracle_lsrk_esdg(double *q, const double *phi, const double *geom, const double *D,
                     const int32_t *nbr, const double *omega, int N, int64_t nelem, double dt,
                     int nsteps, int nthreads)
{
    if (N < 1 || nelem < 0 || nsteps < 0) return -1;
    if (bad_neighbour(nbr, nelem)) return -2;
    const int64_t n = 5 * nelem * (int64_t)(N + 1) * (N + 1) * (N + 1);
    esdg_ctx c = {phi, geom, D, omega, nbr, N, nthreads, nelem};
    real *qr = promote(q, n);
    lsrk_advance(qr, n, dt, nsteps, esdg_rhs, &c);
    demote(qr, n, q);
    free(qr);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Global integrals of [ESDG-GPU §5.2]: out[0] = sum of the integrals of rho,
 * out[1] of total energy E (= rho e, e including phi), out[2] of the entropy
 * eta = -rho s/(gamma-1), s = ln p - gamma ln rho, by the LGL quadrature:
 * weight w[a] w[b] w[c] J at node a + Nq (b + Nq c).  Plain sums in element
 * and node order.  Returns 0, or -1 on bad sizes. */
int oracle_integrals(const double *q, const double *phi, const double *geom, const double *w,
                     int N, int64_t nelem, double out[3])
{
    if (N < 1 || nelem < 0) return -1;
    const int Nq = N + 1;
    const int64_t Np = (int64_t)Nq * Nq * Nq;
    const int64_t stride = nelem * Np;
    real mass = 0, energy = 0, entropy = 0;
    for (int64_t e = 0; e < nelem; ++e)
        for (int c = 0; c < Nq; ++c)
        for (int b = 0; b < Nq; ++b)
        for (int a = 0; a < Nq; ++a) {
            const int64_t i = a + Nq * (b + Nq * c);
            real qn[5];
            for (int f = 0; f < 5; ++f) qn[f] = q[f * stride + e * Np + i];
            const node_state s = read_node(qn, phi[e * Np + i]);
            const real wJ = (real)w[a] * (real)w[b] * (real)w[c] * (real)geom[9 * stride + e * Np + i];
            const real ent = RLOG(s.p) - ORACLE_GAMMA * RLOG(s.rho);
            mass += wJ * qn[0];
            energy += wJ * qn[4];
            entropy += wJ * (-s.rho * ent / (ORACLE_GAMMA - 1));
        }
    out[0] = (double)mass;
    out[1] = (double)energy;
    out[2] = (double)entropy;
    return 0;
}

/* ---------------------------------------------------------------------------
 * Perturbation variables about a reference state at rest ([ESDG-GPU §5.2,
 * last paragraph on the baroclinic test]: the state carried as its
 * difference from a reference state).  The reference is given by its density
 * and pressure, rbar and pbar, at rest, so its total energy is
 * Ebar = pbar/(gamma-1) + rbar phi.  The full state is
 *     rho = rbar + rho',  U = U',  E = Ebar + E'.
 * qp [5][n], ref [2][n] (rbar, pbar), phi [n] -> q [5][n]. */
void oracle_full_state(const double *qp, const double *ref, const double *phi, int64_t n,
                       double *q)
{
    for (int64_t i = 0; i < n; ++i) {
        const real rbar = ref[i], pbar = ref[n + i];
        const real Ebar = pbar / (ORACLE_GAMMA - 1) + rbar * (real)phi[i];
        q[i] = (double)(rbar + (real)qp[i]);
        for (int m = 1; m < 4; ++m) q[m * n + i] = qp[m * n + i];
        q[4 * n + i] = (double)(Ebar + (real)qp[4 * n + i]);
    }
}

/* Significand bits of the arithmetic type (64 for long double on x86-64, 53
 * for double). */
int oracle_mantissa_bits(void) { return REAL_MANT_DIG; }

/* Threads the OpenMP runtime would use by default (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
