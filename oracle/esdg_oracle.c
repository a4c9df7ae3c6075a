/*
 * esdg_oracle.c -- plain, slow CPU oracle of the ESDG flux-differencing
 * volume term, in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file: only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header, table or constant with the HIP
 * library; it receives the same seeded input arrays and nothing else.
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
 *   - gamma = 1.4.
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
 * Every ordered pair is evaluated on its own: no symmetry, no hoisting, no
 * reuse.  That is the plain definition of what the volume term computes.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static const double ORACLE_GAMMA = 1.4;

/* State at one node, read off the conserved variables. */
typedef struct {
    double rho;
    double u[3];
    double usq;  /* |u|^2 */
    double p;
    double b;    /* rho / (2 p) */
    double phi;
} node_state;

/* Pressure law of [ESDG-GPU §2]: P = (gamma-1)(E - U.U/(2 rho) - rho phi). */
static node_state read_node(const double q[5], double phi)
{
    node_state s;
    s.rho = q[0];
    s.u[0] = q[1] / q[0];
    s.u[1] = q[2] / q[0];
    s.u[2] = q[3] / q[0];
    s.usq = s.u[0] * s.u[0] + s.u[1] * s.u[1] + s.u[2] * s.u[2];
    double UU = q[1] * q[1] + q[2] * q[2] + q[3] * q[3];
    s.p = (ORACLE_GAMMA - 1.0) * (q[4] - UU / (2.0 * q[0]) - q[0] * phi);
    s.b = q[0] / (2.0 * s.p);
    s.phi = phi;
    return s;
}

/* {{a}} of [ESDG-GPU §4.1, Eq. 3]. */
static double avg(double am, double ap) { return 0.5 * (am + ap); }

/* {{a}}_log of [ESDG-GPU §4.1, Eq. 3]: (a+ - a-)/(log a+ - log a-), with the
 * limit a- when the two are equal.  Written as d / log1p(d/a-), d = a+ - a-,
 * which is the same quotient and is accurate for nearby arguments. */
static double logmean(double am, double ap)
{
    double d = ap - am;
    if (d == 0.0) return am;
    return d / log1p(d / am);
}

/* Two-point flux F_j(q_i, q_l) in physical direction j (0, 1, 2), with the
 * own node i as the "-" state and the partner l as the "+" state. */
static void ec_flux(const node_state *si, const node_state *sl, int j, double F[5])
{
    double rho_avg = avg(si->rho, sl->rho);
    double rho_log = logmean(si->rho, sl->rho);
    double b_avg = avg(si->b, sl->b);
    double b_log = logmean(si->b, sl->b);
    double u_avg[3];
    for (int m = 0; m < 3; ++m) u_avg[m] = avg(si->u[m], sl->u[m]);
    double usq_avg = avg(si->usq, sl->usq);
    double phi_avg = avg(si->phi, sl->phi);
    double phi_jump = sl->phi - si->phi;

    double p_tilde = rho_avg / (2.0 * b_avg);          /* {{rho}}/(2{{b}}), Eq. 4 */
    double rho_hat = b_avg * rho_log / si->b;           /* Eq. 5 */

    double Frho = rho_log * u_avg[j];
    F[0] = Frho;
    for (int m = 0; m < 3; ++m) {
        double Fm = Frho * u_avg[m];
        if (m == j) Fm += p_tilde + 0.5 * rho_hat * phi_jump;   /* Eq. 4 */
        F[1 + m] = Fm;
    }
    double FE = (1.0 / (2.0 * (ORACLE_GAMMA - 1.0) * b_log) - 0.5 * usq_avg + phi_avg) * Frho;
    for (int m = 0; m < 3; ++m) {
        double sym = Frho * u_avg[m];
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
        node_state si = read_node(qi + 5 * n, phii[n]);
        node_state sl = read_node(ql + 5 * n, phil[n]);
        ec_flux(&si, &sl, j, F + 5 * n);
    }
}

/* Primitive state per node, for the tests: out[n][6] = rho, u1, u2, u3, p, b. */
void oracle_node_state(const double *q /* [n][5] */, const double *phi, int64_t n_nodes,
                       double *out)
{
    for (int64_t n = 0; n < n_nodes; ++n) {
        node_state s = read_node(q + 5 * n, phi[n]);
        out[6 * n + 0] = s.rho;
        out[6 * n + 1] = s.u[0];
        out[6 * n + 2] = s.u[1];
        out[6 * n + 3] = s.u[2];
        out[6 * n + 4] = s.p;
        out[6 * n + 5] = s.b;
    }
}

/*
 * Volume term of Eq. 2 (reading above) on every element.
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
 * Node index n = a + Nq (b + Nq c).  Returns 0, or -1 on bad sizes.
 */
int oracle_volume_rhs(const double *q, const double *phi, const double *geom,
                      const double *D, int N, int64_t nelem, double *rhs, double *mag,
                      int nthreads)
{
    if (N < 1 || nelem < 0) return -1;
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
            double qn[5];
            for (int f = 0; f < 5; ++f) qn[f] = q[f * stride + e * Np + n];
            st[n] = read_node(qn, phi[e * Np + n]);
        }
        for (int c = 0; c < Nq; ++c)
        for (int b = 0; b < Nq; ++b)
        for (int a = 0; a < Nq; ++a) {
            const int64_t i = a + Nq * (b + Nq * c);
            const double Ji = geom[9 * stride + e * Np + i];
            double acc[5] = {0, 0, 0, 0, 0};
            double absacc[5] = {0, 0, 0, 0, 0};
            for (int k = 0; k < 3; ++k) {
                const int ik = (k == 0) ? a : (k == 1) ? b : c;
                for (int l = 0; l < Nq; ++l) {
                    if (l == ik) continue; /* diagonal pairs omitted */
                    const int64_t il = (k == 0) ? l + Nq * (b + Nq * c)
                                     : (k == 1) ? a + Nq * (l + Nq * c)
                                                : a + Nq * (b + Nq * l);
                    double term[5] = {0, 0, 0, 0, 0};
                    for (int j = 0; j < 3; ++j) {
                        const double nj = geom[(3 * k + j) * stride + e * Np + i]
                                        + geom[(3 * k + j) * stride + e * Np + il];
                        double F[5];
                        ec_flux(&st[i], &st[il], j, F);
                        for (int f = 0; f < 5; ++f) term[f] += nj * F[f];
                    }
                    const double d = D[ik * Nq + l];
                    for (int f = 0; f < 5; ++f) {
                        acc[f] += d * term[f];
                        absacc[f] += fabs(d * term[f]);
                    }
                }
            }
            for (int f = 0; f < 5; ++f) {
                rhs[f * stride + e * Np + i] = -acc[f] / Ji;
                if (mag) mag[f * stride + e * Np + i] = absacc[f] / fabs(Ji);
            }
        }
        free(st);
    }
    return 0;
}

/*
 * Surface term of Eq. 2 with the entropy-conservative flux (readings above),
 * ADDED to rhs (and, if mag is not NULL, its absolute value to mag).
 *
 *   nbr [nelem][6]  neighbour across faces -xi1, +xi1, -xi2, +xi2, -xi3,
 *                   +xi3; -1 = slip wall
 *
 * Returns 0, -1 on bad sizes, -2 if a neighbour index is outside [-1, nelem).
 */
int oracle_surface_rhs(const double *q, const double *phi, const double *geom,
                       const int32_t *nbr, int N, int64_t nelem, double *rhs, double *mag,
                       int nthreads)
{
    if (N < 1 || nelem < 0) return -1;
    for (int64_t i = 0; i < 6 * nelem; ++i)
        if (nbr[i] < -1 || nbr[i] >= nelem) return -2;
    const int Nq = N + 1;
    const int64_t Np = (int64_t)Nq * Nq * Nq;
    const int64_t stride = nelem * Np;
    const double w_end = 2.0 / ((double)N * (double)(N + 1));  /* LGL weight of xi = +-1 */
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
            double qi[5];
            for (int f = 0; f < 5; ++f) qi[f] = q[f * stride + e * Np + i];
            const node_state si = read_node(qi, phi[e * Np + i]);
            const double Ji = geom[9 * stride + e * Np + i];
            for (int k = 0; k < 3; ++k) {
                const int ik = (k == 0) ? a : (k == 1) ? b : c;
                if (ik != 0 && ik != N) continue;  /* not on a xi_k face */
                const int side = (ik == N) ? 1 : -1;
                const int32_t nb = nbr[6 * e + 2 * k + (side > 0 ? 1 : 0)];
                double n[3];
                for (int j = 0; j < 3; ++j) n[j] = geom[(3 * k + j) * stride + e * Np + i];
                node_state sp;
                if (nb < 0) {
                    /* mirror state across the face */
                    sp = si;
                    const double un = (si.u[0] * n[0] + si.u[1] * n[1] + si.u[2] * n[2])
                                    / (n[0] * n[0] + n[1] * n[1] + n[2] * n[2]);
                    for (int j = 0; j < 3; ++j) sp.u[j] = si.u[j] - 2.0 * un * n[j];
                    sp.usq = sp.u[0] * sp.u[0] + sp.u[1] * sp.u[1] + sp.u[2] * sp.u[2];
                } else {
                    const int jk = N - ik;  /* matching node on the neighbour's opposite face */
                    const int64_t ip = (k == 0) ? jk + Nq * (b + Nq * c)
                                     : (k == 1) ? a + Nq * (jk + Nq * c)
                                                : a + Nq * (b + Nq * jk);
                    double qp[5];
                    for (int f = 0; f < 5; ++f) qp[f] = q[f * stride + (int64_t)nb * Np + ip];
                    sp = read_node(qp, phi[(int64_t)nb * Np + ip]);
                }
                double term[5] = {0, 0, 0, 0, 0};
                for (int j = 0; j < 3; ++j) {
                    double F[5];
                    ec_flux(&si, &sp, j, F);
                    for (int f = 0; f < 5; ++f) term[f] += n[j] * F[f];
                }
                for (int f = 0; f < 5; ++f) {
                    const double v = (double)side * term[f] / (w_end * Ji);
                    rhs[f * stride + e * Np + i] -= v;
                    if (mag) mag[f * stride + e * Np + i] += fabs(v);
                }
            }
        }
    }
    return 0;
}

/*
 * Source term h of Eq. 2 from the Coriolis term of Eq. 1b: h = -omega x U on
 * the momentum components, U = (q1, q2, q3) the momentum, omega the rotation
 * vector as Eq. 1b writes it (for a planet rotating at Omega it is 2 Omega).
 * ADDED to rhs at every node; density and energy get nothing.
 */
void oracle_add_coriolis(const double *q, const double omega[3], int64_t nnodes, double *rhs)
{
    const int64_t stride = nnodes;
    for (int64_t n = 0; n < nnodes; ++n) {
        const double U[3] = {q[1 * stride + n], q[2 * stride + n], q[3 * stride + n]};
        const double wxU[3] = {omega[1] * U[2] - omega[2] * U[1],
                               omega[2] * U[0] - omega[0] * U[2],
                               omega[0] * U[1] - omega[1] * U[0]};
        for (int m = 0; m < 3; ++m) rhs[(1 + m) * stride + n] -= wxU[m];
    }
}

/* Threads the OpenMP runtime would use by default (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
