// ablation.hip -- libesdg_ablation.so: the volume term of esdg.h computed by
// a ladder of thread-per-node kernels, one per step of the cumulative
// optimisation study of "GPU Performance of an Entropy-Stable Discontinuous
// Galerkin Euler Solver with Non-Conservative Terms" (§4.1, Fig. 1, Fig. 2,
// Eq. 6).  These kernels exist to be measured against the line-per-thread
// production kernel; see include/esdg_ablation.h for the variant list.
//
// Common structure: one workgroup per element, one thread per node
// (workgroup size rounded up to whole waves); node data staged in LDS; for
// direction k the thread walks its k-line.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "esdg.h"
#include "esdg_ablation.h"
#include "volume_kernel.hpp"

namespace esdg_abl {
using esdg::Arith;
using esdg::NodeRegs;
using esdg::kBScale;
using esdg::kGamma;

enum Variant {
    BASELINE = ESDG_ABL_BASELINE,
    HOIST = ESDG_ABL_HOIST,
    LOGMEAN = ESDG_ABL_LOGMEAN,
    CONTRA = ESDG_ABL_CONTRA,
    SYM_UPPER = ESDG_ABL_SYM_UPPER,
    SYM_INDEXED = ESDG_ABL_SYM_INDEXED,
    SYM_WEIGHTED = ESDG_ABL_SYM_WEIGHTED,
    FUSED = ESDG_ABL_FUSED,
};

template <int N>
struct Geo {
    static constexpr int Nq = N + 1, Nq2 = Nq * Nq, Np = Nq2 * Nq;
    static constexpr int NT = (Np + 63) / 64 * 64;
};

// LDS staging, field-major over the element's nodes.
//   conserved layout (BASELINE): q0..q4, phi, Ja (9), J
//   primitive layout (the rest): rho, u1, u2, u3, p, b, phi, Ja (9), J,
//                                then s_b b, ln rho, ln(s_b b), w, 1/(s_b b)
enum Cons { cQ = 0, cPhi = 5, cJa = 6, cJ = 15, kCons = 16 };
enum Prim { pRho = 0, pU = 1, pP = 4, pB = 5, pPhi = 6, pJa = 7, pJ = 16, pBs = 17, pLRho = 18,
            pLB = 19, pW = 20, pIB = 21, kPrim = 22 };

constexpr int kXch = 5;  // exchange slots per node (half-sweep variants)

__device__ inline double logmean_log1p(double am, double ap)
{
    // {{a}}_log evaluated per pair with its own logarithm (no hoisting)
    const double d = ap - am;
    return d == 0.0 ? am : d / log1p(d / am);
}

// Two-point flux matrix F_j (j = 0..2) of own node "m" and partner "p" from
// primitive values, log means per pair, contracted afterwards.
__device__ inline void flux_matrix(double rm, const double *um, double pm, double bm, double fm,
                                   double rp, const double *up, double pp, double bp, double fp,
                                   double F[3][5])
{
    const double ravg = 0.5 * (rm + rp), rlog = logmean_log1p(rm, rp);
    const double bavg = 0.5 * (bm + bp), blog = logmean_log1p(bm, bp);
    double uavg[3];
    for (int m = 0; m < 3; ++m) uavg[m] = 0.5 * (um[m] + up[m]);
    const double usq = 0.5 * ((um[0] * um[0] + um[1] * um[1] + um[2] * um[2]) +
                              (up[0] * up[0] + up[1] * up[1] + up[2] * up[2]));
    const double phiavg = 0.5 * (fm + fp), dphi = fp - fm;
    const double ptil = ravg / (2.0 * bavg);
    const double rhat = bavg * rlog / bm;
    (void)pm;
    (void)pp;
    for (int j = 0; j < 3; ++j) {
        const double Fr = rlog * uavg[j];
        F[j][0] = Fr;
        double FE = (1.0 / (2.0 * (kGamma - 1.0) * blog) - 0.5 * usq + phiavg) * Fr;
        for (int m = 0; m < 3; ++m) {
            double sym = Fr * uavg[m];
            if (m == j) sym += ptil;
            FE += uavg[m] * sym;
            F[j][1 + m] = sym + (m == j ? 0.5 * rhat * dphi : 0.0);
        }
        F[j][4] = FE;
    }
}

// Flux matrix with logs hoisted per node and the series log mean (LOGMEAN).
// xm, xp: the own and partner node's first staged value (value v at v * Np).
template <int Np>
__device__ inline void flux_matrix_series(const double *xm, const double *xp, double F[3][5])
{
    using A = Arith<double>;
    const double eps = A::kSeries;
    const double rm = xm[pRho * Np], rp = xp[pRho * Np], bm = xm[pBs * Np], bp = xp[pBs * Np];
    const double sr = rm + rp, dr = rp - rm, sb = bm + bp, db = bp - bm;
    // log means as in the page's efficient form: series near equality, else
    // the quotient of hoisted log differences (separate divisions here)
    const double fr = (dr / sr) * (dr / sr);
    const double fb = (db / sb) * (db / sb);
    const double rlog = fabs(dr) < eps * sr
        ? sr * fma(fma(fma(-22.0 / 945.0, fr, -2.0 / 45.0), fr, -1.0 / 6.0), fr, 0.5)
        : dr / (xp[pLRho * Np] - xm[pLRho * Np]);
    const double blog_s = fabs(db) < eps * sb
        ? sb / fma(fma(fma(2.0 / 7.0, fb, 2.0 / 5.0), fb, 2.0 / 3.0), fb, 2.0)
        : db / (xp[pLB * Np] - xm[pLB * Np]);
    const double blog = blog_s / kBScale;
    double uavg[3];
    for (int m = 0; m < 3; ++m) uavg[m] = 0.5 * (xm[(pU + m) * Np] + xp[(pU + m) * Np]);
    const double wavg = 0.5 * (xm[pW * Np] + xp[pW * Np]);
    const double ravg = 0.5 * sr, bavg = 0.5 * (xm[pB * Np] + xp[pB * Np]);
    const double ptil = ravg / (2.0 * bavg);
    const double rhat = bavg * rlog / xm[pB * Np];
    const double dphi = xp[pPhi * Np] - xm[pPhi * Np];
    for (int j = 0; j < 3; ++j) {
        const double Fr = rlog * uavg[j];
        F[j][0] = Fr;
        double FE = (1.0 / (2.0 * (kGamma - 1.0) * blog) + wavg) * Fr;
        for (int m = 0; m < 3; ++m) {
            double sym = Fr * uavg[m];
            if (m == j) sym += ptil;
            FE += uavg[m] * sym;
            F[j][1 + m] = sym + (m == j ? 0.5 * rhat * dphi : 0.0);
        }
        F[j][4] = FE;
    }
}

template <int N>
__device__ inline void stage(const double *__restrict__ q, const double *__restrict__ phi,
                             const double *__restrict__ geom, int64_t e, int64_t fstride,
                             int variant, double *lds)
{
    using G = Geo<N>;
    using A = Arith<double>;
    const int t = threadIdx.x;
    if (t >= G::Np) return;
    const int64_t g = e * G::Np + t;
    if (variant == BASELINE) {
        for (int f = 0; f < 5; ++f) lds[(cQ + f) * G::Np + t] = q[f * fstride + g];
        lds[cPhi * G::Np + t] = phi[g];
        for (int m = 0; m < 9; ++m) lds[(cJa + m) * G::Np + t] = geom[m * fstride + g];
        lds[cJ * G::Np + t] = geom[9 * fstride + g];
        return;
    }
    const double rho = q[g], E = q[4 * fstride + g], ph = phi[g];
    const double u1 = q[fstride + g] / rho, u2 = q[2 * fstride + g] / rho, u3 = q[3 * fstride + g] / rho;
    const double usq = u1 * u1 + u2 * u2 + u3 * u3;
    const double p = (kGamma - 1.0) * (E - 0.5 * rho * usq - rho * ph);
    const double b = rho / (2.0 * p);
    lds[pRho * G::Np + t] = rho;
    lds[(pU + 0) * G::Np + t] = u1;
    lds[(pU + 1) * G::Np + t] = u2;
    lds[(pU + 2) * G::Np + t] = u3;
    lds[pP * G::Np + t] = p;
    lds[pB * G::Np + t] = b;
    lds[pPhi * G::Np + t] = ph;
    for (int m = 0; m < 9; ++m) lds[(pJa + m) * G::Np + t] = geom[m * fstride + g];
    lds[pJ * G::Np + t] = geom[9 * fstride + g];
    if (variant >= LOGMEAN) {
        // b is scaled by 2^17 for its log; the rungs that call the production
        // pair routine stage 2b (and 1/(2b)) as it expects
        const double bs = (variant >= CONTRA ? esdg::kBStage : kBScale) * b;
        lds[pBs * G::Np + t] = bs;
        lds[pLRho * G::Np + t] = A::node_log(rho);
        lds[pLB * G::Np + t] = A::node_log(kBScale * b);
        lds[pW * G::Np + t] = ph - 0.5 * usq;
        lds[pIB * G::Np + t] = 1.0 / bs;
    }
    if (variant >= CONTRA) {
        // the production pair routine takes u/2, w/2 and phi/4
        for (int m = 0; m < 3; ++m) lds[(pU + m) * G::Np + t] *= 0.5;
        lds[pW * G::Np + t] *= 0.5;
        lds[pPhi * G::Np + t] *= 0.25;
    }
}

// NodeRegs of the production pair math, read from the primitive layout (for
// these rungs u, w and phi are staged as u/2, w/2 and phi/4).
template <int N>
__device__ inline NodeRegs<double> node_regs(const double *lds, int s, int k)
{
    using G = Geo<N>;
    NodeRegs<double> X;
    X.rho = lds[pRho * G::Np + s];
    X.u1 = lds[(pU + 0) * G::Np + s];
    X.u2 = lds[(pU + 1) * G::Np + s];
    X.u3 = lds[(pU + 2) * G::Np + s];
    X.b = lds[pBs * G::Np + s];
    X.lrho = lds[pLRho * G::Np + s];
    X.lb = lds[pLB * G::Np + s];
    X.ph = lds[pPhi * G::Np + s];
    X.w = lds[pW * G::Np + s];
    X.ib = lds[pIB * G::Np + s];
    X.n1 = lds[(pJa + 3 * k + 0) * G::Np + s];
    X.n2 = lds[(pJa + 3 * k + 1) * G::Np + s];
    X.n3 = lds[(pJa + 3 * k + 2) * G::Np + s];
    return X;
}

// Own contribution of every ordered pair on the k-line (variants 0..3).
template <int N>
__device__ inline void ordered_pairs(const double *lds, const double *__restrict__ D, int variant,
                                     int k, int s0, int ik, int stride, double acc[5])
{
    using G = Geo<N>;
    constexpr int Nq = G::Nq;
    for (int l = 0; l < Nq; ++l) {
        if (l == ik) continue;
        const int sl = s0 + (l - ik) * stride;
        const double Dal = D[ik * Nq + l];
        if (variant == BASELINE || variant == HOIST) {
            double rm, rp, pm, pp, bm, bp, fm, fp, um[3], up[3];
            if (variant == BASELINE) {
                // primitives recomputed from the conserved variables per pair
                rm = lds[cQ * G::Np + s0];
                rp = lds[cQ * G::Np + sl];
                for (int m = 0; m < 3; ++m) {
                    um[m] = lds[(cQ + 1 + m) * G::Np + s0] / rm;
                    up[m] = lds[(cQ + 1 + m) * G::Np + sl] / rp;
                }
                fm = lds[cPhi * G::Np + s0];
                fp = lds[cPhi * G::Np + sl];
                pm = (kGamma - 1.0) * (lds[(cQ + 4) * G::Np + s0] -
                                       0.5 * rm * (um[0] * um[0] + um[1] * um[1] + um[2] * um[2]) - rm * fm);
                pp = (kGamma - 1.0) * (lds[(cQ + 4) * G::Np + sl] -
                                       0.5 * rp * (up[0] * up[0] + up[1] * up[1] + up[2] * up[2]) - rp * fp);
                bm = rm / (2.0 * pm);
                bp = rp / (2.0 * pp);
            } else {
                rm = lds[pRho * G::Np + s0];
                rp = lds[pRho * G::Np + sl];
                for (int m = 0; m < 3; ++m) {
                    um[m] = lds[(pU + m) * G::Np + s0];
                    up[m] = lds[(pU + m) * G::Np + sl];
                }
                pm = lds[pP * G::Np + s0];
                pp = lds[pP * G::Np + sl];
                bm = lds[pB * G::Np + s0];
                bp = lds[pB * G::Np + sl];
                fm = lds[pPhi * G::Np + s0];
                fp = lds[pPhi * G::Np + sl];
            }
            double F[3][5];
            flux_matrix(rm, um, pm, bm, fm, rp, up, pp, bp, fp, F);
            const int ja = variant == BASELINE ? cJa : pJa;
            for (int j = 0; j < 3; ++j) {
                const double nj = lds[(ja + 3 * k + j) * G::Np + s0] + lds[(ja + 3 * k + j) * G::Np + sl];
                for (int f = 0; f < 5; ++f) acc[f] = fma(Dal * nj, F[j][f], acc[f]);
            }
        } else if (variant == LOGMEAN) {
            double F[3][5];
            flux_matrix_series<G::Np>(lds + s0, lds + sl, F);
            for (int j = 0; j < 3; ++j) {
                const double nj = lds[(pJa + 3 * k + j) * G::Np + s0] + lds[(pJa + 3 * k + j) * G::Np + sl];
                for (int f = 0; f < 5; ++f) acc[f] = fma(Dal * nj, F[j][f], acc[f]);
            }
        } else {  // CONTRA: the production pair math, own contribution only
            double unused[5] = {0, 0, 0, 0, 0};
            esdg::pair_update(node_regs<N>(lds, s0, k), node_regs<N>(lds, sl, k), D + ik * Nq + l,
                              D + l * Nq + ik, acc, unused);
        }
    }
}

// Half-sweep along the k-line with LDS exchange of the partner contribution
// (variants 4..7).  Step s pairs own index a with (a + s) mod Nq; which
// threads work at step s, and with what weight, is the schedule.
template <int N>
__device__ inline void half_sweep(double *lds, double *xch, const double *__restrict__ D,
                                  int variant, int k, int s0, int ik, int stride, bool node,
                                  double acc[5])
{
    constexpr int Nq = Geo<N>::Nq;
    constexpr bool even = (Nq % 2) == 0;
    const int nsteps = (variant == SYM_UPPER) ? Nq - 1 : Nq / 2;
    for (int s = 1; s <= nsteps; ++s) {
        const int l = (ik + s) % Nq;  // partner line index
        bool work;
        double w = 1.0;
        if (variant == SYM_UPPER) {
            work = ik + s < Nq;
        } else if (variant == SYM_INDEXED) {
            // Eq. 6: for even Nq the antipodal step is done by the first half only
            work = !(even && s == Nq / 2 && ik >= Nq / 2);
        } else {  // weighted: everyone works; antipodal pairs at weight 1/2
            work = true;
            if (even && s == Nq / 2) w = 0.5;
        }
        double out[5] = {0, 0, 0, 0, 0};
        if (node && work) {
            const int sl = s0 + (l - ik) * stride;
            const double Dal = w * D[ik * Nq + l];
            const double Dla = w * D[l * Nq + ik];
            esdg::pair_update(node_regs<N>(lds, s0, k), node_regs<N>(lds, sl, k), &Dal, &Dla, acc,
                              out);
            for (int f = 0; f < 5; ++f) xch[f * Geo<N>::Np + sl] = out[f];
        }
        __syncthreads();
        // did the thread at index ik - s send to me this step?
        const int from = (ik - s + Nq) % Nq;
        bool recv;
        if (variant == SYM_UPPER) recv = ik - s >= 0;
        else if (variant == SYM_INDEXED) recv = !(even && s == Nq / 2 && from >= Nq / 2);
        else recv = true;
        if (node && recv)
            for (int f = 0; f < 5; ++f) acc[f] += xch[f * Geo<N>::Np + s0];
        __syncthreads();
    }
}

// One kernel per (order, variant): the variant is a template constant, so
// every rung is compiled on its own (registers, LDS and branches of the
// other rungs do not leak into it).
template <int N, int variant, bool FUSE>
__global__ void __launch_bounds__(Geo<N>::NT)
ablation_kernel(int k_only, const double *__restrict__ q, const double *__restrict__ phi,
                const double *__restrict__ geom, const double *__restrict__ D, int64_t nelem,
                double *__restrict__ rhs)
{
    using G = Geo<N>;
    constexpr int Nq = G::Nq, Nq2 = G::Nq2, Np = G::Np;
    // staged values: the conserved layout, the primitive layout without or
    // with the per-node logs; the exchange slots only for the half-sweeps
    constexpr int kStaged = variant == BASELINE ? kCons : variant == HOIST ? pBs : kPrim;
    __shared__ double lds[kStaged * Np];
    __shared__ double xch[variant >= SYM_UPPER ? kXch * Np : 1];
    const int64_t e = blockIdx.x;
    const int64_t fstride = nelem * Np;
    stage<N>(q, phi, geom, e, fstride, variant, lds);
    __syncthreads();

    const int t = threadIdx.x;
    const bool node = t < Np;
    const int a = t % Nq, b = (t / Nq) % Nq, c = t / Nq2;
    double acc[5] = {0, 0, 0, 0, 0};
    const int k0 = FUSE ? 0 : k_only, k1 = FUSE ? 3 : k_only + 1;
    for (int k = k0; k < k1; ++k) {
        const int ik = (k == 0) ? a : (k == 1) ? b : c;
        const int stride = (k == 0) ? 1 : (k == 1) ? Nq : Nq2;
        if constexpr (variant <= CONTRA) {
            if (node) ordered_pairs<N>(lds, D, variant, k, t, ik, stride, acc);
        } else {
            half_sweep<N>(lds, xch, D, variant, k, t, ik, stride, node, acc);
        }
    }
    if (node) {
        const int64_t g = e * Np + t;
        const double J = lds[(variant == BASELINE ? cJ : pJ) * Np + t];
        for (int f = 0; f < 5; ++f) {
            const double v = -acc[f] / J;
            rhs[f * fstride + g] = (FUSE || k_only == 0) ? v : rhs[f * fstride + g] + v;
        }
    }
}

template <int N, int V, bool FUSE>
int launch_variant(const double *q, const double *phi, const double *geom, const double *D,
                   int64_t nelem, double *rhs, hipStream_t stream)
{
    // one workgroup per element; one launch per direction unless fused
    const int launches = FUSE ? 1 : 3;
    for (int k = 0; k < launches; ++k) {
        hipLaunchKernelGGL((ablation_kernel<N, V, FUSE>), dim3((unsigned)nelem), dim3(Geo<N>::NT),
                           0, stream, k, q, phi, geom, D, nelem, rhs);
        if (hipGetLastError() != hipSuccess) return ESDG_ERR_LAUNCH;
    }
    return ESDG_OK;
}

template <int N, int V>
int launch_rung(bool fuse, const double *q, const double *phi, const double *geom,
                const double *D, int64_t nelem, double *rhs, hipStream_t stream)
{
    if (V == FUSED || fuse) return launch_variant<N, V, true>(q, phi, geom, D, nelem, rhs, stream);
    return launch_variant<N, V, false>(q, phi, geom, D, nelem, rhs, stream);
}

template <int N>
int launch(int variant, bool fuse, const double *q, const double *phi, const double *geom,
           const double *D, int64_t nelem, double *rhs, hipStream_t stream)
{
    switch (variant) {
        case BASELINE: return launch_rung<N, BASELINE>(fuse, q, phi, geom, D, nelem, rhs, stream);
        case HOIST: return launch_rung<N, HOIST>(fuse, q, phi, geom, D, nelem, rhs, stream);
        case LOGMEAN: return launch_rung<N, LOGMEAN>(fuse, q, phi, geom, D, nelem, rhs, stream);
        case CONTRA: return launch_rung<N, CONTRA>(fuse, q, phi, geom, D, nelem, rhs, stream);
        case SYM_UPPER: return launch_rung<N, SYM_UPPER>(fuse, q, phi, geom, D, nelem, rhs, stream);
        case SYM_INDEXED: return launch_rung<N, SYM_INDEXED>(fuse, q, phi, geom, D, nelem, rhs, stream);
        case SYM_WEIGHTED: return launch_rung<N, SYM_WEIGHTED>(fuse, q, phi, geom, D, nelem, rhs, stream);
        case FUSED: return launch_rung<N, FUSED>(true, q, phi, geom, D, nelem, rhs, stream);
    }
    return ESDG_ERR_VARIANT;
}

}  // namespace esdg_abl

extern "C" {

int esdg_ablation_volume_rhs_f64(int variant, const double *q, const double *phi,
                                 const double *geom, const double *D, int N, int64_t nelem,
                                 double *rhs, hipStream_t stream)
{
    const bool fuse = (variant & ESDG_ABL_FUSE_FLAG) != 0;
    variant &= ~ESDG_ABL_FUSE_FLAG;
    if (variant < 0 || variant >= ESDG_ABL_COUNT) return ESDG_ERR_VARIANT;
    if (N != 3 && N != 4 && N != 7) return ESDG_ERR_ORDER;
    if (nelem < 0) return ESDG_ERR_NELEM;
    if (nelem == 0) return ESDG_OK;
    if (!q || !phi || !geom || !D || !rhs) return ESDG_ERR_NULL;
    const int64_t Np = (int64_t)(N + 1) * (N + 1) * (N + 1);
    // one workgroup per element: the grid holds at most INT32_MAX of them
    // (which also keeps every byte count below in range)
    if (nelem > INT32_MAX) return ESDG_ERR_NELEM;
    const uintptr_t r0 = (uintptr_t)rhs, r1 = r0 + (uintptr_t)(5 * nelem * Np * 8);
    const uintptr_t in[4][2] = {{(uintptr_t)q, (uintptr_t)q + (uintptr_t)(5 * nelem * Np * 8)},
                                {(uintptr_t)phi, (uintptr_t)phi + (uintptr_t)(nelem * Np * 8)},
                                {(uintptr_t)geom, (uintptr_t)geom + (uintptr_t)(10 * nelem * Np * 8)},
                                {(uintptr_t)D, (uintptr_t)D + (uintptr_t)((N + 1) * (N + 1) * 8)}};
    for (int i = 0; i < 4; ++i)
        if (r0 < in[i][1] && in[i][0] < r1) return ESDG_ERR_ALIAS;
    switch (N) {
        case 3: return esdg_abl::launch<3>(variant, fuse, q, phi, geom, D, nelem, rhs, stream);
        case 4: return esdg_abl::launch<4>(variant, fuse, q, phi, geom, D, nelem, rhs, stream);
        case 7: return esdg_abl::launch<7>(variant, fuse, q, phi, geom, D, nelem, rhs, stream);
    }
    return ESDG_ERR_ORDER;
}

int esdg_ablation_two_lane_volume_rhs_f64(const double *q, const double *phi, const double *geom,
                                          const double *D, int N, int64_t nelem, double *rhs,
                                          hipStream_t stream)
{
    // LaunchCfg<EPB, NT, waves, metric in LDS, line cache, direction-major, FIN, series,
    // series (surface), row pad, plane pad, element pad, waves (surface), lanes per line>
    using C5 = esdg::LaunchCfg<1, 256, 3, false, false, 1, false, true, false, 0, 0, 0, 0, 2>;
    using C7 = esdg::LaunchCfg<1, 384, 3, false, false, 1, true, true, false, 1, 0, 0, 0, 2>;
    if (N != 5 && N != 7) return ESDG_ERR_ORDER;
    if (nelem < 0) return ESDG_ERR_NELEM;
    if (nelem == 0) return ESDG_OK;
    if (!q || !phi || !geom || !D || !rhs) return ESDG_ERR_NULL;
    if (nelem > INT32_MAX) return ESDG_ERR_NELEM;  // one workgroup per element
    const int64_t Np = (int64_t)(N + 1) * (N + 1) * (N + 1);
    const uintptr_t r0 = (uintptr_t)rhs, r1 = r0 + (uintptr_t)(5 * nelem * Np * 8);
    const uintptr_t in[4][2] = {{(uintptr_t)q, (uintptr_t)q + (uintptr_t)(5 * nelem * Np * 8)},
                                {(uintptr_t)phi, (uintptr_t)phi + (uintptr_t)(nelem * Np * 8)},
                                {(uintptr_t)geom, (uintptr_t)geom + (uintptr_t)(10 * nelem * Np * 8)},
                                {(uintptr_t)D, (uintptr_t)D + (uintptr_t)((N + 1) * (N + 1) * 8)}};
    for (int i = 0; i < 4; ++i)
        if (r0 < in[i][1] && in[i][0] < r1) return ESDG_ERR_ALIAS;
    const esdg::Rotation<double> rot{0.0, 0.0, 0.0, false};
    const esdg::Sink<double, false> sink{rhs, nullptr, 0.0, 0.0, 0.0};
    if (N == 5)
        hipLaunchKernelGGL((esdg::volume_rhs_kernel<double, 5, C5>), dim3((unsigned)nelem),
                           dim3(C5::NT), 0, stream, q, nullptr, phi, geom, D, nullptr, rot, nelem,
                           sink);
    else
        hipLaunchKernelGGL((esdg::volume_rhs_kernel<double, 7, C7>), dim3((unsigned)nelem),
                           dim3(C7::NT), 0, stream, q, nullptr, phi, geom, D, nullptr, rot, nelem,
                           sink);
    return hipGetLastError() == hipSuccess ? ESDG_OK : ESDG_ERR_LAUNCH;
}

const char *esdg_ablation_name(int variant)
{
    if (variant & ESDG_ABL_FUSE_FLAG) {
        switch (variant & ~ESDG_ABL_FUSE_FLAG) {
            case ESDG_ABL_BASELINE: return "baseline, fused directions";
            case ESDG_ABL_HOIST: return "hoisted primitives, fused directions";
            case ESDG_ABL_LOGMEAN: return "per-node logs, series log mean, fused directions";
            case ESDG_ABL_CONTRA: return "contravariant flux, inverse log mean, fused directions";
            case ESDG_ABL_SYM_UPPER: return "half-sweep, upper-triangular, fused directions";
            case ESDG_ABL_SYM_INDEXED: return "half-sweep, cyclic indexing (Eq. 6), fused directions";
            case ESDG_ABL_SYM_WEIGHTED:
            case ESDG_ABL_FUSED: return "weighted cyclic, fused directions";
        }
        return "unknown";
    }
    switch (variant) {
        case ESDG_ABL_BASELINE: return "baseline";
        case ESDG_ABL_HOIST: return "hoisted primitives";
        case ESDG_ABL_LOGMEAN: return "per-node logs, series log mean";
        case ESDG_ABL_CONTRA: return "contravariant flux, inverse log mean";
        case ESDG_ABL_SYM_UPPER: return "half-sweep, upper-triangular";
        case ESDG_ABL_SYM_INDEXED: return "half-sweep, cyclic indexing (Eq. 6)";
        case ESDG_ABL_SYM_WEIGHTED: return "half-sweep, weighted cyclic";
        case ESDG_ABL_FUSED: return "weighted cyclic, fused directions";
    }
    return "unknown";
}

}  // extern "C"
