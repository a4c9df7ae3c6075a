// integrals_kernel.hpp -- global conservation integrals of the ESDG state and
// the plain device copy the time stepper uses, for AMD CDNA4 (gfx950).
//
// Page: "GPU Performance of an Entropy-Stable Discontinuous Galerkin Euler
// Solver with Non-Conservative Terms" (arXiv 2605.16684v2), [ESDG-GPU].
//
//   sum over elements of the integrals of rho, of rho e (= E, the total
//   energy with the geopotential) and of the entropy, tracked over time to
//   verify conservation ............................ [ESDG-GPU §5.2]
//
// The integrals use the LGL quadrature of the collocation nodes, weight
// w_a w_b w_c J at node (a, b, c); the entropy is eta = -rho s/(gamma-1) with
// s = ln p - gamma ln rho.  Every node's terms are formed and summed in fp64
// whatever the state's precision, so the drift of an fp32 state is measured
// on its stored values, not on the summation.  The sums are deterministic:
// a fixed grid of at most kIntegralBlocks workgroups, each summing a fixed
// set of nodes in a fixed order and reducing through LDS in a fixed tree,
// then one workgroup reducing the partial sums the same way.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace esdg {

constexpr int kIntegralBlocks = 1024;   // most partial sums one call writes
constexpr int kIntegralThreads = 256;

// Workgroup sum of three values per thread, in a fixed order; thread 0 gets
// the totals.
__device__ inline void block_sum3(double (&v)[3])
{
    __shared__ double red[3][kIntegralThreads];
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 3; ++i) red[i][t] = v[i];
    __syncthreads();
#pragma unroll
    for (int half = kIntegralThreads / 2; half > 0; half /= 2) {
        if (t < half) {
#pragma unroll
            for (int i = 0; i < 3; ++i) red[i][t] += red[i][t + half];
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) v[i] = red[i][0];
}

// Partial sums of block b over nodes b*256 + t + k*gridDim*256 of the whole
// mesh (nnodes = nelem Nq^3), written to part[3*b .. 3*b+2].  With PERT the
// state is carried as perturbation variables about the reference at rest
// ref = (rbar, pbar): rho = rbar + r, E = pbar/(gamma-1) + rbar phi + E'.
template <typename T, bool PERT>
__global__ void __launch_bounds__(kIntegralThreads)
integrals_partial_kernel(const T *__restrict__ q, const T *__restrict__ ref,
                         const T *__restrict__ phi, const T *__restrict__ geom,
                         const T *__restrict__ w, int Nq, int64_t nnodes,
                         double *__restrict__ part)
{
    const double gamma = 1.4, gm1 = gamma - 1.0;
    const int64_t Np = (int64_t)Nq * Nq * Nq;
    double acc[3] = {0.0, 0.0, 0.0};
    for (int64_t g = (int64_t)blockIdx.x * kIntegralThreads + threadIdx.x; g < nnodes;
         g += (int64_t)gridDim.x * kIntegralThreads) {
        const int n = (int)(g % Np);
        const int a = n % Nq, b = (n / Nq) % Nq, c = n / (Nq * Nq);
        const double wJ = (double)w[a] * (double)w[b] * (double)w[c] * (double)geom[9 * nnodes + g];
        const double ph = phi[g];
        double rho = q[g], E = q[4 * nnodes + g];
        if constexpr (PERT) {
            const double rbar = ref[g], pbar = ref[nnodes + g];
            E += pbar / gm1 + rbar * ph;
            rho += rbar;
        }
        const double m1 = q[nnodes + g], m2 = q[2 * nnodes + g], m3 = q[3 * nnodes + g];
        const double p = gm1 * (E - (m1 * m1 + m2 * m2 + m3 * m3) / (2.0 * rho) - rho * ph);
        const double s = log(p) - gamma * log(rho);
        acc[0] += wJ * rho;
        acc[1] += wJ * E;
        acc[2] += wJ * (-rho * s / gm1);
    }
    block_sum3(acc);
    if (threadIdx.x == 0) {
#pragma unroll
        for (int i = 0; i < 3; ++i) part[3 * blockIdx.x + i] = acc[i];
    }
}

// out[i] = sum over the nparts partial sums (one workgroup).
__global__ void __launch_bounds__(kIntegralThreads)
integrals_final_kernel(const double *__restrict__ part, int nparts, double *__restrict__ out)
{
    double acc[3] = {0.0, 0.0, 0.0};
    for (int b = threadIdx.x; b < nparts; b += kIntegralThreads) {
#pragma unroll
        for (int i = 0; i < 3; ++i) acc[i] += part[3 * b + i];
    }
    block_sum3(acc);
    if (threadIdx.x == 0) {
#pragma unroll
        for (int i = 0; i < 3; ++i) out[i] = acc[i];
    }
}

// dst[i] = src[i] for i < n.
template <typename T>
__global__ void __launch_bounds__(256) copy_kernel(const T *__restrict__ src, T *__restrict__ dst,
                                                   int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        dst[i] = src[i];
}

}  // namespace esdg
