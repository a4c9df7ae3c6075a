// volume_kernel.hpp -- fused flux-differencing volume kernel of the ESDG
// Euler-with-gravity discretisation, written for AMD CDNA4 (gfx950).
//
// Page: "GPU Performance of an Entropy-Stable Discontinuous Galerkin Euler
// Solver with Non-Conservative Terms" (arXiv 2605.16684v2), [ESDG-GPU].
//
//   volume term ....................... [ESDG-GPU §3, Eq. 2] (volume part, h = 0)
//   pressure law ...................... [ESDG-GPU §2]
//   means, log mean, jump ............. [ESDG-GPU §4.1, Eq. 3]
//   momentum flux and gravity ......... [ESDG-GPU §4.1, Eq. 4-5]
//   symmetric part S once per pair,
//   partner gravity G -> -G b-/b+ ..... [ESDG-GPU §4.1]
//   per-node primitives and logs,
//   log mean from separate logs ...... [ESDG-GPU §4.1]
//   contravariant flux built directly,
//   inverse log mean directly ......... [ESDG-GPU §4.1]
//   element data staged on chip,
//   three directions in one launch .... [ESDG-GPU §4.1]
//
// Work mapping (MI355X-specific; the pages map a thread to a node):
//   * A workgroup owns EPB consecutive elements.
//   * Phase A, one thread per node: coalesced SoA loads of the 5 conserved
//     fields and phi (non-temporal in the volume term alone, where nothing
//     reads them again); primitives, p, the staged 2b = rho/p, the logs of
//     rho and b and 1/(2b) are computed once per node and staged in LDS.
//     The metric terms Ja^k_j are either staged in LDS too or loaded by each
//     line thread for its own line straight into registers (a per-order
//     launch choice).
//   * Phase B, one thread per grid line (3 Nq^2 lines per element): every
//     unordered pair (a, l) of the line is evaluated once, with both nodes'
//     values read from LDS where the pair needs them:
//     the symmetric contravariant flux S~ serves both nodes, the gravity part
//     is g/b_a for node a and -g/b_l for node l.  Both contributions are
//     accumulated in registers, so there is no cross-thread scatter, no load
//     imbalance and no duplicated antipodal pair at any N.  Where every line
//     of a wave lies within the log means' series threshold (one wave vote,
//     a per-order launch option), the wave runs a second copy of the pair
//     loop without the log branch and its selects; both copies give the same
//     values.  Both copies are compiled into one kernel: where the launch
//     table asks for it, the general copy forms its pair metric sums with
//     different instructions, so that the compiler hoists nothing common to
//     both above the form branch (pair_update).
//   * LDS layout: field-major, one array per staged value over the node
//     grid of the workgroup's elements; per-order launch options pad that
//     grid (per row, plane or element) and start each direction's line
//     tasks on a 32-lane boundary, so that the lanes of a wave, each reading
//     one node of its own line, fall on different LDS banks, and may round
//     the arrays' stride to 64 slots so that two values of a node come with
//     one paired read.
//   * Phase C: each line writes its Nq x 5 partial sums to LDS (one array per
//     direction, every slot written by exactly one thread: no atomics, the
//     result is bitwise reproducible).
//   * Phase D, one thread per node: sum of the three directional partials,
//     scaling by -1/J, coalesced SoA store, non-temporal (or, with FIN, the
//     direction-3 line threads finish their own nodes).
//
// The whole right-hand side (SURF) reuses this kernel: a line's two end
// nodes lie on the element's two xi_k faces, so the line thread adds the
// entropy-conservative face flux with each end's partner in the neighbouring
// element (or the mirror state at a slip wall) to that end's accumulator
// ([ESDG-GPU §3, Eq. 2], surface part); the Coriolis source of Eq. 1b is
// added at the store, and a low-storage Runge-Kutta stage can be fused into
// that store (Sink).  The measurement probes launch the same kernel with
// phase marks (WallMarks); the library's instances take NoMarks, which
// compiles to nothing.
//
// On perturbation variables in fp32 (the page's cure for 32-bit noise,
// [ESDG-GPU §5.2]) the momentum flux's pressure mean is formed relative to
// each element's reference pressure, and the constant part is added once per
// line node in fp64 (pressure_reference): the same values in exact
// arithmetic, with the O(p) rounding of every pair taken out.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace esdg {

constexpr double kGamma = 1.4;
// b = rho/(2p) is O(1e-6) for air.  Logs of b are taken of s_b b with
// s_b = 2^17 (exact scaling), so they stay O(1) (this matters in fp32).
// The pairs work with the staged value 2b = rho/p: then a pair's pressure
// mean {{rho}}/(2{{b}}) is its density sum over its staged-b sum, with no
// constant factor.  {{s b}}_log = s {{b}}_log, so only constants change.
constexpr double kBScale = 131072.0;
constexpr double kBStage = 2.0;

template <typename T> struct Arith;

// Natural log for positive normal doubles, for the per-node logs that feed the
// log means.  x = m 2^e with m in [1/sqrt2, sqrt2); ln m = 2 atanh(s),
// s = (m-1)/(m+1), |s| <= 0.1716, from the odd series of atanh truncated after
// s^23 (remainder below 2e-19 relative); e ln2 is added in two parts (ln2 split
// into a 32-bit head and a tail) so e ln2_hi is exact.  Absolute error is a
// few ulp of |ln x|; only differences of two such logs larger than ~0.02 are
// used, so this is ample (the division by m+1 carries a relative error below
// 3e-15, i.e. below 1e-15 absolute in ln m).
__device__ inline double ln_pos(double x)
{
    int e;
    double m = frexp(x, &e);            // x = m 2^e, m in [0.5, 1)
    if (m < 0.70710678118654752440) {   // move m into [1/sqrt2, sqrt2)
        m = m + m;
        e -= 1;
    }
    const double num = m - 1.0, den = m + 1.0;
    double r = __builtin_amdgcn_rcp(den);
    r = fma(r, fma(-den, r, 1.0), r);     // one Newton step: relative error < 3e-15
    const double t = num * r;
    const double t2 = t * t;
    double p = 1.0 / 23.0;
    p = fma(p, t2, 1.0 / 21.0);
    p = fma(p, t2, 1.0 / 19.0);
    p = fma(p, t2, 1.0 / 17.0);
    p = fma(p, t2, 1.0 / 15.0);
    p = fma(p, t2, 1.0 / 13.0);
    p = fma(p, t2, 1.0 / 11.0);
    p = fma(p, t2, 1.0 / 9.0);
    p = fma(p, t2, 1.0 / 7.0);
    p = fma(p, t2, 1.0 / 5.0);
    p = fma(p, t2, 1.0 / 3.0);
    const double lnm = fma(2.0 * t * t2, p, 2.0 * t);   // 2t + 2t^3 p(t^2)
    const double ln2_hi = 0.693147180369123816490;       // 32 significant bits
    const double ln2_lo = 1.90821492927058770002e-10;    // ln2 - ln2_hi
    const double de = (double)e;
    return fma(de, ln2_hi, fma(de, ln2_lo, lnm));
}

template <> struct Arith<double> {
    // series branch of the log mean when |c-a| < kSeries (c+a), i.e.
    // f = ((c-a)/(c+a))^2 < 1e-4: truncation after f^3 leaves an error below
    // f^4/9 < 2e-17.
    static constexpr double kSeries = 1.0e-2;
    // node logs are natural logs
    static constexpr double kLogToLn = 1.0;
    __device__ static inline double node_log(double x) { return ln_pos(x); }
    // 1/x: the hardware estimate (relative error below 5e-8 on gfx950)
    // refined by one Newton step, which squares the error: below 3e-15,
    // far inside the 1e-11 the volume term is held to.
    __device__ static inline double rcp(double x) {
        const double r = __builtin_amdgcn_rcp(x);
        return fma(r, fma(-x, r, 1.0), r);
    }
};

template <> struct Arith<float> {
    // |c-a| < 0.1 (c+a), f < 1e-2: truncation after f^3 leaves an error
    // below 1.2e-9
    static constexpr float kSeries = 1.0e-1f;
    // node logs are base-2 logs (hardware v_log_f32); ln x = ln2 * log2 x
    static constexpr float kLogToLn = 0.693147180559945309f;
    __device__ static inline float node_log(float x) { return __builtin_amdgcn_logf(x); }
    __device__ static inline float rcp(float x) { return __builtin_amdgcn_rcpf(x); }
};

// Log of a node's b from its staged value 2b (the log of 2^17 b).
template <typename T>
__device__ inline T b_log(T b_staged)
{
    return Arith<T>::node_log(T(kBScale / kBStage) * b_staged);
}

// Branch-free select of a and b on c.  Both operands are always computed
// (they are a few multiplies each); a plain ?: lets the compiler sink their
// computation into divergent branches, which costs more than it saves.
__device__ inline double select(bool c, double a, double b)
{
    const unsigned long long ua = __builtin_bit_cast(unsigned long long, a);
    const unsigned long long ub = __builtin_bit_cast(unsigned long long, b);
    return __builtin_bit_cast(double, c ? ua : ub);
}
__device__ inline float select(bool c, float a, float b)
{
    const unsigned ua = __builtin_bit_cast(unsigned, a);
    const unsigned ub = __builtin_bit_cast(unsigned, b);
    return __builtin_bit_cast(float, c ? ua : ub);
}

// Values staged per node in LDS, field-major: value v of node t at
// v*SLOTS + slot(t), where slot() may pad rows, planes and elements of the
// node grid (Shape below).
// Scaled where the pair only needs a pair mean or a jump, so the pair does
// not multiply by constants: kU1..kU3 hold u/2 (X.u + Y.u = {{u}}), kW holds
// w/2 with w = phi - |u|^2/2 (the energy flux needs {{w}} only), kPhi holds
// phi/4 (the gravity term needs (1/4) [[phi]] only).
// The three metric values Ja^k_1..3 of a node sit at kJa + 3k.
enum NodeValue {
    kRho = 0, kU1, kU2, kU3, kB, kLogRho, kLogB, kPhi, kW, kInvB, kJa,
    kNodeValues = kJa + 9
};
constexpr int kPartialValues = 15;  // 3 directions x 5 fields

// Launch configuration of one kernel instance: EPB elements per workgroup of
// NT threads; WAVES > 0 asks the compiler to fit at least WAVES waves per
// SIMD in the volume-term kernel (it then caps the registers), WAVES_SURF the
// same for the kernel with the surface term; METRIC_LDS stages the metric
// terms in LDS (coalesced loads in phase A) instead of loading them per line
// thread.
template <int EPB_, int NT_, int WAVES_ = 0, bool METRIC_LDS_ = true, bool CACHE_ = false,
          int KMAJOR_ = 0, bool FIN_ = false, bool SERIES_ = false, bool SERIES_SURF_ = false,
          int ROW_PAD_ = 0, int PLANE_PAD_ = 0, int ELEM_PAD_ = 0, int WAVES_SURF_ = 0,
          int LANES_ = 1, bool DISTINCT_ = false, bool SLOTS64_ = false>
struct LaunchCfg {
    static constexpr int EPB = EPB_;
    static constexpr int NT = NT_;
    static constexpr int WAVES = WAVES_;
    static constexpr bool kMetricInLds = METRIC_LDS_;
    // CACHE: read the line's N+1 nodes from LDS once into registers (fewer
    // LDS reads, more registers); otherwise stream them per pair.
    static constexpr bool kCacheLine = CACHE_;
    // KMAJOR: order line tasks direction-major (all direction-1 lines of the
    // workgroup first), so each wave reads LDS with one stride pattern;
    // KMAJOR = 2 starts each direction on a 32-lane boundary (idle lanes in
    // between), so that no half-wave mixes lines of two directions.
    static constexpr bool kDirMajor = KMAJOR_ != 0;
    static constexpr bool kDirAligned = KMAJOR_ == 2;
    // FIN: the direction-3 line threads finish their own nodes (adding the
    // two other directions' partials from LDS, scaling by -1/J, storing), so
    // LDS holds two directional partials instead of three.
    static constexpr bool kFinalizeInLine = FIN_;
    // SERIES: the pair loop has a second form for waves whose lines all take
    // the series branch of the log means (fewer instructions per pair, more
    // registers); SERIES_SURF the same for the kernel with the surface term.
    static constexpr bool kSeriesForm = SERIES_;
    static constexpr bool kSeriesFormSurf = SERIES_SURF_;
    // Padding of the LDS node grid (in values): after every row of N+1
    // nodes along xi_1, every plane and every element.  Lines read LDS at a
    // fixed slot stride per direction, and the pads change those strides so
    // that the 64 lanes of a wave spread over the LDS banks.
    static constexpr int kRowPad = ROW_PAD_;
    static constexpr int kPlanePad = PLANE_PAD_;
    static constexpr int kElemPad = ELEM_PAD_;
    static constexpr int WAVES_SURF = WAVES_SURF_;
    // LANES = 2: two adjacent lanes share a line, each owning half its nodes
    // (line_pairs_x2); otherwise one lane per line.
    static constexpr int kLanes = LANES_;
    // DISTINCT: the general form of the pair loop forms the pair's metric
    // sums as exact fma(x, 1, y) with an opaque 1 (pair_update), so that
    // where both forms are compiled the compiler finds no common
    // instructions to hoist above the form branch.
    static constexpr bool kDistinctSums = DISTINCT_;
    // SLOTS64: round the stride between staged value arrays up to a multiple
    // of 64 slots, so that the compiler can fetch two values of a node with
    // one ds_read2st64 (offsets in units of 64 elements).
    static constexpr bool kSlots64 = SLOTS64_;
};

template <int N, class C>
struct Shape {
    static constexpr int Nq = N + 1;
    static constexpr int Nq2 = Nq * Nq;
    static constexpr int Np = Nq2 * Nq;
    static constexpr int kNodes = C::EPB * Np;          // nodes per workgroup
    // LDS slot strides of the node grid: x + kRow y + kPlane z + kElem eb
    static constexpr int kRow = Nq + C::kRowPad;
    static constexpr int kPlane = Nq * kRow + C::kPlanePad;
    static constexpr int kElem = Nq * kPlane + C::kElemPad;
    static constexpr bool kPadded = kElem != Np;
    // LDS slots per staged value (the stride between value arrays)
    static constexpr int kSlots = C::kSlots64 ? (C::EPB * kElem + 63) / 64 * 64 : C::EPB * kElem;
    static constexpr int kLines = 3 * C::EPB * Nq2;     // line tasks per workgroup
    // thread-index stride between the directions' first line tasks
    static constexpr int kDirStride = C::kDirAligned ? (C::EPB * Nq2 + 31) / 32 * 32 : C::EPB * Nq2;
    static constexpr int kTaskThreads = C::kLanes * (C::kDirMajor ? 3 * kDirStride : kLines);
    // nodes of a line each lane owns
    static constexpr int kOwn = Nq / C::kLanes;
    static_assert(C::kLanes == 1 || (C::kLanes == 2 && Nq % 2 == 0 && !C::kMetricInLds &&
                                     !C::kCacheLine),
                  "two lanes per line: an even node count, the line metric in registers");
    static constexpr int kNodeIters = (kNodes + C::NT - 1) / C::NT;  // nodes per thread
    static constexpr int kStaged = C::kMetricInLds ? kNodeValues : kJa;
    static constexpr int kPartials = C::kFinalizeInLine ? 10 : kPartialValues;
    static constexpr int kRegion = kStaged > kPartials ? kStaged : kPartials;
    // with FIN, -1/J of every node is staged after the shared region
    static constexpr int kMinusInvJ = kRegion;
    static constexpr int kFixedValues = kRegion + (C::kFinalizeInLine ? 1 : 0);
    // The split pressure (pressure_reference below) stages one more value per
    // node, b (p - P): inside the shared region when the partials leave a
    // value free there, else after everything else.
    static constexpr int kBDelta = kStaged < kPartials ? kStaged : kFixedValues;
    template <bool PSPLIT>
    static constexpr int kLdsValues =
        (kFixedValues + (PSPLIT && kBDelta == kFixedValues ? 1 : 0)) * kSlots;
    static_assert(kTaskThreads <= C::NT, "one line task per thread");
    static_assert(!C::kDirAligned || C::kDirMajor, "aligned order is direction-major");
    static_assert(C::kRowPad >= 0 && C::kPlanePad >= 0 && C::kElemPad >= 0, "pads");
    // LDS slot of node t of the workgroup (t = eb Np + x + Nq y + Nq^2 z)
    __device__ static inline int slot(int t) {
        if constexpr (!kPadded) {
            return t;
        } else {
            const int eb = t / Np, r = t - eb * Np;
            const int z = r / Nq2, r2 = r - z * Nq2;
            const int y = r2 / Nq, x = r2 - y * Nq;
            return eb * kElem + z * kPlane + y * kRow + x;
        }
    }
};

// One node's staged values, read from LDS where a pair needs them.
template <typename T>
struct NodeRegs {
    T rho, u1, u2, u3, b, lrho, lb, ph, w, ib, n1, n2, n3;
    T bd;  // b (p - P) for the split pressure (pressure_reference)
    __device__ inline void load_state(const T *lds, int SLOTS, int s) {
        rho = lds[kRho * SLOTS + s];
        u1 = lds[kU1 * SLOTS + s];
        u2 = lds[kU2 * SLOTS + s];
        u3 = lds[kU3 * SLOTS + s];
        b = lds[kB * SLOTS + s];
        lrho = lds[kLogRho * SLOTS + s];
        lb = lds[kLogB * SLOTS + s];
        ph = lds[kPhi * SLOTS + s];
        w = lds[kW * SLOTS + s];
        ib = lds[kInvB * SLOTS + s];
    }
    __device__ inline void load_bd(const T *lds, int SLOTS, int s, int index) {
        bd = lds[index * SLOTS + s];
    }
    __device__ inline void load_metric(const T *lds, int SLOTS, int s, int k) {
        n1 = lds[(kJa + 3 * k + 0) * SLOTS + s];
        n2 = lds[(kJa + 3 * k + 1) * SLOTS + s];
        n3 = lds[(kJa + 3 * k + 2) * SLOTS + s];
    }
};

// Series branch of the log means in f = s^2, s = jump/sum of the two states:
// s/atanh(s) = 1 - f/3 - 4f^2/45 - 44f^3/945 - ... (halved here) and
// atanh(s)/s = 1 + f/3 + f^2/5 + f^3/7 + ... (doubled here).
template <typename T>
__device__ inline T half_s_over_atanh(T f)
{
    return fma(fma(fma(T(-22.0 / 945.0), f, T(-2.0 / 45.0)), f, T(-1.0 / 6.0)), f, T(0.5));
}
template <typename T>
__device__ inline T two_atanh_over_s(T f)
{
    return fma(fma(fma(T(2.0 / 7.0), f, T(2.0 / 5.0)), f, T(2.0 / 3.0)), f, T(2));
}

// Contribution of the unordered pair (a, l) of one line, both directions of
// the pair, added to the accumulators of nodes a and l.
// X and Y are taken by value: a reference would take the address of the
// caller's locals, and the compiler fence in the pair loop would then keep
// them in scratch memory.  D[a][l] and D[l][a] are read where they are used.
// PSPLIT: the momentum flux takes the pressure mean relative to the
// element's reference pressure P (pressure_reference), from the staged
// b (p - P); the energy flux keeps its whole pressure mean.
template <typename T, bool SERIES = false, bool PSPLIT = false, bool DISTINCT = false>
__device__ inline void pair_update(const NodeRegs<T> X, const NodeRegs<T> Y,
                                   const T *__restrict__ Dal_p, const T *__restrict__ Dla_p,
                                   T *acc_a, T *acc_l, T P = T(0))
{
    // Every fused multiply-add is written out: the two forms of the pair
    // loop (and the face pairs) are compiled separately and must round
    // identically, so the compiler may not contract on its own.
#pragma clang fp contract(off)
    using A = Arith<T>;
    const T eps = T(A::kSeries);
    const T lnk = T(A::kLogToLn);
    const T cE = T(kBStage / (2.0 * (kGamma - 1.0)));  // 2/(2(gamma-1)) for the staged 2b
    // sums and jumps (jumps are partner l minus receiving node a)
    const T sr = X.rho + Y.rho, dr = Y.rho - X.rho;
    const T sb = X.b + Y.b, db = Y.b - X.b;
    T Lr, iLb, isb;
    if constexpr (SERIES) {
        // The caller guarantees that both log means take their series form
        // (every pair of the line is within the threshold).  The values are
        // those of the general form below with its log-difference factors
        // Ar = Bb = 1 (exact), so the result does not depend on the form.
        const T srsb = sr * sb;
        const T R = A::rcp(srsb);
        const T isr = R * sb;
        isb = R * sr;
        const T tr = dr * isr;
        Lr = sr * half_s_over_atanh(tr * tr);
        const T tb = db * isb;
        iLb = two_atanh_over_s(tb * tb) * isb;
    } else {
        const bool ser_r = fabs(dr) < eps * sr;
        const bool ser_b = fabs(db) < eps * sb;
        // one reciprocal serves 1/sr, 1/sb, 1/(ln rho_l - ln rho_a), 1/db
        const T Ar = select(ser_r, T(1), lnk * (Y.lrho - X.lrho));
        const T Bb = select(ser_b, T(1), db);
        const T srsb = sr * sb, AB = Ar * Bb;
        const T R = A::rcp(srsb * AB);
        const T isr = R * sb * AB;
        isb = R * sr * AB;
        const T iAr = R * srsb * Bb;
        const T iBb = R * srsb * Ar;
        // {{rho}}_log: series sr/2 * s/atanh(s) (s = dr/sr), else dr/(ln-difference)
        const T tr = dr * isr;
        Lr = select(ser_r, sr * half_s_over_atanh(tr * tr), dr * iAr);
        // 1/{{2b}}_log: series 2 atanh(s)/s / sb, else (ln-difference)/db
        const T tb = db * isb;
        iLb = select(ser_b, two_atanh_over_s(tb * tb) * isb, lnk * (Y.lb - X.lb) * iBb);
    }
    // {{rho}}/(2{{b}}): the density sum over the staged-2b sum; split: {{rho}}/(2{{b}}) - P
    // = (b_a (p_a - P) + b_l (p_l - P)) / (b_a + b_l)
    const T pt = PSPLIT ? (X.bd + Y.bd) * isb : sr * isb;
    // metric of the pair: Ja^k(a) + Ja^k(l); {{u}} (staged u is halved)
    T c1, c2, c3;
    if constexpr (!SERIES && DISTINCT) {
        // The same sums as fma(x, 1, y) (exact: one rounding of x + y) with
        // a 1 the compiler cannot see through.  Where a kernel carries both
        // forms, identical sums in both would be hoisted above the form
        // branch, making the sums of every pair of the line live there at
        // once (spills in the general form of the fp64 N = 4 whole rhs).
        T one = T(1);
        asm volatile("" : "+s"(one));
        c1 = fma(X.n1, one, Y.n1);
        c2 = fma(X.n2, one, Y.n2);
        c3 = fma(X.n3, one, Y.n3);
    } else {
        c1 = X.n1 + Y.n1;
        c2 = X.n2 + Y.n2;
        c3 = X.n3 + Y.n3;
    }
    const T s1 = X.u1 + Y.u1, s2 = X.u2 + Y.u2, s3 = X.u3 + Y.u3;
    // contravariant density flux {{rho}}_log ({{u}} . c)
    const T cs = fma(c1, s1, fma(c2, s2, c3 * s3));
    const T Fr = Lr * cs;
    // symmetric momentum part S~_m = F~rho {{u_m}} + c_m {{rho}}/(2{{b}})
    const T S1 = fma(Fr, s1, c1 * pt);
    const T S2 = fma(Fr, s2, c2 * pt);
    const T S3 = fma(Fr, s3, c3 * pt);
    // energy: (1/(2(g-1){{b}}_log) - {{|u|^2}}/2 + {{phi}}) F~rho + {{u}} . S~,
    // with -{{|u|^2}}/2 + {{phi}} = {{w}} (staged w is halved)
    // (split: S~ lacks c P, so {{u}} . S~ lacks P ({{u}} . c), added back here)
    const T coef = fma(cE, iLb, X.w + Y.w);
    const T uS = fma(s1, S1, fma(s2, S2, s3 * S3));
    const T FE = fma(coef, Fr, PSPLIT ? fma(P, cs, uS) : uS);
    // gravity: 1/2 rhohat [[phi]] with rhohat = {{b}}{{rho}}_log / b_own
    // = (2b_a + 2b_l) {{rho}}_log [[phi/4]] / (2b_own)  (staged phi is phi/4)
    const T g = sb * Lr * (Y.ph - X.ph);
    const T ga = g * X.ib;
    const T gl = -g * Y.ib;
    const T Dal = *Dal_p;
    const T Dla = *Dla_p;
    acc_a[0] = fma(Dal, Fr, acc_a[0]);
    acc_l[0] = fma(Dla, Fr, acc_l[0]);
    acc_a[1] = fma(Dal, fma(ga, c1, S1), acc_a[1]);
    acc_l[1] = fma(Dla, fma(gl, c1, S1), acc_l[1]);
    acc_a[2] = fma(Dal, fma(ga, c2, S2), acc_a[2]);
    acc_l[2] = fma(Dla, fma(gl, c2, S2), acc_l[2]);
    acc_a[3] = fma(Dal, fma(ga, c3, S3), acc_a[3]);
    acc_l[3] = fma(Dla, fma(gl, c3, S3), acc_l[3]);
    acc_a[4] = fma(Dal, FE, acc_a[4]);
    acc_l[4] = fma(Dla, FE, acc_l[4]);
}

// XCD-aware order of the batches.  The hardware hands workgroup i to
// accelerator die (XCD) i mod kXcds, each with its own L2; this permutation
// gives every XCD one contiguous range of batches instead, so elements that
// are neighbours in the mesh order run on the same die at about the same
// time and the surface term's face partners come from that die's L2.  It is
// a bijection of [0, nb) for any nb, so results do not depend on the real
// dispatch order.
constexpr int kXcds = 8;

__device__ inline int64_t xcd_batch(int64_t block, int64_t nb)
{
    const int64_t x = block % kXcds, i = block / kXcds;
    const int64_t q = nb / kXcds, r = nb % kXcds;
    return x * q + (x < r ? x : r) + i;
}

// Per-thread view of one workgroup's batch of elements.
template <int N, class C>
struct Batch {
    using S = Shape<N, C>;
    int64_t g0;      // first node of the batch
    int nvalid;      // nodes of the batch that exist (EPB * Np except at the tail)
    __device__ inline Batch(int64_t batch, int64_t nelem) {
        const int64_t e0 = batch * C::EPB;
        const int64_t left = nelem - e0;
        nvalid = (left < C::EPB ? (int)left : C::EPB) * S::Np;
        g0 = e0 * S::Np;
    }
};

// The line task of this thread in phase B (fixed for the kernel's lifetime).
template <int N, class C>
struct LineTask {
    using S = Shape<N, C>;
    // nb, step: LDS slot of the line's first node and the slot stride along
    // the line; n0, nstep: the same in the node numbering of one element
    int eb, k, nb, step, n0, nstep;
    int half;  // which half of the line's nodes this lane owns (two lanes per line)
    __device__ inline LineTask() {
        constexpr int Nq = S::Nq, Nq2 = S::Nq2, Np = S::Np;
        const int task = (int)threadIdx.x / C::kLanes;
        half = (int)threadIdx.x % C::kLanes;
        int line;
        if constexpr (C::kDirMajor) {
            k = task / S::kDirStride;
            const int r = task - k * S::kDirStride;
            eb = r / Nq2;  // r beyond the direction's lines (aligned order) gives eb >= EPB
            line = r - eb * Nq2;
            if (k > 2) { k = 2; eb = C::EPB; }  // idle thread: marked inactive below
        } else {
            eb = task / (3 * Nq2);
            const int r3 = task - eb * (3 * Nq2);
            k = r3 / Nq2;
            line = r3 - k * Nq2;
        }
        const int p1 = line % Nq, p2 = line / Nq;
        n0 = (k == 0) ? Nq * (p1 + Nq * p2) : (k == 1) ? p1 + Nq2 * p2 : p1 + Nq * p2;
        nstep = (k == 0) ? 1 : (k == 1) ? Nq : Nq2;
        if constexpr (S::kPadded) {
            constexpr int R = S::kRow, P = S::kPlane;
            const int base = (k == 0) ? R * p1 + P * p2 : (k == 1) ? p1 + P * p2 : p1 + R * p2;
            step = (k == 0) ? 1 : (k == 1) ? R : P;
            nb = eb * S::kElem + base;
        } else {
            step = nstep;
            nb = eb * Np + n0;
        }
    }
    // Node numbering for global memory: the workgroup-relative index of the
    // line's node a (node(a) = node_base() + a node_step()), and the line's
    // first node within its element.  Without pads the node and slot
    // numberings coincide.
    __device__ inline int node(int a) const {
        if constexpr (S::kPadded) return eb * S::Np + n0 + a * nstep;
        else return nb + a * step;
    }
    __device__ inline int node_base() const {
        if constexpr (S::kPadded) return eb * S::Np + n0;
        else return nb;
    }
    __device__ inline int first_in_element() const {
        if constexpr (S::kPadded) return n0;
        else return nb - eb * S::Np;
    }
    __device__ inline int node_step() const {
        if constexpr (S::kPadded) return nstep;
        else return step;
    }
    __device__ inline bool active(int nvalid) const {
        return (int)threadIdx.x < S::kTaskThreads && eb * S::Np < nvalid;
    }
    // Two lanes per line: the lane with half 0 owns line nodes 0..kOwn-1 as
    // its local nodes 0..kOwn-1, the lane with half 1 owns N..N-kOwn+1 (its
    // local node j is line node N - j).  own(j) / other(j): the line index of
    // this lane's / the other lane's local node j.
    __device__ inline int own(int j) const { return half ? N - j : j; }
    __device__ inline int other(int j) const { return half ? j : N - j; }
};

// The node whose reference pressure is its element's P (pressure_reference).
template <int N>
constexpr int kPressureNode = (N / 2) * (1 + (N + 1) + (N + 1) * (N + 1));

// A global load, non-temporal with STREAM.
template <bool STREAM, typename T>
__device__ inline T load(const T *p)
{
    if constexpr (STREAM) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool STREAM, typename T>
__device__ inline T load(__attribute__((address_space(1))) const T *p)
{
    if constexpr (STREAM) return __builtin_nontemporal_load(p);
    else return *p;
}

// &p[i] for a workgroup-uniform base p and a lane index 0 <= i with
// i * sizeof(T) < 2^32, in the form the global memory instructions take
// natively: a 64-bit base in scalar registers plus a 32-bit lane offset, so
// no 64-bit address arithmetic runs per lane.  The base passes through
// readfirstlane (exact for a uniform value), which keeps the compiler from
// folding it back into per-lane arithmetic.
template <typename T>
using global_ptr = __attribute__((address_space(1))) T *;
template <typename T>
__device__ inline global_ptr<T> lane_at(T *p, int i)
{
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return reinterpret_cast<global_ptr<T>>((hi << 32 | lo) + (uint32_t)i * (uint32_t)sizeof(T));
}

// Global values one thread loads for phase A: IT nodes x (5 fields, phi,
// with PERT the reference density and pressure, 9 metric terms when staged,
// J).  STREAM loads the state, phi and J non-temporally: in the volume term
// alone nothing reads them again, so they need not displace the line
// threads' metric loads, which revisit their cache lines, from the caches
// (the whole rhs re-reads neighbours' states for the face partners and
// keeps ordinary loads).
template <typename T, int N, class C, bool PERT = false, bool PSPLIT = false>
struct NodeLoads {
    using S = Shape<N, C>;
    static constexpr int IT = S::kNodeIters;
    T v[IT][PSPLIT ? 9 : PERT ? 8 : 6];
    T m[C::kMetricInLds ? IT : 1][9];
    T J[IT];
    template <bool STREAM = false>
    __device__ inline void issue(const T *__restrict__ q, const T *__restrict__ ref,
                                 const T *__restrict__ phi, const T *__restrict__ geom,
                                 int64_t fstride, const Batch<N, C> &B) {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            // Every lane loads, one past the batch's nodes the batch's last
            // node (in bounds, unused): with the loads under a branch the
            // compiler could not count them, and the later partner loads of
            // the whole rhs waited for all of them.
            const int t0 = threadIdx.x + it * C::NT;
            const int t = t0 < B.nvalid ? t0 : B.nvalid - 1;
            {
                // field bases of the batch are uniform; t is the lane offset
#pragma unroll
                for (int f = 0; f < 5; ++f)
                    v[it][f] = load<STREAM>(lane_at(q + (f * fstride + B.g0), t));
                v[it][5] = load<STREAM>(lane_at(phi + B.g0, t));
                if constexpr (PERT) {
                    v[it][6] = *lane_at(ref + B.g0, t);
                    v[it][7] = *lane_at(ref + (fstride + B.g0), t);
                }
                if constexpr (PSPLIT) {
                    // the element's reference pressure P (pressure_reference)
                    v[it][8] = *lane_at(ref + (fstride + B.g0), (t / S::Np) * S::Np + kPressureNode<N>);
                }
                if constexpr (C::kMetricInLds) {
#pragma unroll
                    for (int j = 0; j < 9; ++j) m[it][j] = *lane_at(geom + (j * fstride + B.g0), t);
                }
                J[it] = load<STREAM>(lane_at(geom + (9 * fstride + B.g0), t));
            }
        }
    }
};

// Per-node values the pairs use (primitives, 2b, logs, 1/(2b), w), from the
// conserved state and phi.  Phase A stages them for the element's own nodes;
// the surface term builds them for the face partners in a neighbouring
// element with the same operations, so both sides of a face see identical
// values.
//
// With PERT the state is carried as perturbation variables about a reference
// at rest with density rbar and pressure pbar (total energy
// Ebar = pbar/(gamma-1) + rbar phi): r = rho - rbar, E = E_full - Ebar, the
// momentum unchanged.  Then rho = rbar + r and
//     p = pbar + (gamma-1)(E - |m|^2/(2 rho) - r phi),
// the same pressure law with the reference's share taken out before the
// subtraction, so the small differences are formed without the large
// reference values.
//
// With PSPLIT (perturbation variables in fp32) the node also gets
// bd = b (p - P) for the split pressure (pressure_reference), with
// p - P = (pbar - P) + (gamma-1)(...) formed without p itself.  Without
// LOGS the two logs are left out (a face partner whose pair takes the
// series form of both log means does not need them).
template <typename T, bool PERT = false, bool PSPLIT = false, bool LOGS = true>
__device__ inline NodeRegs<T> node_values(T r, T m1, T m2, T m3, T E, T ph, T rbar = T(0),
                                          T pbar = T(0), T P = T(0))
{
    // fused multiply-adds written out, as in pair_update: a face partner's
    // values must round exactly as its own element's staged values
#pragma clang fp contract(off)
    using A = Arith<T>;
    const T gm1 = T(kGamma - 1.0);
    NodeRegs<T> V;
    const T rho = PERT ? rbar + r : r;
    const T irho = A::rcp(rho);
    const T hirho = T(0.5) * irho;
    V.rho = rho;
    V.u1 = m1 * hirho;                                  // u/2
    V.u2 = m2 * hirho;
    V.u3 = m3 * hirho;
    const T usq4 = fma(V.u1, V.u1, fma(V.u2, V.u2, V.u3 * V.u3));  // |u|^2 / 4
    const T dE = fma(-r, ph, E - fma(m1, V.u1, fma(m2, V.u2, m3 * V.u3)));
    const T p = PERT ? fma(gm1, dE, pbar) : gm1 * dE;
    V.b = rho * A::rcp(p);                        // 2b = rho/p
    V.ib = p * irho;                              // 1/(2b)
    if constexpr (PSPLIT) V.bd = V.b * fma(gm1, dE, pbar - P);
    if constexpr (LOGS) {
        V.lrho = A::node_log(rho);
        V.lb = b_log(V.b);
    }
    V.ph = T(0.25) * ph;                          // phi/4
    V.w = fma(T(0.5), ph, -usq4);                 // w/2 = (phi - |u|^2/2)/2
    return V;
}

// Phase A compute: per-node primitives and logs into LDS; returns -1/J per node.
template <typename T, int N, class C, bool PERT, bool PSPLIT = false>
__device__ inline void stage_nodes(const NodeLoads<T, N, C, PERT, PSPLIT> &L, const Batch<N, C> &B,
                                   T *lds, T (&mJ)[Shape<N, C>::kNodeIters])
{
    using A = Arith<T>;
    constexpr int SLOTS = Shape<N, C>::kSlots;
#pragma unroll
    for (int it = 0; it < Shape<N, C>::kNodeIters; ++it) {
        const int t = threadIdx.x + it * C::NT;
        if (t < B.nvalid) {
            const int st = Shape<N, C>::slot(t);
            NodeRegs<T> V;
            if constexpr (PSPLIT)
                V = node_values<T, true, true>(L.v[it][0], L.v[it][1], L.v[it][2], L.v[it][3],
                                               L.v[it][4], L.v[it][5], L.v[it][6], L.v[it][7],
                                               L.v[it][8]);
            else if constexpr (PERT)
                V = node_values<T, true>(L.v[it][0], L.v[it][1], L.v[it][2], L.v[it][3],
                                         L.v[it][4], L.v[it][5], L.v[it][6], L.v[it][7]);
            else
                V = node_values(L.v[it][0], L.v[it][1], L.v[it][2], L.v[it][3], L.v[it][4],
                                L.v[it][5]);
            lds[kRho * SLOTS + st] = V.rho;
            lds[kU1 * SLOTS + st] = V.u1;
            lds[kU2 * SLOTS + st] = V.u2;
            lds[kU3 * SLOTS + st] = V.u3;
            lds[kB * SLOTS + st] = V.b;
            lds[kLogRho * SLOTS + st] = V.lrho;
            lds[kLogB * SLOTS + st] = V.lb;
            lds[kPhi * SLOTS + st] = V.ph;
            lds[kW * SLOTS + st] = V.w;
            lds[kInvB * SLOTS + st] = V.ib;
            if constexpr (PSPLIT) lds[Shape<N, C>::kBDelta * SLOTS + st] = V.bd;
            if constexpr (C::kMetricInLds) {
#pragma unroll
                for (int j = 0; j < 9; ++j) lds[(kJa + j) * SLOTS + st] = L.m[it][j];
            }
            mJ[it] = -A::rcp(L.J[it]);
            if constexpr (C::kFinalizeInLine) lds[Shape<N, C>::kMinusInvJ * SLOTS + st] = mJ[it];
        }
    }
}

// Surface term, fused into the line tasks: the two ends of a direction-k line
// lie on the element's -xi_k and +xi_k faces, and the line thread adds the
// face flux of each end to that end's accumulator.
//
// Face neighbours come from nbr[nelem][6] (faces -xi1, +xi1, -xi2, +xi2,
// -xi3, +xi3): the neighbour holds the matching node on its opposite face,
// at the other end of the same line (conforming faces, same orientation);
// kFaceWall marks a slip wall, whose partner is the mirror state of the own
// node (velocity reflected in the face normal Ja^k).
constexpr int32_t kFaceWall = -1;

template <typename T, bool PERT = false>
struct FaceLoads {
    int32_t nb[2];   // neighbour across the face at line end 0 (a = 0) and end 1 (a = N)
    T v[2][PERT ? 8 : 6];  // its matching node: 5 conserved fields, phi (and the reference)
    // `nbr_batch` points at the batch's first element's entries (uniform),
    // `eb` is the lane's element within the batch.
    __device__ inline void issue_neighbours(const int32_t *__restrict__ nbr_batch, int eb, int k) {
        nb[0] = *lane_at(nbr_batch, 6 * eb + 2 * k);
        nb[1] = *lane_at(nbr_batch, 6 * eb + 2 * k + 1);
    }
    // Loads of the matching nodes; `local0` is the line's first node within
    // its element, `step` the node stride along the line.  A neighbour index
    // outside [0, nelem) (a wall, or an invalid index) loads the node of the
    // lane's own element (first node `own0`) instead, in bounds and unused.
    // The loads are issued unconditionally: behind a branch, the compiler
    // could no longer count them and made the node values wait for them too.
    // The index is non-negative where used, so its product with Np is formed
    // from 32 bits (a 64-bit product's expansion may read a register a load
    // is still writing, and wait for it).
    template <int N>
    __device__ inline void issue_states(const T *__restrict__ q, const T *__restrict__ ref,
                                        const T *__restrict__ phi, int64_t fstride, int64_t nelem,
                                        int64_t own0, int local0, int step) {
        constexpr int Np = (N + 1) * (N + 1) * (N + 1);
#pragma unroll
        for (int end = 0; end < 2; ++end) {
            const bool valid = nb[end] >= 0 && nb[end] < nelem;
            const int64_t e0 = valid ? (int64_t)((uint64_t)(uint32_t)nb[end] * (uint64_t)Np) : own0;
            const int64_t g = e0 + local0 + (end == 0 ? N : 0) * step;
#pragma unroll
            for (int f = 0; f < 5; ++f) v[end][f] = q[f * fstride + g];
            v[end][5] = phi[g];
            if constexpr (PERT) {
                v[end][6] = ref[g];
                v[end][7] = ref[fstride + g];
            }
        }
    }
    // P: the own element's reference pressure (PSPLIT); LOGS as node_values
    template <bool PSPLIT = false, bool LOGS = true>
    __device__ inline NodeRegs<T> partner(int end, T P = T(0)) const {
        if constexpr (PSPLIT)
            return node_values<T, true, true, LOGS>(v[end][0], v[end][1], v[end][2], v[end][3],
                                                    v[end][4], v[end][5], v[end][6], v[end][7],
                                                    P);
        else if constexpr (PERT)
            return node_values<T, true, false, LOGS>(v[end][0], v[end][1], v[end][2], v[end][3],
                                                     v[end][4], v[end][5], v[end][6], v[end][7]);
        else
            return node_values<T, false, false, LOGS>(v[end][0], v[end][1], v[end][2],
                                                      v[end][3], v[end][4], v[end][5]);
    }
};

template <typename T, int N, class C, bool PERT, bool PSPLIT = false>
__device__ inline void surface_ends(const T *lds, const LineTask<N, C> &L,
                                    const T (&lm)[C::kMetricInLds ? 1 : N + 1][3],
                                    const FaceLoads<T, PERT> &F, int64_t nelem, T P,
                                    T (&acc)[N + 1][5])
{
    using A = Arith<T>;
    constexpr int SLOTS = Shape<N, C>::kSlots;
    // The surface term at an end node is -(+-1) Ja^k . F*(own, partner) / (w_end J)
    // with the LGL end weight w_end = 2/(N(N+1)); pair_update contracts with
    // Ja^k(own) + Ja^k(partner) = 2 Ja^k(own), so the coefficient is
    // +-1/(2 w_end) = +-N(N+1)/4.
    // A partner's logs are formed only when some lane of the wave has a face
    // pair outside the log means' series threshold (one wave vote per end,
    // the general form's own test): the series form gives the same values.
    constexpr double kEnd = N * (N + 1) / 4.0;
    const T eps = T(A::kSeries);
#pragma unroll
    for (int end = 0; end < 2; ++end) {
        const int a = end ? N : 0;
        NodeRegs<T> X;
        X.load_state(lds, SLOTS, L.nb + a * L.step);
        if constexpr (PSPLIT) X.load_bd(lds, SLOTS, L.nb + a * L.step, Shape<N, C>::kBDelta);
        if constexpr (C::kMetricInLds) {
            X.load_metric(lds, SLOTS, L.nb + a * L.step, L.k);
        } else {
            X.n1 = lm[a][0]; X.n2 = lm[a][1]; X.n3 = lm[a][2];
        }
        const int32_t nb = F.nb[end];
        NodeRegs<T> Y = X;
        if (nb == kFaceWall) {
            const T nn = X.n1 * X.n1 + X.n2 * X.n2 + X.n3 * X.n3;
            const T un2 = T(2) * (X.u1 * X.n1 + X.u2 * X.n2 + X.u3 * X.n3) * A::rcp(nn);
            Y.u1 = X.u1 - un2 * X.n1;
            Y.u2 = X.u2 - un2 * X.n2;
            Y.u3 = X.u3 - un2 * X.n3;
        } else if (nb >= 0 && nb < nelem) {
            Y = F.template partner<PSPLIT, false>(end, P);
            Y.n1 = X.n1; Y.n2 = X.n2; Y.n3 = X.n3;
        } else {
            Y.rho = T(__builtin_nan(""));  // invalid neighbour index: the result says so
        }
        const T coef = end ? T(kEnd) : T(-kEnd);
        T partner[5] = {T(0), T(0), T(0), T(0), T(0)};
        const bool series = fabs(Y.rho - X.rho) < eps * (X.rho + Y.rho) &&
                            fabs(Y.b - X.b) < eps * (X.b + Y.b);
        if (__all(series)) {
            pair_update<T, true, PSPLIT>(X, Y, &coef, &coef, acc[a], partner, P);
        } else {
            if (nb >= 0 && nb < nelem) {  // the mirror state keeps the own node's logs
                Y.lrho = A::node_log(Y.rho);
                Y.lb = b_log(Y.b);
            }
            pair_update<T, false, PSPLIT>(X, Y, &coef, &coef, acc[a], partner, P);
        }
    }
}

// True when every pair of this thread's line takes the series form of both
// log means: any pair's jump is at most max - min along the line and its sum
// at least 2 min, so (max - min) < 2 eps min implies the per-pair test; the
// 1 % margin covers that test's rounding.  Non-positive or infinite states
// give false; fmin/fmax skip a NaN state, but a NaN node makes every pair of
// its line NaN in either form, so the forms still agree.
template <typename T, int N, class C>
__device__ inline bool line_in_series(const T *lds, const LineTask<N, C> &L)
{
    constexpr int SLOTS = Shape<N, C>::kSlots;
    T rmin = lds[kRho * SLOTS + L.nb], rmax = rmin;
    T bmin = lds[kB * SLOTS + L.nb], bmax = bmin;
#pragma unroll
    for (int a = 1; a < N + 1; ++a) {
        const T r = lds[kRho * SLOTS + L.nb + a * L.step];
        const T b = lds[kB * SLOTS + L.nb + a * L.step];
        rmin = fmin(rmin, r);
        rmax = fmax(rmax, r);
        bmin = fmin(bmin, b);
        bmax = fmax(bmax, b);
    }
    const T lim = T(0.99 * 2.0 * Arith<T>::kSeries);
    return (rmax - rmin) < lim * rmin && (bmax - bmin) < lim * bmin;
}

// Phase B: every unordered pair of this thread's line.
template <typename T, int N, class C, bool SERIES, bool PSPLIT>
__device__ inline void line_pairs_form(const T *lds, const T *__restrict__ D,
                                       const LineTask<N, C> &L,
                                       const T (&lm)[C::kMetricInLds ? 1 : N + 1][3],
                                       T (&acc)[N + 1][5], T P)
{
    constexpr int Nq = N + 1, SLOTS = Shape<N, C>::kSlots, BD = Shape<N, C>::kBDelta;
    if constexpr (C::kCacheLine) {
        NodeRegs<T> V[Nq];
#pragma unroll
        for (int a = 0; a < Nq; ++a) {
            V[a].load_state(lds, SLOTS, L.nb + a * L.step);
            if constexpr (PSPLIT) V[a].load_bd(lds, SLOTS, L.nb + a * L.step, BD);
            if constexpr (C::kMetricInLds) {
                V[a].load_metric(lds, SLOTS, L.nb + a * L.step, L.k);
            } else {
                V[a].n1 = lm[a][0]; V[a].n2 = lm[a][1]; V[a].n3 = lm[a][2];
            }
        }
#pragma unroll
        for (int a = 0; a < Nq - 1; ++a)
#pragma unroll
            for (int l = a + 1; l < Nq; ++l)
                pair_update<T, SERIES, PSPLIT, C::kDistinctSums>(V[a], V[l], D + a * Nq + l,
                                                                 D + l * Nq + a, acc[a], acc[l], P);
        return;
    }
#pragma unroll
    for (int a = 0; a < Nq - 1; ++a) {
        // Re-read node values from LDS in every outer iteration instead of
        // keeping the whole line live in registers.
        asm volatile("" ::: "memory");
        NodeRegs<T> X;
        X.load_state(lds, SLOTS, L.nb + a * L.step);
        if constexpr (PSPLIT) X.load_bd(lds, SLOTS, L.nb + a * L.step, BD);
        if constexpr (C::kMetricInLds) {
            X.load_metric(lds, SLOTS, L.nb + a * L.step, L.k);
        } else {
            X.n1 = lm[a][0]; X.n2 = lm[a][1]; X.n3 = lm[a][2];
        }
#pragma unroll
        for (int l = a + 1; l < Nq; ++l) {
            NodeRegs<T> Y;
            Y.load_state(lds, SLOTS, L.nb + l * L.step);
            if constexpr (PSPLIT) Y.load_bd(lds, SLOTS, L.nb + l * L.step, BD);
            if constexpr (C::kMetricInLds) {
                Y.load_metric(lds, SLOTS, L.nb + l * L.step, L.k);
            } else {
                Y.n1 = lm[l][0]; Y.n2 = lm[l][1]; Y.n3 = lm[l][2];
            }
            pair_update<T, SERIES, PSPLIT, C::kDistinctSums>(X, Y, D + a * Nq + l, D + l * Nq + a,
                                                             acc[a], acc[l], P);
        }
    }
}

// Phase B.  With SPLIT the form is chosen once per wave: when every line of
// the wave is within the series threshold (smooth flow), the pairs skip the
// log branch and the selects; otherwise each pair selects for itself.  Both
// forms give the same values.
template <typename T, int N, class C, bool SPLIT, bool PSPLIT = false>
__device__ inline void line_pairs(const T *lds, const T *__restrict__ D, const LineTask<N, C> &L,
                                  const T (&lm)[C::kMetricInLds ? 1 : N + 1][3],
                                  T (&acc)[N + 1][5], T P = T(0))
{
    if (SPLIT && __all(line_in_series<T, N, C>(lds, L)))
        line_pairs_form<T, N, C, true, PSPLIT>(lds, D, L, lm, acc, P);
    else
        line_pairs_form<T, N, C, false, PSPLIT>(lds, D, L, lm, acc, P);
}

// Split pressure (PSPLIT; the fp32 kernels on perturbation variables).
// The momentum flux of a pair carries the pressure mean p^ = {{rho}}/(2{{b}})
// times the pair's metric c = Ja^k(a) + Ja^k(l); for a state near
// hydrostatic balance p^ is O(p) while the line's net momentum flux is far
// smaller, so rounding p^ c to fp32 in every pair leaves noise of
// eps * p * |Ja| * sum|D| in the momentum.  For any P fixed per element,
//     p^ = P + (b_a (p_a - P) + b_l (p_l - P)) / (b_a + b_l)
// exactly, with b = rho/(2p).  The pairs and the face ends take the second
// part, formed from the staged b (p - P) (small near balance, so its
// rounding is small), and this function adds the first part once per line
// node: P times the sum over the line's pairs of D_al c_m and over its face
// ends of +-N(N+1)/4 * 2 Ja^k_m(a), a sum of metric and D values only that
// is formed in fp64, where the fp32 products are exact and the face parts
// cancel the volume's end-node parts without rounding.  P is the element's
// reference pressure at its node (N/2, N/2, N/2), the same for the element's
// nodes, lines and face partners.
template <typename T, int N, class C>
__device__ inline void pressure_reference(const T *lds, const T *__restrict__ D,
                                          const LineTask<N, C> &L,
                                          const T (&lm)[C::kMetricInLds ? 1 : N + 1][3], T P,
                                          T (&acc)[N + 1][5])
{
    constexpr int Nq = N + 1, SLOTS = Shape<N, C>::kSlots;
    constexpr double kEnd2 = N * (N + 1) / 2.0;  // 2 x the face coefficient N(N+1)/4
    // P Ja^k_m(l) in fp64 (exact: a product of two fp32 values)
    double pj[Nq][3];
    const double Pd = (double)P;
#pragma unroll
    for (int l = 0; l < Nq; ++l) {
        T n[3];
        if constexpr (C::kMetricInLds) {
#pragma unroll
            for (int m = 0; m < 3; ++m)
                n[m] = lds[(kJa + 3 * L.k + m) * SLOTS + L.nb + l * L.step];
        } else {
#pragma unroll
            for (int m = 0; m < 3; ++m) n[m] = lm[l][m];
        }
#pragma unroll
        for (int m = 0; m < 3; ++m) pj[l][m] = Pd * (double)n[m];
    }
#pragma unroll
    for (int a = 0; a < Nq; ++a) {
        // P sum_l D_al (Ja(a) + Ja(l)) + face part = P Ja(a) rs + sum_l D_al P Ja(l)
        double rs = (a == N) ? kEnd2 : (a == 0) ? -kEnd2 : 0.0;
        double g[3] = {0.0, 0.0, 0.0};
#pragma unroll
        for (int l = 0; l < Nq; ++l) {
            if (l == a) continue;
            const double d = (double)D[a * Nq + l];
            rs += d;
#pragma unroll
            for (int m = 0; m < 3; ++m) g[m] = fma(d, pj[l][m], g[m]);
        }
#pragma unroll
        for (int m = 0; m < 3; ++m) acc[a][1 + m] += (T)fma(pj[a][m], rs, g[m]);
    }
}

// ---------------------------------------------------------------------------
// Two lanes per line (LANES = 2, an even node count Nq = 2H).  Adjacent lanes
// 2t and 2t+1 share a line; each owns H of its nodes (LineTask::own) and
// holds only their accumulators and metric, about half the registers of a
// whole line.  Every unordered pair of the line is evaluated once, except the
// H pairs (j, N-j) that join the two halves' mirror nodes, which both lanes
// evaluate at half weight:
//   * pairs within a half: by the owning lane, both contributions local;
//   * pairs across the halves, for each local index y of the other lane:
//     pairs (own x, other y) with x <= y.  The lane with half 0 covers the
//     line pairs (x, N-y), x <= y; the lane with half 1 the pairs (N-x, y),
//     x <= y, i.e. (x', N-y') with x' >= y': together every cross pair once,
//     the mirror pairs x = y twice.  The partner's contributions are summed
//     in registers over x and handed to the other lane once per y, with the
//     partner's metric, by a DPP swap of adjacent lanes.
// The LGL differentiation matrix satisfies D[N-a][N-l] = -D[a][l], so the
// coefficients of the lane with half 1 are those of the lane with half 0 at
// the same local indices with the opposite sign: both lanes read the same
// (uniform) D values, and the lane with half 1 keeps its accumulators
// negated, which it undoes when it writes them (line_sign).  What a lane
// receives from the other is therefore always subtracted.

// The value of the adjacent lane (2t <-> 2t+1): DPP quad_perm [1, 0, 3, 2].
__device__ inline float swap_lanes(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1,
                                                             0xF, 0xF, false));
}
__device__ inline double swap_lanes(double x)
{
    const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
    const int lo = __builtin_amdgcn_mov_dpp((int)(unsigned)u, 0xB1, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(unsigned)(u >> 32), 0xB1, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

// +1 for the lane with half 0, -1 for the one with half 1 (see above).
template <typename T, int N, class C>
__device__ inline T line_sign(const LineTask<N, C> &L)
{
    return L.half ? T(-1) : T(1);
}

template <typename T, int N, class C, bool SERIES>
__device__ inline void line_pairs_x2_form(const T *lds, const T *__restrict__ D,
                                          const LineTask<N, C> &L, const T (&lm)[(N + 1) / 2][3],
                                          T (&acc)[(N + 1) / 2][5])
{
    constexpr int Nq = N + 1, H = Nq / 2, SLOTS = Shape<N, C>::kSlots;
    // pairs within the own half
#pragma unroll
    for (int x = 0; x < H - 1; ++x) {
        asm volatile("" ::: "memory");
        NodeRegs<T> X;
        X.load_state(lds, SLOTS, L.nb + L.own(x) * L.step);
        X.n1 = lm[x][0]; X.n2 = lm[x][1]; X.n3 = lm[x][2];
#pragma unroll
        for (int y = x + 1; y < H; ++y) {
            NodeRegs<T> Y;
            Y.load_state(lds, SLOTS, L.nb + L.own(y) * L.step);
            Y.n1 = lm[y][0]; Y.n2 = lm[y][1]; Y.n3 = lm[y][2];
            pair_update<T, SERIES>(X, Y, D + x * Nq + y, D + y * Nq + x, acc[x], acc[y]);
        }
    }
    // pairs across the halves
#pragma unroll
    for (int y = 0; y < H; ++y) {
        asm volatile("" ::: "memory");
        NodeRegs<T> P;
        P.load_state(lds, SLOTS, L.nb + L.other(y) * L.step);
        P.n1 = swap_lanes(lm[y][0]);
        P.n2 = swap_lanes(lm[y][1]);
        P.n3 = swap_lanes(lm[y][2]);
        T pacc[5] = {T(0), T(0), T(0), T(0), T(0)};
#pragma unroll
        for (int x = 0; x <= y; ++x) {
            NodeRegs<T> X;
            X.load_state(lds, SLOTS, L.nb + L.own(x) * L.step);
            X.n1 = lm[x][0]; X.n2 = lm[x][1]; X.n3 = lm[x][2];
            if (x == y) {
                // the mirror pair (x, N-x): both lanes evaluate it, each at half weight
                const T dal = T(0.5) * D[x * Nq + (N - y)];
                const T dla = T(0.5) * D[(N - y) * Nq + x];
                pair_update<T, SERIES>(X, P, &dal, &dla, acc[x], pacc);
            } else {
                pair_update<T, SERIES>(X, P, D + x * Nq + (N - y), D + (N - y) * Nq + x, acc[x],
                                       pacc);
            }
        }
#pragma unroll
        for (int f = 0; f < 5; ++f) acc[y][f] -= swap_lanes(pacc[f]);
    }
}

template <typename T, int N, class C, bool SPLIT>
__device__ inline void line_pairs_x2(const T *lds, const T *__restrict__ D, const LineTask<N, C> &L,
                                     const T (&lm)[(N + 1) / 2][3], T (&acc)[(N + 1) / 2][5])
{
    if (SPLIT && __all(line_in_series<T, N, C>(lds, L)))
        line_pairs_x2_form<T, N, C, true>(lds, D, L, lm, acc);
    else
        line_pairs_x2_form<T, N, C, false>(lds, D, L, lm, acc);
}

// The face neighbour of the one line end a lane owns (its local node 0: line
// node 0 for half 0, N for half 1).
template <typename T, bool PERT = false>
struct FaceLoad1 {
    int32_t nb;
    T v[PERT ? 8 : 6];
    __device__ inline void issue_neighbour(const int32_t *__restrict__ nbr, int64_t e, int k,
                                           int end) {
        nb = nbr[6 * e + 2 * k + end];
    }
    template <int N>
    __device__ inline void issue_state(const T *__restrict__ q, const T *__restrict__ ref,
                                       const T *__restrict__ phi, int64_t fstride, int64_t nelem,
                                       int local0, int step, int end) {
        constexpr int Np = (N + 1) * (N + 1) * (N + 1);
        if (nb >= 0 && nb < nelem) {
            const int64_t g = (int64_t)nb * Np + local0 + (end == 0 ? N : 0) * step;
#pragma unroll
            for (int f = 0; f < 5; ++f) v[f] = q[f * fstride + g];
            v[5] = phi[g];
            if constexpr (PERT) {
                v[6] = ref[g];
                v[7] = ref[fstride + g];
            }
        }
    }
    __device__ inline NodeRegs<T> partner() const {
        if constexpr (PERT)
            return node_values<T, true>(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]);
        else
            return node_values(v[0], v[1], v[2], v[3], v[4], v[5]);
    }
};

// Surface term of the owned line end (see surface_ends).  The owned end's
// coefficient is -N(N+1)/4 on the -xi_k face (half 0) and +N(N+1)/4 on the
// +xi_k face (half 1), whose accumulators are kept negated: -N(N+1)/4 for both.
template <typename T, int N, class C, bool PERT>
__device__ inline void surface_end_x2(const T *lds, const LineTask<N, C> &L,
                                      const T (&lm)[(N + 1) / 2][3], const FaceLoad1<T, PERT> &F,
                                      int64_t nelem, T (&acc)[(N + 1) / 2][5])
{
    using A = Arith<T>;
    constexpr int SLOTS = Shape<N, C>::kSlots;
    constexpr double kEnd = N * (N + 1) / 4.0;
    NodeRegs<T> X;
    X.load_state(lds, SLOTS, L.nb + L.own(0) * L.step);
    X.n1 = lm[0][0]; X.n2 = lm[0][1]; X.n3 = lm[0][2];
    NodeRegs<T> Y = X;
    if (F.nb == kFaceWall) {
        const T nn = X.n1 * X.n1 + X.n2 * X.n2 + X.n3 * X.n3;
        const T un2 = T(2) * (X.u1 * X.n1 + X.u2 * X.n2 + X.u3 * X.n3) * A::rcp(nn);
        Y.u1 = X.u1 - un2 * X.n1;
        Y.u2 = X.u2 - un2 * X.n2;
        Y.u3 = X.u3 - un2 * X.n3;
    } else if (F.nb >= 0 && F.nb < nelem) {
        Y = F.partner();
        Y.n1 = X.n1; Y.n2 = X.n2; Y.n3 = X.n3;
    } else {
        Y.rho = T(__builtin_nan(""));  // invalid neighbour index: the result says so
    }
    const T coef = T(-kEnd);
    T partner[5] = {T(0), T(0), T(0), T(0), T(0)};
    pair_update(X, Y, &coef, &coef, acc[0], partner);
}

// Phase C with two lanes per line: each lane writes its own nodes' partials
// (sign restored).
template <typename T, int N, class C>
__device__ inline void write_partials_x2(T *lds, const LineTask<N, C> &L, bool active,
                                         const T (&acc)[(N + 1) / 2][5])
{
    constexpr int SLOTS = Shape<N, C>::kSlots;
    if (active && (!C::kFinalizeInLine || L.k < 2)) {
        const T sg = line_sign<T>(L);
#pragma unroll
        for (int j = 0; j < (N + 1) / 2; ++j) {
            const int s = L.nb + L.own(j) * L.step;
#pragma unroll
            for (int f = 0; f < 5; ++f) lds[(L.k * 5 + f) * SLOTS + s] = sg * acc[j][f];
        }
    }
}

// Source term h of the whole right-hand side: the Coriolis term of the
// momentum equation, h = -omega x U (U the momentum).  `on` is uniform over
// the launch; the momentum is re-read at the store (the workgroup loaded it
// in phase A, so it comes from cache).
template <typename T>
struct Rotation {
    T w1, w2, w3;
    bool on;
    __device__ inline void add(T U1, T U2, T U3, T &h1, T &h2, T &h3) const {
        h1 -= w2 * U3 - w3 * U2;
        h2 -= w3 * U1 - w1 * U3;
        h3 -= w1 * U2 - w2 * U1;
    }
};

// Where a node's right-hand side r goes.  Without STAGE it is stored as is.
// With STAGE the kernel is one stage of a 2N-storage low-storage Runge-Kutta
// scheme ([ESDG-GPU §3] steps with such a scheme and recomputes the fluxes
// at every stage), fused into the store:
//     dq <- a dq + dt r,    q_out <- q + b dq,
// with `out` the register dq and q the stage's input state (perturbation
// variables with PERT: the reference is fixed in time).  a == 0 does not
// read dq (the first stage may find it uninitialised).  The source term is
// added to r before the update.
template <typename T, bool STAGE>
struct Sink {
    T *__restrict__ out;    // rhs, or the register dq with STAGE
    T *__restrict__ q_out;  // STAGE: the stage's output state
    T a, b, dt;             // STAGE: the stage's coefficients and the step
    // Address of node i of field f of the batch that starts at node g0
    // (uniform), for the stage's loads and stores: a uniform base plus a
    // 32-bit lane offset in fp32; the fp64 stage keeps the per-lane 64-bit
    // form, which measured 7 % faster in its register-capped kernel.
    template <typename P>
    __device__ inline auto stage_at(P *p, int64_t fstride, int f, int64_t g0, int i) const {
        if constexpr (sizeof(T) == 4) return lane_at(p + (f * fstride + g0), i);
        else return p + (f * fstride + g0 + i);
    }
    // The node is i of the batch that starts at node g0 (uniform).
    __device__ inline void put(const T *__restrict__ q, int64_t fstride, int64_t g0, int i,
                               const Rotation<T> &rot, T (&r)[5]) const {
        T U[5];
        if (STAGE || rot.on) {
#pragma unroll
            for (int f = STAGE ? 0 : 1; f < (STAGE ? 5 : 4); ++f)
                U[f] = *stage_at(q, fstride, f, g0, i);
        }
        if (rot.on) rot.add(U[1], U[2], U[3], r[1], r[2], r[3]);
        if constexpr (STAGE) {
            T k[5];
#pragma unroll
            for (int f = 0; f < 5; ++f) k[f] = dt * r[f];
            if (a != T(0)) {
#pragma unroll
                for (int f = 0; f < 5; ++f) k[f] = fma(a, *stage_at(out, fstride, f, g0, i), k[f]);
            }
#pragma unroll
            for (int f = 0; f < 5; ++f) {
                *stage_at(out, fstride, f, g0, i) = k[f];
                *stage_at(q_out, fstride, f, g0, i) = fma(b, k[f], U[f]);
            }
        } else {
            // Nothing reads the right-hand side back within the launch: it
            // streams past the caches (the stage's outputs above stay cached
            // for the next stage, which reads them).
#pragma unroll
            for (int f = 0; f < 5; ++f)
                __builtin_nontemporal_store(r[f], lane_at(out + (f * fstride + g0), i));
        }
    }
};

// Phases C and D: directional partials through LDS, scaling, store.
template <typename T, int N, class C>
__device__ inline void write_partials(T *lds, const LineTask<N, C> &L, bool active,
                                      const T (&acc)[N + 1][5])
{
    constexpr int SLOTS = Shape<N, C>::kSlots;
    if (active && (!C::kFinalizeInLine || L.k < 2)) {
#pragma unroll
        for (int a = 0; a < N + 1; ++a) {
            const int s = L.nb + a * L.step;
#pragma unroll
            for (int f = 0; f < 5; ++f) lds[(L.k * 5 + f) * SLOTS + s] = acc[a][f];
        }
    }
}

// FIN: a direction-3 line thread adds the direction-1 and -2 partials of its
// nodes to its own (same order as store_rhs), scales by -1/J and stores.
template <typename T, int N, class C, bool STAGE>
__device__ inline void finish_line(const T *lds, const LineTask<N, C> &L, bool active,
                                   const Batch<N, C> &B, int64_t fstride,
                                   const T (&acc)[N + 1][5], const T *__restrict__ q,
                                   const Rotation<T> &rot, const Sink<T, STAGE> &sink)
{
    constexpr int SLOTS = Shape<N, C>::kSlots;
    if (active && L.k == 2) {
#pragma unroll
        for (int a = 0; a < N + 1; ++a) {
            const int s = L.nb + a * L.step;
            const T mJ = lds[Shape<N, C>::kMinusInvJ * SLOTS + s];
            T r[5];
#pragma unroll
            for (int f = 0; f < 5; ++f)
                r[f] = (lds[f * SLOTS + s] + lds[(5 + f) * SLOTS + s] + acc[a][f]) * mJ;
            sink.put(q, fstride, B.g0, L.node(a), rot, r);
        }
    }
}

// FIN with two lanes per line: a direction-3 lane finishes its own nodes.
template <typename T, int N, class C, bool STAGE>
__device__ inline void finish_line_x2(const T *lds, const LineTask<N, C> &L, bool active,
                                      const Batch<N, C> &B, int64_t fstride,
                                      const T (&acc)[(N + 1) / 2][5], const T *__restrict__ q,
                                      const Rotation<T> &rot, const Sink<T, STAGE> &sink)
{
    constexpr int SLOTS = Shape<N, C>::kSlots;
    if (active && L.k == 2) {
        const T sg = line_sign<T>(L);
#pragma unroll
        for (int j = 0; j < (N + 1) / 2; ++j) {
            const int a = L.own(j);
            const int s = L.nb + a * L.step;
            const T mJ = lds[Shape<N, C>::kMinusInvJ * SLOTS + s];
            T r[5];
#pragma unroll
            for (int f = 0; f < 5; ++f)
                r[f] = (lds[f * SLOTS + s] + lds[(5 + f) * SLOTS + s] + sg * acc[j][f]) * mJ;
            sink.put(q, fstride, B.g0, L.node(a), rot, r);
        }
    }
}

template <typename T, int N, class C, bool STAGE>
__device__ inline void store_rhs(const T *lds, const Batch<N, C> &B, int64_t fstride,
                                 const T (&mJ)[Shape<N, C>::kNodeIters], const T *__restrict__ q,
                                 const Rotation<T> &rot, const Sink<T, STAGE> &sink)
{
    constexpr int SLOTS = Shape<N, C>::kSlots;
#pragma unroll
    for (int it = 0; it < Shape<N, C>::kNodeIters; ++it) {
        const int t = threadIdx.x + it * C::NT;
        if (t < B.nvalid) {
            const int st = Shape<N, C>::slot(t);
            T r[5];
#pragma unroll
            for (int f = 0; f < 5; ++f) {
                const T s = lds[f * SLOTS + st] + lds[(5 + f) * SLOTS + st] + lds[(10 + f) * SLOTS + st];
                r[f] = s * mJ[it];
            }
            sink.put(q, fstride, B.g0, t, rot, r);
        }
    }
}

// Phase marks for the measurement probes: NoMarks (the library's kernels)
// compiles to nothing; WallMarks has lane 0 of each workgroup write the wall
// clock on entry (0), after phase A's barrier (1), after phase B's barrier
// (2), the hardware id of its compute unit (4) and its batch (5), and lane 0
// of every wave raise slot 3 to the clock when the wave has issued its last
// store (no barrier added: waves that finish early leave early, as in the
// library's kernels), all to out[blockIdx.x * kMarkValues + i]; slot 3 must
// start at zero.
constexpr int kMarkValues = 6;

struct NoMarks {
    static constexpr bool on = false;
    __device__ inline void at(int) const {}
    __device__ inline void where(int64_t) const {}
    __device__ inline void wave_end() const {}
};

struct WallMarks {
    static constexpr bool on = true;
    unsigned long long *out;
    __device__ inline void at(int i) const {
        if (threadIdx.x == 0) out[(int64_t)blockIdx.x * kMarkValues + i] = (unsigned long long)wall_clock64();
    }
    __device__ inline void where(int64_t batch) const {
        if (threadIdx.x == 0) {
            out[(int64_t)blockIdx.x * kMarkValues + 4] = __smid();
            out[(int64_t)blockIdx.x * kMarkValues + 5] = (unsigned long long)batch;
        }
    }
    __device__ inline void wave_end() const {
        if ((threadIdx.x & 63) == 0)
            atomicMax(out + (int64_t)blockIdx.x * kMarkValues + 3,
                      (unsigned long long)wall_clock64());
    }
};

// One workgroup per batch of EPB elements.  SURF adds the entropy-conservative
// surface term (face neighbours from nbr), giving the whole right-hand side;
// rot.on adds the Coriolis source.  STAGE fuses a Runge-Kutta stage into the
// store (Sink); PERT reads the state as perturbation variables about the
// reference ref = (rbar, pbar) (node_values).
template <typename T, int N, class C, bool SURF = false, bool STAGE = false, bool PERT = false,
          class Marks = NoMarks>
__global__ void __attribute__((amdgpu_flat_work_group_size(1, C::NT)))
__attribute__((amdgpu_waves_per_eu(SURF ? (C::WAVES_SURF > 0 ? C::WAVES_SURF : 1)
                                         : (C::WAVES > 0 ? C::WAVES : 1))))
volume_rhs_kernel(const T *__restrict__ q, const T *__restrict__ ref, const T *__restrict__ phi,
                  const T *__restrict__ geom, const T *__restrict__ D,
                  const int32_t *__restrict__ nbr, Rotation<T> rot, int64_t nelem,
                  Sink<T, STAGE> sink, Marks marks = Marks())
{
    static_assert(SURF || !(STAGE || PERT), "stages and perturbation variables need the whole rhs");
    using S = Shape<N, C>;
    constexpr int Nq = N + 1;
    // fp32 on perturbation variables splits the pressure (pressure_reference)
    constexpr bool PSPLIT = PERT && sizeof(T) == 4;
    static_assert(!PSPLIT || C::kLanes == 1, "the split pressure takes one lane per line");
    __shared__ T lds[S::template kLdsValues<PSPLIT>];
    const int64_t fstride = nelem * S::Np;
    // the whole right-hand side walks the batches in XCD-contiguous order
    const int64_t batch = SURF ? xcd_batch(blockIdx.x, gridDim.x) : (int64_t)blockIdx.x;
    const Batch<N, C> B(batch, nelem);
    const LineTask<N, C> L;
    const bool active = L.active(B.nvalid);
    if constexpr (!SURF) rot.on = false;  // the volume term alone has no source
    marks.at(0);
    marks.where(batch);

    // phase A: issue every global load first
    if constexpr (C::kLanes == 2) {
        constexpr int H = Nq / 2;
        FaceLoad1<T, PERT> face;
        if constexpr (SURF) {
            const int64_t e = batch * C::EPB + L.eb;  // in bounds for idle lanes (unused)
            face.issue_neighbour(nbr, e < nelem ? e : nelem - 1, L.k, L.half);
        }
        NodeLoads<T, N, C, PERT> ld;
        ld.template issue<!SURF>(q, ref, phi, geom, fstride, B);
        T lm[H][3];
        if (active) {
#pragma unroll
            for (int j = 0; j < H; ++j)
#pragma unroll
                for (int c = 0; c < 3; ++c)
                    lm[j][c] = geom[(3 * L.k + c) * fstride + B.g0 + L.node(L.own(j))];
        }
        if constexpr (SURF) {
            if (active) face.template issue_state<N>(q, ref, phi, fstride, nelem,
                                                    L.first_in_element(), L.node_step(), L.half);
        }
        T mJ[S::kNodeIters];
        stage_nodes<T, N, C, PERT>(ld, B, lds, mJ);
        __syncthreads();
        marks.at(1);

        // phase B
        T acc[H][5];
#pragma unroll
        for (int j = 0; j < H; ++j)
#pragma unroll
            for (int f = 0; f < 5; ++f) acc[j][f] = T(0);
        if constexpr (SURF) {
            if (active) surface_end_x2<T, N, C, PERT>(lds, L, lm, face, nelem, acc);
        }
        constexpr bool kSplit = SURF ? C::kSeriesFormSurf : C::kSeriesForm;
        if (active) line_pairs_x2<T, N, C, kSplit>(lds, D, L, lm, acc);
        __syncthreads();
        marks.at(2);

        // phases C, D
        write_partials_x2<T, N, C>(lds, L, active, acc);
        __syncthreads();
        if constexpr (C::kFinalizeInLine) {
            finish_line_x2<T, N, C, STAGE>(lds, L, active, B, fstride, acc, q, rot, sink);
        } else {
            store_rhs<T, N, C, STAGE>(lds, B, fstride, mJ, q, rot, sink);
        }
        marks.wave_end();
        return;
    } else {
    FaceLoads<T, PERT> face;
    // The lane's element within the batch, clamped to the batch's last one
    // for idle lanes, and its first node: a uniform base plus a 32-bit offset.
    const int own_eb = L.eb < B.nvalid / S::Np ? L.eb : B.nvalid / S::Np - 1;
    const int64_t own0 = B.g0 + own_eb * S::Np;
    if constexpr (SURF) {
        // Every lane loads its neighbour indices, an idle lane those of the
        // batch's last element (in bounds; unused): loaded under a branch, the
        // indices were moved between registers at the branch's end, which
        // made each wave wait for them before issuing its node loads.
        face.issue_neighbours(nbr + 6 * batch * C::EPB, own_eb, L.k);
        // keep the index loads first in the queue: the partner loads wait for
        // them, not for the node loads issued after them
        asm volatile("" ::: "memory");
    }
    NodeLoads<T, N, C, PERT, PSPLIT> ld;
    ld.template issue<!SURF>(q, ref, phi, geom, fstride, B);
    // Issued unconditionally, the loads may not sink towards their uses
    // (behind the later loads): keep the issue order.
    asm volatile("" ::: "memory");
    // The remaining phase-A loads are issued by every lane, an idle lane
    // reading its clamped element's values (in bounds, unused), so that the
    // compiler can count them past the node values' wait.
    T P = T(0);  // the element's reference pressure (PSPLIT)
    if constexpr (PSPLIT) P = ref[fstride + own0 + kPressureNode<N>];
    T lm[C::kMetricInLds ? 1 : Nq][3];
    if constexpr (!C::kMetricInLds) {
        // the line's Ja^k_1 at its first node, then uniform field offsets and
        // a pointer step along the line.  3k fstride for k in {0, 1, 2} is
        // formed with masks: the expansion of a 64-bit product reads an
        // undefined high half, which the compiler may place in a register a
        // node load is still writing, and then waits for that load.
        const int64_t f3 = 3 * fstride;
        const int64_t koff = (f3 & -(int64_t)(L.k >= 1)) + (f3 & -(int64_t)(L.k >= 2));
        const T *p = geom + (koff + own0 + L.first_in_element());
        const int step = L.node_step();
#pragma unroll
        for (int a = 0; a < Nq; ++a) {
#pragma unroll
            for (int j = 0; j < 3; ++j) lm[a][j] = p[j * fstride];
            p += step;
        }
    }
    if constexpr (SURF) {
        asm volatile("" ::: "memory");
        face.template issue_states<N>(q, ref, phi, fstride, nelem, own0, L.first_in_element(),
                                      L.node_step());
    }
    T mJ[S::kNodeIters];
    stage_nodes<T, N, C, PERT, PSPLIT>(ld, B, lds, mJ);
    __syncthreads();
    marks.at(1);

    // phase B
    T acc[Nq][5];
#pragma unroll
    for (int a = 0; a < Nq; ++a)
#pragma unroll
        for (int f = 0; f < 5; ++f) acc[a][f] = T(0);
    // the face partners first: their loaded states die before the pair loop
    if constexpr (SURF) {
        if (active) surface_ends<T, N, C, PERT, PSPLIT>(lds, L, lm, face, nelem, P, acc);
    }
    constexpr bool kSplit = SURF ? C::kSeriesFormSurf : C::kSeriesForm;
    if (active) line_pairs<T, N, C, kSplit, PSPLIT>(lds, D, L, lm, acc, P);
    if constexpr (PSPLIT) {
        if (active) pressure_reference<T, N, C>(lds, D, L, lm, P, acc);
    }
    __syncthreads();  // node values are dead from here on: LDS becomes the partials
    marks.at(2);

    // phases C, D
    write_partials<T, N, C>(lds, L, active, acc);
    __syncthreads();
    if constexpr (C::kFinalizeInLine) {
        finish_line<T, N, C, STAGE>(lds, L, active, B, fstride, acc, q, rot, sink);
    } else {
        store_rhs<T, N, C, STAGE>(lds, B, fstride, mJ, q, rot, sink);
    }
    marks.wave_end();
    }
}

}  // namespace esdg
