"""The line-level test that selects the series-only pair loop implies the
per-pair test, evaluated in the kernel's precision.

The kernel evaluates the log means (page: GPU Performance of an
Entropy-Stable DG Euler Solver with Non-Conservative Terms, section 4.1) on
their series branch for a pair when |x_l - x_a| < eps (x_l + x_a), for
x = rho and x = s_b b, with eps = 1e-2 (fp64) and 1e-1 (fp32).  A wave skips
that per-pair test when every one of its lines satisfies
(max - min) < 0.99 * 2 eps * min along the line.  Any pair's jump is at most
max - min and its sum at least 2 min, and the 1 % margin covers the rounding
of both tests; here lines are drawn with their spread right at the line
bound, and every pair of every accepted line must pass the per-pair test
computed the way the kernel computes it (sum, difference, product by eps,
compare, all rounded to the precision).
"""
import numpy as np
import pytest

EPS = {np.float64: 1e-2, np.float32: 1e-1}


def line_test(x, eps, dtype):
    lo, hi = x.min(axis=1), x.max(axis=1)
    lim = dtype(0.99 * 2.0 * eps)
    return (hi - lo) < lim * lo


def pair_test(x, eps, dtype):
    e = dtype(eps)
    n = x.shape[1]
    ok = np.ones(x.shape[0], dtype=bool)
    for a in range(n):
        for l in range(a + 1, n):
            s = x[:, a] + x[:, l]
            d = x[:, l] - x[:, a]
            ok &= np.abs(d) < e * s
    return ok


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("nq", [2, 5, 9])
def test_line_bound_implies_pair_test(dtype, nq):
    eps = EPS[dtype]
    rng = np.random.default_rng(nq + (1 if dtype == np.float32 else 0))
    m = 200_000
    base = np.exp(rng.uniform(-30, 30, m))
    # spreads straddling the line bound, down to a few ulp from it
    frac = 0.99 * 2 * eps * (1.0 + rng.choice([-1, 1], m) * np.exp(rng.uniform(-40, -1, m)))
    u = rng.uniform(0, 1, (m, nq))
    u[:, 0], u[:, -1] = 0.0, 1.0                 # the extremes are on the line
    x = (base[:, None] * (1.0 + frac[:, None] * u)).astype(dtype)
    rng.permuted(x, axis=1, out=x)
    accepted = line_test(x, eps, dtype)
    assert 0.2 < accepted.mean() < 0.8           # both sides of the bound are exercised
    assert pair_test(x[accepted], eps, dtype).all()


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_line_bound_rejects_nan_and_large_jumps(dtype):
    eps = EPS[dtype]
    x = np.array([[1.0, 1.0, np.nan], [1.0, 1.0 + 2.5 * eps, 1.0], [1.0, 1.0, 1.0]], dtype=dtype)
    assert line_test(x, eps, dtype).tolist() == [False, False, True]
