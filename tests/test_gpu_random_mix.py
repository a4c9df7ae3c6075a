"""Seeded random cases with a per-element mix of smooth and rough states.

The pair loop runs a series-only form on waves whose lines all lie within
the log means' series threshold (page: GPU Performance of an Entropy-Stable
DG Euler Solver with Non-Conservative Terms, section 4.1) and the general
form elsewhere.  Here each case draws an order, a precision, a box of 1-45
elements, the volume term or the whole right-hand side (random periodicity),
and marks a random share of the elements rough (density and pressure
scaled node by node by 0.5-2, velocities perturbed by up to 30 m/s) on a
smooth hydrostatic-like base, so that waves mix lines of both kinds in
every arrangement.  Every case is held to the oracle at the parity
tolerance.
"""
import numpy as np
import pytest

import oracle
from entropy_stable_dg_amd import esdg
from entropy_stable_dg_amd import inputs as I
from tests.test_gpu_parity import dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {np.float64: 1e-11, np.float32: 2e-5}


def case_inputs(seed):
    rng = np.random.default_rng(7000 + seed)
    N = int(rng.integers(1, 9))
    dtype = np.float64 if rng.random() < 0.6 else np.float32
    K = (int(rng.integers(1, 6)), int(rng.integers(1, 4)), int(rng.integers(1, 4)))
    X = I.box_mesh(K, (0, 0, 0), tuple(300.0 * k for k in K), N, warp_frac=0.05, seed=seed)
    D = I.diff_matrix(N)
    geom = I.metrics(X, D)
    ne = X.shape[1]
    x, y, z = X.reshape(3, ne, -1)
    rho = 1.2 * np.exp(-z / 8000.0) * (1 + 1e-4 * np.sin(x / 97.0))
    p = rho * I.R_GAS * (300.0 + 0.01 * np.cos(y / 53.0))
    u = np.stack([0.5 * np.sin(z / 71.0), 0.3 * np.cos(x / 61.0), 0.1 * np.sin(y / 41.0)])
    rough = rng.random(ne) < rng.choice([0.0, 0.05, 0.3])
    for e in np.nonzero(rough)[0]:
        rho[e] *= rng.uniform(0.5, 2.0, rho[e].shape)
        p[e] *= rng.uniform(0.5, 2.0, p[e].shape)
        u[:, e] += rng.uniform(-30, 30, u[:, e].shape)
    phi = I.GRAV * z
    q = I.conserved(rho, u, p, phi)
    full = rng.random() < 0.4
    nbr = I.box_connectivity(K, tuple(bool(b) for b in rng.random(3) < 0.5)) if full else None
    q, phi, geom, D = (a.astype(dtype) for a in (q, phi, geom, D))
    return N, dtype, q, phi, geom, D, nbr, int(rough.sum())


@pytest.mark.parametrize("seed", range(48))
def test_random_mixed_waves(seed):
    N, dtype, q, phi, geom, D, nbr, nrough = case_inputs(seed)
    t = [torch.from_numpy(np.ascontiguousarray(a)).to(dev()) for a in (q, phi, geom, D)]
    if nbr is None:
        got = esdg.volume_rhs(*t).cpu().numpy()
        ref = oracle.volume_rhs(q, phi, geom, D, N)
        scale = np.abs(ref).reshape(5, -1).max(axis=1)
    else:
        got = esdg.rhs(*t, torch.from_numpy(nbr).to(dev())).cpu().numpy()
        ref, mag = oracle.rhs(q, phi, geom, D, nbr, N, with_magnitude=True)
        scale = np.abs(mag).reshape(5, -1).max(axis=1)
    err = np.abs(got.astype(np.float64) - ref).reshape(5, -1).max(axis=1) / scale
    print(f"[mix] seed={seed} N={N} {np.dtype(dtype).name} nelem={q.shape[1]} rough={nrough} "
          f"{'rhs' if nbr is not None else 'vol'} err={err.max():.2e}", flush=True)
    assert np.all(np.isfinite(got))
    assert err.max() <= TOL[dtype], err
