"""Pins of the oracle's Coriolis source h = -omega x U ([ESDG-GPU §2, Eq. 1b;
§3, h in Eq. 2], page "GPU Performance of an Entropy-Stable Discontinuous
Galerkin Euler Solver with Non-Conservative Terms").

  f-plane closed form ........... omega = (0, 0, f): h = (f U2, -f U1, 0) on the
                                  momentum (the textbook f-plane Coriolis force)
  general omega ................. numpy's cross product (a library routine)
  no work, no entropy ........... u . h = 0 and v . h = 0 node by node, so the
                                  whole right-hand side still conserves entropy
                                  globally and leaves mass and energy alone
"""
import numpy as np
import pytest

import oracle
from entropy_stable_dg_amd import inputs as I
from tests.test_oracle_surface import global_entropy_rate, nodewise_random_state, periodic_mesh
from tests.test_oracle_pins import weights3


def check_f_plane(orc):
    rng = np.random.default_rng(1)
    q = rng.uniform(-2, 2, (5, 3, 27))
    q[0] = rng.uniform(0.5, 1.5, (3, 27))
    f = 1.03e-4
    h = np.zeros_like(q)
    orc.add_coriolis(q, [0.0, 0.0, f], h)
    assert np.array_equal(h[0], np.zeros_like(h[0])) and np.array_equal(h[4], np.zeros_like(h[4]))
    assert np.allclose(h[1], f * q[2], rtol=1e-15, atol=0)
    assert np.allclose(h[2], -f * q[1], rtol=1e-15, atol=0)
    assert np.array_equal(h[3], np.zeros_like(h[3]))


def test_f_plane(orc):
    check_f_plane(orc)


def check_general_omega(orc):
    rng = np.random.default_rng(2)
    q = rng.uniform(-2, 2, (5, 4, 8))
    om = rng.uniform(-1e-4, 1e-4, 3)
    h = np.zeros_like(q)
    orc.add_coriolis(q, om, h)
    ref = -np.cross(om[None, :], q[1:4].reshape(3, -1).T).T.reshape(3, 4, 8)
    assert np.allclose(h[1:4], ref, rtol=1e-14, atol=1e-22)


def test_general_omega(orc):
    check_general_omega(orc)


def check_entropy_with_rotation(orc, N):
    rng = np.random.default_rng(90 + N)
    K = (3, 2, 2)
    D, X, geom, nbr = periodic_mesh(K, N, 0.05, 5, (True, True, False))
    rho, u, p, phi = nodewise_random_state(rng, X[0].shape)
    q = I.conserved(rho, u, p, phi)
    om = np.array([1e-4, -2e-4, 1.4e-4])
    rhs = orc.rhs(q, phi, geom, D, nbr, N, omega=om)
    W, _ = weights3(N)
    total, scale = global_entropy_rate(rhs, geom, W, rho, u, p, phi)
    assert abs(total) <= 1e-12 * scale
    base = orc.rhs(q, phi, geom, D, nbr, N)
    assert np.array_equal(rhs[0], base[0]) and np.array_equal(rhs[4], base[4])
    assert not np.array_equal(rhs[1], base[1])


@pytest.mark.parametrize("N", [2, 4])
def test_entropy_with_rotation(orc, N):
    check_entropy_with_rotation(orc, N)
