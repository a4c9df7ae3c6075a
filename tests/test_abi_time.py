"""Host-side checks of the time-stepping, perturbation-variable and integral
entry points of the C ABI: synchronous argument errors before any HIP call
(fake, never-dereferenced addresses), and the stage coefficients."""
import numpy as np
import pytest

import oracle
from entropy_stable_dg_amd import esdg

OK, NULL, ORDER, NELEM, ALIAS = (esdg.ESDG_OK, esdg.ESDG_ERR_NULL, esdg.ESDG_ERR_ORDER,
                                 esdg.ESDG_ERR_NELEM, esdg.ESDG_ERR_ALIAS)

# distinct fake device addresses, far apart
Q, REF, PHI, GEOM, D, NBR, DQ, QO, QT, W, WORK, OUT = (0x10000000 * (i + 1) for i in range(12))


@pytest.mark.parametrize("fn", [esdg.esdg_rhs_pert_f64, esdg.esdg_rhs_pert_f32])
def test_rhs_pert_argument_errors(fn):
    assert fn(Q, REF, PHI, GEOM, D, NBR, None, 0, 1, OUT, 0) == ORDER
    assert fn(Q, REF, PHI, GEOM, D, NBR, None, 4, -1, OUT, 0) == NELEM
    assert fn(0, 0, 0, 0, 0, 0, None, 4, 0, 0, 0) == OK
    ptrs = [Q, REF, PHI, GEOM, D, NBR, OUT]
    for i in range(len(ptrs)):
        p = list(ptrs)
        p[i] = 0
        assert fn(p[0], p[1], p[2], p[3], p[4], p[5], None, 4, 10, p[6], 0) == NULL, i
    # rhs overlapping the reference
    assert fn(Q, REF, PHI, GEOM, D, NBR, None, 4, 10, REF + 64, 0) == ALIAS


@pytest.mark.parametrize("fn,size", [(esdg.esdg_lsrk_stage_f64, 8), (esdg.esdg_lsrk_stage_f32, 4)])
def test_stage_argument_errors(fn, size):
    N, nelem = 4, 10
    field = nelem * 125 * size
    args = dict(q_in=Q, ref=REF, phi=PHI, geom=GEOM, D=D, nbr=NBR, dq=DQ, q_out=QO)

    def call(**kw):
        a = dict(args, **kw)
        return fn(a["q_in"], a["ref"], a["phi"], a["geom"], a["D"], a["nbr"], None, 0.5, 0.25, 0.1,
                  kw.get("N", N), kw.get("nelem", nelem), a["dq"], a["q_out"], 0)

    assert call(N=9) == ORDER
    assert call(nelem=-3) == NELEM
    assert fn(0, 0, 0, 0, 0, 0, None, 0.0, 1.0, 1.0, N, 0, 0, 0, 0) == OK
    for name in ("q_in", "phi", "geom", "D", "nbr", "dq", "q_out"):
        assert call(**{name: 0}) == NULL, name
    assert call(ref=0) != NULL          # the reference is optional
    # outputs may not overlap inputs or each other; q_out may not be q_in
    assert call(q_out=Q) == ALIAS
    assert call(q_out=Q + 4 * field) == ALIAS
    assert call(dq=REF + field) == ALIAS
    assert call(dq=QO + 5 * field - size) == ALIAS
    assert call(q_out=NBR + 8) == ALIAS


@pytest.mark.parametrize("fn,size", [(esdg.esdg_lsrk_steps_f64, 8), (esdg.esdg_lsrk_steps_f32, 4)])
def test_steps_argument_errors(fn, size):
    N, nelem = 3, 10
    field = nelem * 64 * size

    def call(q=Q, qt=QT, dq=DQ, ref=REF, nsteps=2, N=N, nelem=nelem, nbr=NBR):
        return fn(q, qt, dq, ref, PHI, GEOM, D, nbr, None, 0.01, nsteps, N, nelem, 0)

    assert call(N=0) == ORDER
    assert call(nelem=-1) == NELEM
    assert call(nsteps=-1) == NELEM
    assert call(q=0, qt=0, dq=0, nsteps=0) == OK     # no steps: nothing read
    assert call(q=0, qt=0, dq=0, nelem=0) == OK
    assert call(qt=0) == NULL and call(dq=0) == NULL and call(nbr=0) == NULL
    assert call(qt=Q + field) == ALIAS
    assert call(q=GEOM + 3 * field) == ALIAS
    assert call(dq=QT) == ALIAS


@pytest.mark.parametrize("fn", [esdg.esdg_integrals_f64, esdg.esdg_integrals_f32])
def test_integrals_argument_errors(fn):
    assert fn(Q, REF, PHI, GEOM, W, 0, 10, WORK, OUT, 0) == ORDER
    assert fn(Q, REF, PHI, GEOM, W, 4, -1, WORK, OUT, 0) == NELEM
    assert fn(Q, REF, PHI, GEOM, W, 4, 10, 0, OUT, 0) == NULL
    assert fn(Q, REF, PHI, GEOM, W, 4, 10, WORK, 0, 0) == NULL
    for i in (0, 2, 3, 4):
        p = [Q, REF, PHI, GEOM, W]
        p[i] = 0
        assert fn(*p, 4, 10, WORK, OUT, 0) == NULL, i
    assert fn(Q, REF, PHI, GEOM, W, 4, 10, WORK, WORK + 8, 0) == ALIAS
    assert fn(Q, REF, PHI, GEOM, W, 4, 10, Q + 16, OUT, 0) == ALIAS
    assert fn(Q, REF, PHI, GEOM, W, 4, 10, WORK, W, 0) == ALIAS


def test_workspace_size():
    assert esdg.esdg_integrals_workspace_bytes() == 3 * 1024 * 8


def test_stage_coefficients_agree_with_the_oracle():
    """The library's table and the oracle's (each typed from the published
    ratios on its own) agree to rounding; the oracle's is pinned by the order
    conditions."""
    A, B = esdg.esdg_lsrk_coefficients()
    oA, oB = oracle.default().lsrk_coefficients()
    assert esdg.esdg_lsrk_stages() == 5
    np.testing.assert_allclose(A, oA, rtol=4e-16, atol=0)
    np.testing.assert_allclose(B, oB, rtol=4e-16, atol=0)
