"""The oracle's pins have teeth: each plausible mistake below, planted in a
temporary copy of the oracle's C source (on the CPU, never in the tree),
must make at least one pin fail."""
import os

import pytest

import oracle
from tests import test_oracle_pins as P
from tests import test_oracle_surface as S
from tests import test_oracle_coriolis as R
from tests import test_oracle_time as T

SRC = os.path.join(os.path.dirname(oracle.__file__), "esdg_oracle.c")

# (name, text in esdg_oracle.c, replacement)
MUTANTS = [
    ("energy flux without the mean geopotential",
     "- usq_avg / 2 + phi_avg) * Frho", "- usq_avg / 2) * Frho"),
    ("gravity term with the wrong sign",
     "Fm += p_tilde + rho_hat * phi_jump / 2", "Fm += p_tilde - rho_hat * phi_jump / 2"),
    ("one-sided density weight on the partner's side",
     "b_avg * rho_log / si->b", "b_avg * rho_log / sl->b"),
    ("arithmetic mean in place of the log mean of b",
     "real b_log = logmean(si->b, sl->b);", "real b_log = avg(si->b, sl->b);"),
    ("arithmetic mean in place of the log mean of rho",
     "real rho_log = logmean(si->rho, sl->rho);", "real rho_log = avg(si->rho, sl->rho);"),
    ("|{{u}}|^2 in place of {{|u|^2}}",
     "real usq_avg = avg(si->usq, sl->usq);",
     "real usq_avg = u_avg[0]*u_avg[0] + u_avg[1]*u_avg[1] + u_avg[2]*u_avg[2];"),
    ("pressure law without rho*phi",
     "- UU / (2 * q[0]) - q[0] * phi)", "- UU / (2 * q[0]))"),
    ("pressure mean with the log mean of b",
     "rho_avg / (2 * b_avg);", "rho_avg / (2 * b_log);"),
    ("transposed differentiation matrix",
     "D[ik * Nq + l]", "D[l * Nq + ik]"),
    ("transposed metric terms",
     "(real)geom[(3 * k + j) * stride + e * Np + i]\n                                      + (real)geom[(3 * k + j) * stride + e * Np + il]",
     "(real)geom[(3 * j + k) * stride + e * Np + i]\n                                      + (real)geom[(3 * j + k) * stride + e * Np + il]"),
    ("own metric only instead of the pair sum",
     "+ (real)geom[(3 * k + j) * stride + e * Np + il]", "+ (real)geom[(3 * k + j) * stride + e * Np + i]"),
    ("missing 1/J",
     "rhs[f * stride + e * Np + i] = -acc[f] / Ji;", "rhs[f * stride + e * Np + i] = -acc[f];"),
    ("wrong overall sign",
     "rhs[f * stride + e * Np + i] = -acc[f] / Ji;", "rhs[f * stride + e * Np + i] = acc[f] / Ji;"),
    ("wrong line stride in direction 2",
     ": (k == 1) ? a + Nq * (l + Nq * c)", ": (k == 1) ? l + Nq * (b + Nq * c)"),
    ("energy flux with the full momentum flux (gravity included)",
     "if (m == j) sym += p_tilde;", "if (m == j) sym += p_tilde + rho_hat * phi_jump / 2;"),
    # surface term
    ("surface term with the wrong face sign",
     "const int side = (ik == N) ? 1 : -1;", "const int side = (ik == N) ? -1 : 1;"),
    ("surface weight 1/(N(N+1)) instead of the LGL end weight",
     "const real w_end = (real)2 / ((real)N * (real)(N + 1));",
     "const real w_end = (real)1 / ((real)N * (real)(N + 1));"),
    ("neighbour's node not taken on the opposite face",
     "const int jk = N - ik;", "const int jk = ik;"),
    ("wall partner not reflected",
     "sp.u[j] = si.u[j] - 2 * un * n[j];", "sp.u[j] = si.u[j];"),
    ("wall reflection with an unnormalised normal",
     "/ (n[0] * n[0] + n[1] * n[1] + n[2] * n[2]);", ";"),
    ("surface term without 1/J",
     "(real)side * term[f] / (w_end * Ji);", "(real)side * term[f] / w_end;"),
    # Coriolis source
    ("Coriolis term with the wrong sign",
     "rhs[(1 + m) * stride + n] -= wxU[m];", "rhs[(1 + m) * stride + n] += wxU[m];"),
    ("Coriolis cross product with swapped components",
     "omega[2] * U[0] - omega[0] * U[2]", "omega[0] * U[2] - omega[2] * U[0]"),
    # time stepping
    ("a digit of a Runge-Kutta weight swapped",
     "B[2] = (real)1720146321549", "B[2] = (real)1720146321594"),
    ("a Runge-Kutta register coefficient with the wrong sign",
     "A[3] = -(real)3550918686646", "A[3] = (real)3550918686646"),
    ("Runge-Kutta register not carried between stages",
     "k[i] = A[s] * k[i] + dt * Lq[i];", "k[i] = dt * Lq[i];"),
    ("Runge-Kutta update from the stage's rhs instead of the register",
     "q[i] = q[i] + B[s] * k[i];", "q[i] = q[i] + B[s] * dt * Lq[i];"),
    # conservation integrals and perturbation variables
    ("entropy integral with the wrong sign",
     "wJ * (-s.rho * ent / (ORACLE_GAMMA - 1))", "wJ * (s.rho * ent / (ORACLE_GAMMA - 1))"),
    ("quadrature weight of the third direction taken from the second",
     "(real)w[a] * (real)w[b] * (real)w[c]", "(real)w[a] * (real)w[b] * (real)w[b]"),
    ("integral without the Jacobian",
     "* (real)geom[9 * stride + e * Np + i];", ";"),
    ("reference energy without its potential energy",
     "pbar / (ORACLE_GAMMA - 1) + rbar * (real)phi[i]", "pbar / (ORACLE_GAMMA - 1)"),
]

# a cheap battery of pins: every check raises AssertionError on a mismatch
BATTERY = [
    (P.check_consistency, (0,)), (P.check_consistency, (2,)),
    (P.check_pairwise_entropy_condition, (0,)), (P.check_pairwise_entropy_condition, (1,)),
    (P.check_gravity_partner_scaling, (2,)),
    (P.check_element_entropy_identity, (2, True)), (P.check_element_entropy_identity, (3, False)),
    (P.check_free_stream, (2,)),
    (P.check_isothermal_hydrostatic, (3, False)), (P.check_isothermal_hydrostatic, (4, True)),
    (P.check_cartesian_reduction, (1,)),
    (P.check_element_vs_50_digits, (1,)),
    (S.check_global_entropy_conservation, (2, (True, True, True))),
    (S.check_global_entropy_conservation, (3, (True, False, False))),
    (S.check_conservation, (3, (True, False, False))),
    (S.check_free_stream_full, (2, (True, True, True))),
    (S.check_hydrostatic_full, (3, 0.05)),
    (S.check_surface_vs_50_digits, (1,)),
    (R.check_f_plane, ()), (R.check_general_omega, ()),
    (T.check_stability_polynomial, ()), (T.check_nonlinear_order, ()),
    (T.check_stepping_conservation, (2, (True, True, True))),
    (T.check_integrals_constant_state, (3,)), (T.check_integrals_polynomial_fields, (2,)),
    (T.check_integrals_isothermal_entropy, ()), (T.check_full_state, ()),
]


def failing_pins(orc):
    failed = []
    for fn, args in BATTERY:
        try:
            fn(orc, *args)
        except (AssertionError, FloatingPointError, ValueError):
            failed.append(fn.__name__)
    return failed


def test_battery_passes_on_the_oracle():
    assert failing_pins(oracle.default()) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site not found: {name}"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.compile_library(str(mutated), str(tmp_path / "libmutant.so"))
    failed = failing_pins(oracle.Oracle(lib))
    assert failed, f"no pin catches: {name}"
