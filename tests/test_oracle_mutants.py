"""The oracle's pins have teeth: each plausible mistake below, planted in a
temporary copy of the oracle's C source (on the CPU, never in the tree),
must make at least one pin fail."""
import os

import pytest

import oracle
from tests import test_oracle_pins as P
from tests import test_oracle_surface as S
from tests import test_oracle_coriolis as R

SRC = os.path.join(os.path.dirname(oracle.__file__), "esdg_oracle.c")

# (name, text in esdg_oracle.c, replacement)
MUTANTS = [
    ("energy flux without the mean geopotential",
     "- 0.5 * usq_avg + phi_avg) * Frho", "- 0.5 * usq_avg) * Frho"),
    ("gravity term with the wrong sign",
     "Fm += p_tilde + 0.5 * rho_hat * phi_jump", "Fm += p_tilde - 0.5 * rho_hat * phi_jump"),
    ("one-sided density weight on the partner's side",
     "b_avg * rho_log / si->b", "b_avg * rho_log / sl->b"),
    ("arithmetic mean in place of the log mean of b",
     "double b_log = logmean(si->b, sl->b);", "double b_log = avg(si->b, sl->b);"),
    ("arithmetic mean in place of the log mean of rho",
     "double rho_log = logmean(si->rho, sl->rho);", "double rho_log = avg(si->rho, sl->rho);"),
    ("|{{u}}|^2 in place of {{|u|^2}}",
     "double usq_avg = avg(si->usq, sl->usq);",
     "double usq_avg = u_avg[0]*u_avg[0] + u_avg[1]*u_avg[1] + u_avg[2]*u_avg[2];"),
    ("pressure law without rho*phi",
     "- UU / (2.0 * q[0]) - q[0] * phi)", "- UU / (2.0 * q[0]))"),
    ("pressure mean with the log mean of b",
     "rho_avg / (2.0 * b_avg);", "rho_avg / (2.0 * b_log);"),
    ("transposed differentiation matrix",
     "D[ik * Nq + l]", "D[l * Nq + ik]"),
    ("transposed metric terms",
     "geom[(3 * k + j) * stride + e * Np + i]\n                                        + geom[(3 * k + j) * stride + e * Np + il]",
     "geom[(3 * j + k) * stride + e * Np + i]\n                                        + geom[(3 * j + k) * stride + e * Np + il]"),
    ("own metric only instead of the pair sum",
     "+ geom[(3 * k + j) * stride + e * Np + il]", "+ geom[(3 * k + j) * stride + e * Np + i]"),
    ("missing 1/J",
     "rhs[f * stride + e * Np + i] = -acc[f] / Ji;", "rhs[f * stride + e * Np + i] = -acc[f];"),
    ("wrong overall sign",
     "rhs[f * stride + e * Np + i] = -acc[f] / Ji;", "rhs[f * stride + e * Np + i] = acc[f] / Ji;"),
    ("wrong line stride in direction 2",
     ": (k == 1) ? a + Nq * (l + Nq * c)", ": (k == 1) ? l + Nq * (b + Nq * c)"),
    ("energy flux with the full momentum flux (gravity included)",
     "if (m == j) sym += p_tilde;", "if (m == j) sym += p_tilde + 0.5 * rho_hat * phi_jump;"),
    # surface term
    ("surface term with the wrong face sign",
     "const int side = (ik == N) ? 1 : -1;", "const int side = (ik == N) ? -1 : 1;"),
    ("surface weight 1/(N(N+1)) instead of the LGL end weight",
     "const double w_end = 2.0 / ((double)N * (double)(N + 1));",
     "const double w_end = 1.0 / ((double)N * (double)(N + 1));"),
    ("neighbour's node not taken on the opposite face",
     "const int jk = N - ik;", "const int jk = ik;"),
    ("wall partner not reflected",
     "sp.u[j] = si.u[j] - 2.0 * un * n[j];", "sp.u[j] = si.u[j];"),
    ("wall reflection with an unnormalised normal",
     "/ (n[0] * n[0] + n[1] * n[1] + n[2] * n[2]);", ";"),
    ("surface term without 1/J",
     "(double)side * term[f] / (w_end * Ji);", "(double)side * term[f] / w_end;"),
    # Coriolis source
    ("Coriolis term with the wrong sign",
     "rhs[(1 + m) * stride + n] -= wxU[m];", "rhs[(1 + m) * stride + n] += wxU[m];"),
    ("Coriolis cross product with swapped components",
     "omega[2] * U[0] - omega[0] * U[2]", "omega[0] * U[2] - omega[2] * U[0]"),
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
