"""The two forms of the pair loop give bitwise equal results.

Where every line of a wave is within the series threshold of the log means
(page: GPU Performance of an Entropy-Stable DG Euler Solver with
Non-Conservative Terms, section 4.1, the log mean with its series branch), the
kernel runs a pair loop without the log branch and the selects; otherwise
each pair selects for itself.  The volume term is element-local, so a large
density jump at one node of one element (which sends every wave holding that
element's lines to the general form) must leave every other element's
result bitwise unchanged, although the waves shared with the perturbed
element now evaluate those elements' pairs with the other form (the host
checks that premise from the state: every line of the base state is within
the series range, and the perturbed element has lines outside it in every
direction).  The 125-element mesh leaves the last workgroup partly empty for
the launch shapes of N = 3, 4 and 5.  At fp64 N = 4 and 5 the general form
forms its metric sums differently from the series form (same values, other
instructions), and the bitwise agreement holds there too.  The whole
right-hand side couples face neighbours, so there the comparison excludes the
perturbed element and its six face neighbours.  Both runs are also held to
the oracle at the parity tolerance.
"""
import numpy as np
import pytest

import oracle
from entropy_stable_dg_amd import esdg
from entropy_stable_dg_amd import inputs as I
from tests.test_gpu_parity import dev, to_gpu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {np.float64: 1e-11, np.float32: 2e-5}


def smooth_workload(N, dtype):
    wl = I.build_workload(f"series_N{N}", (5, 5, 5), (0, 0, 0), (1000, 1000, 1000), N, "bubble",
                          seed=900 + N, warp_frac=0.05, periodic=(True, True, False))
    q, phi, geom, D = (a.astype(dtype) for a in (wl.q, wl.phi, wl.geom, wl.D))
    return q, phi, geom, D, wl.nbr


def perturb(q, e, node):
    """Scale the whole state of one node by 1.5: same velocity and b = rho/(2p),
    a 50 % density jump to its neighbours along every line through it."""
    p = q.copy()
    p[:, e, node] *= 1.5
    return p


def lines_in_series(q, phi, N, eps):
    """Per (element, direction, line): whether rho and b = rho/(2p) vary along
    the line by less than the kernel's sufficient bound 0.99 * 2 eps min (the
    premise of the series form), from the host state."""
    q = q.astype(np.float64)
    rho = q[0]
    p = 0.4 * (q[4] - 0.5 * (q[1] ** 2 + q[2] ** 2 + q[3] ** 2) / rho - rho * phi.astype(np.float64))
    b = rho / (2 * p)
    Nq = N + 1
    out = []
    for v in (rho, b):
        g = v.reshape(-1, Nq, Nq, Nq)           # [e][c][b][a], node a + Nq (b + Nq c)
        ok = []
        for ax in (3, 2, 1):                     # lines along xi1, xi2, xi3
            lo, hi = g.min(axis=ax), g.max(axis=ax)
            ok.append((hi - lo) < 0.99 * 2 * eps * lo)
        out.append(np.stack(ok))
    return out[0] & out[1]


def run(q, phi, geom, D, nbr=None):
    tq, tp, tg, tD = to_gpu(q, phi, geom, D)
    if nbr is None:
        out = esdg.volume_rhs(tq, tp, tg, tD)
    else:
        out = esdg.rhs(tq, tp, tg, tD, torch.from_numpy(np.ascontiguousarray(nbr, dtype=np.int32)).to(dev()))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def held_to_oracle(got, q, phi, geom, D, N, tol, nbr=None):
    if nbr is None:
        ref = oracle.volume_rhs(q, phi, geom, D, N)
        scale = np.abs(ref).reshape(5, -1).max(axis=1)
    else:
        ref, mag = oracle.rhs(q, phi, geom, D, nbr, N, with_magnitude=True)
        scale = np.abs(mag).reshape(5, -1).max(axis=1)
    err = np.abs(got.astype(np.float64) - ref).reshape(5, -1).max(axis=1) / scale
    assert np.all(np.isfinite(got))
    assert err.max() <= tol, err


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("N", [3, 4, 5, 7])
def test_volume_term_forms_agree(N, dtype):
    q, phi, geom, D, _ = smooth_workload(N, dtype)
    nelem = q.shape[1]
    e, node = 37 % nelem, ((N + 1) ** 3) // 2
    eps = 1e-2 if dtype == np.float64 else 1e-1
    qp = perturb(q, e, node)
    # base: every line in series range (the 200 m tall elements cross about
    # 1.6 % of density change vertically, inside the fp64 bound of 1.98 %);
    # perturbed: element e has lines in every direction that are not, so the
    # waves holding them switch to the general form
    assert lines_in_series(q, phi, N, eps).all()
    assert not lines_in_series(qp, phi, N, eps)[:, e].all(axis=(1, 2)).any()
    base = run(q, phi, geom, D)
    pert = run(qp, phi, geom, D)
    others = np.arange(nelem) != e
    print(f"[series] N={N} {np.dtype(dtype).name}: element {e} perturbed; "
          f"it changed {not np.array_equal(base[:, e], pert[:, e])}", flush=True)
    assert not np.array_equal(base[:, e], pert[:, e])
    assert np.array_equal(base[:, others], pert[:, others])
    held_to_oracle(base, q, phi, geom, D, N, TOL[dtype])
    held_to_oracle(pert, qp, phi, geom, D, N, TOL[dtype])


@pytest.mark.parametrize("N,dtype", [(4, np.float32), (4, np.float64), (5, np.float64), (7, np.float64),
                                     (7, np.float32)])
def test_whole_rhs_forms_agree(N, dtype):
    q, phi, geom, D, nbr = smooth_workload(N, dtype)
    nelem = q.shape[1]
    e, node = 37 % nelem, ((N + 1) ** 3) // 2
    base = run(q, phi, geom, D, nbr)
    qp = perturb(q, e, node)
    pert = run(qp, phi, geom, D, nbr)
    touched = {e} | {int(n) for n in nbr[e] if n >= 0}
    keep = np.array([i not in touched for i in range(nelem)])
    assert np.array_equal(base[:, keep], pert[:, keep])
    held_to_oracle(base, q, phi, geom, D, N, TOL[dtype], nbr)
    held_to_oracle(pert, qp, phi, geom, D, N, TOL[dtype], nbr)


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("N", [3, 4, 7])
def test_face_pair_forms_agree(N, dtype):
    """The whole right-hand side forms a face partner's logs, and takes the
    general form of its face pair, only in waves where some face pair is
    outside the series threshold.  A 50 % jump at one face node of element e
    (on its +xi1 face) sends the waves of its neighbour across that face to
    the general form for that end; every element other than e and its face
    neighbours, in those waves or not, keeps bitwise its clean result, the
    neighbour's result changes, and both runs meet the parity bar."""
    q, phi, geom, D, nbr = smooth_workload(N, dtype)
    nelem, Nq = q.shape[1], N + 1
    e = 37 % nelem
    node = N + Nq * (N // 2 + Nq * (N // 2))        # a = N, b = c = N/2
    partner = int(nbr[e][1])
    assert partner >= 0
    qp = perturb(q, e, node)
    base = run(q, phi, geom, D, nbr)
    pert = run(qp, phi, geom, D, nbr)
    touched = {e} | {int(n) for n in nbr[e] if n >= 0}
    keep = np.array([i not in touched for i in range(nelem)])
    print(f"[series] face pair N={N} {np.dtype(dtype).name}: element {e} node {node}, "
          f"partner {partner} changed {not np.array_equal(base[:, partner], pert[:, partner])}",
          flush=True)
    assert not np.array_equal(base[:, partner], pert[:, partner])
    assert np.array_equal(base[:, keep], pert[:, keep])
    held_to_oracle(base, q, phi, geom, D, N, TOL[dtype], nbr)
    held_to_oracle(pert, qp, phi, geom, D, N, TOL[dtype], nbr)


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("N", [4, 7])
def test_nan_state_stays_on_its_lines(N, dtype):
    """A NaN in one node's state reaches exactly the nodes that share one of
    its three lines (every pair on those lines involves it); every other
    value, in that element and elsewhere, is bitwise that of the clean run,
    whichever form the waves take."""
    q, phi, geom, D, _ = smooth_workload(N, dtype)
    nelem, Nq = q.shape[1], N + 1
    e, (a0, b0, c0) = 37 % nelem, (1, 2, 3 % Nq)
    node = a0 + Nq * (b0 + Nq * c0)
    qn = q.copy()
    qn[0, e, node] = np.nan
    base = run(q, phi, geom, D)
    got = run(qn, phi, geom, D)
    a, b, c = np.meshgrid(np.arange(Nq), np.arange(Nq), np.arange(Nq), indexing="ij")
    on_line = ((b == b0) & (c == c0)) | ((a == a0) & (c == c0)) | ((a == a0) & (b == b0))
    poisoned = np.zeros((nelem, Nq ** 3), dtype=bool)
    poisoned[e, (a + Nq * (b + Nq * c))[on_line]] = True
    assert np.isnan(got[:, poisoned]).all()
    assert np.array_equal(got[:, ~poisoned], base[:, ~poisoned])

