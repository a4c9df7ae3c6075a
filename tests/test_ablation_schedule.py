"""Host-side checks of libesdg_ablation (no kernel launch):

* the library exports what include/esdg_ablation.h declares and rejects bad
  arguments before any HIP call;
* the half-sweep schedules of the ablation kernels -- upper-triangular,
  cyclic indexing (Eq. 6) and weighted cyclic (Fig. 1b) -- written out here as
  the kernels take them (which thread evaluates which pair at which step, and
  which thread receives the partner contribution), pinned to the evaluation
  counts of Fig. 1 and Eq. 6, and checked to give every unordered pair a total
  weight of one in both orientations, with no exchange slot written twice in
  one step;
* every LDS and global index the ablation kernels form stays inside its
  buffer, for each order the library accepts.
"""
import os
import re
from collections import defaultdict

import pytest

from entropy_stable_dg_amd import ablation as abl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "esdg_ablation.h")
SOURCE = os.path.join(ROOT, "entropy_stable_dg_amd", "csrc", "ablation.hip")
GOLDEN = os.path.join(ROOT, "tests", "golden", "fig1_thread_assignment.txt")


def golden():
    rows = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            key, *vals = line.split()
            rows[key] = vals
    return rows


# --- schedules (0-based thread index a on a line of Nq nodes) ------------------
def steps(variant, Nq):
    return Nq - 1 if variant == abl.ESDG_ABL_SYM_UPPER else Nq // 2


def works(variant, Nq, a, s):
    """(evaluates the pair (a, (a+s) mod Nq) at step s, weight)."""
    even = Nq % 2 == 0
    if variant == abl.ESDG_ABL_SYM_UPPER:
        return a + s < Nq, 1.0
    if variant == abl.ESDG_ABL_SYM_INDEXED:
        return not (even and s == Nq // 2 and a >= Nq // 2), 1.0
    return True, (0.5 if even and s == Nq // 2 else 1.0)


def receives(variant, Nq, a, s):
    """Whether node a reads its exchange slot after step s."""
    even = Nq % 2 == 0
    frm = (a - s) % Nq
    if variant == abl.ESDG_ABL_SYM_UPPER:
        return a - s >= 0
    if variant == abl.ESDG_ABL_SYM_INDEXED:
        return not (even and s == Nq // 2 and frm >= Nq // 2)
    return True


SCHEDULES = (abl.ESDG_ABL_SYM_UPPER, abl.ESDG_ABL_SYM_INDEXED, abl.ESDG_ABL_SYM_WEIGHTED)


def evaluations(variant, Nq):
    return [sum(works(variant, Nq, a, s)[0] for s in range(1, steps(variant, Nq) + 1))
            for a in range(Nq)]


def test_schedule_source_matches_this_model():
    """The predicates written above are the ones in ablation.hip."""
    src = open(SOURCE).read()
    for frag in ("work = ik + s < Nq;",
                 "work = !(even && s == Nq / 2 && ik >= Nq / 2);",
                 "if (even && s == Nq / 2) w = 0.5;",
                 "recv = ik - s >= 0;",
                 "recv = !(even && s == Nq / 2 && from >= Nq / 2);",
                 "const int nsteps = (variant == SYM_UPPER) ? Nq - 1 : Nq / 2;",
                 "const int l = (ik + s) % Nq;",
                 "const int from = (ik - s + Nq) % Nq;"):
        assert frag in src, frag


def test_fig1_upper_triangular_counts():
    g = golden()
    assert evaluations(abl.ESDG_ABL_SYM_UPPER, 4) == [int(v) for v in g["fig1a_N3_evaluations"]]


def test_fig1_weighted_cyclic_counts_and_antipodes():
    g = golden()
    assert evaluations(abl.ESDG_ABL_SYM_WEIGHTED, 4) == [int(v) for v in g["fig1b_N3_evaluations"]]
    halves = set()
    for a in range(4):
        for s in range(1, steps(abl.ESDG_ABL_SYM_WEIGHTED, 4) + 1):
            ok, w = works(abl.ESDG_ABL_SYM_WEIGHTED, 4, a, s)
            if ok and w == 0.5:
                halves.add(frozenset((a + 1, (a + s) % 4 + 1)))   # 1-based as on the page
    want = {frozenset(map(int, p.split("-"))) for p in g["fig1b_N3_antipodal"]}
    assert halves == want


@pytest.mark.parametrize("N", [2, 3, 4, 7])
def test_eq6_counts(N):
    assert evaluations(abl.ESDG_ABL_SYM_INDEXED, N + 1) == [int(v) for v in golden()[f"eq6_N{N}_evaluations"]]


@pytest.mark.parametrize("variant", SCHEDULES)
@pytest.mark.parametrize("Nq", range(2, 10))
def test_every_pair_has_weight_one_each_way(variant, Nq):
    """Own and partner contributions of every ordered pair (i, j), i != j, sum
    to weight one; exchange slots are written once per step and read by
    their owner exactly when written."""
    weight = defaultdict(float)
    for s in range(1, steps(variant, Nq) + 1):
        written = defaultdict(int)
        for a in range(Nq):
            ok, w = works(variant, Nq, a, s)
            if ok:
                l = (a + s) % Nq
                assert l != a
                weight[(a, l)] += w        # own contribution of a (D[a][l])
                weight[(l, a)] += w        # partner contribution to l (D[l][a])
                written[l] += 1
        for a in range(Nq):
            assert written[a] <= 1
            assert receives(variant, Nq, a, s) == (written[a] == 1), (variant, Nq, s, a)
    for i in range(Nq):
        for j in range(Nq):
            if i != j:
                assert weight[(i, j)] == pytest.approx(1.0), (variant, Nq, i, j)


@pytest.mark.parametrize("N", abl.ORDERS)
def test_index_bounds(N):
    """Replay of the kernels' index arithmetic for one element: node slot t,
    the k-line partner slot and the per-direction line position stay inside
    the Np-node LDS arrays; threads past Np take no node work."""
    Nq = N + 1
    Nq2, Np = Nq * Nq, Nq ** 3
    NT = (Np + 63) // 64 * 64
    assert NT % 64 == 0 and NT <= 1024
    for t in range(NT):
        node = t < Np
        a, b, c = t % Nq, (t // Nq) % Nq, t // Nq2
        for k in range(3):
            ik = (a, b, c)[k]
            stride = (1, Nq, Nq2)[k]
            if not node:
                continue
            assert 0 <= ik < Nq
            for l in range(Nq):
                sl = t + (l - ik) * stride
                assert 0 <= sl < Np
                # sl is the node of the same line with index l
                assert (sl % Nq, (sl // Nq) % Nq, sl // Nq2)[k] == l
    # LDS: staged values x Np + exchange slots x Np doubles within 160 KiB
    src = open(SOURCE).read()
    kprim = int(re.search(r"kPrim = (\d+)", src).group(1))
    kxch = int(re.search(r"kXch = (\d+);", src).group(1))
    assert (kprim + kxch) * Np * 8 <= 160 * 1024


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(esdg_\w+)\s*\(", text)))


def test_header_and_exports():
    assert declared_functions() == sorted(abl.EXPORTS)
    abl.load()
    out = os.popen(f"nm -D --defined-only {abl.ABLATION_LIB_PATH}").read()
    syms = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for name in abl.EXPORTS:
        assert name in syms


def test_variant_names():
    names = [abl.esdg_ablation_name(v) for v in range(abl.ESDG_ABL_COUNT)]
    assert len(set(names)) == abl.ESDG_ABL_COUNT and "unknown" not in names
    assert abl.esdg_ablation_name(-1) == "unknown"
    assert abl.esdg_ablation_name(abl.ESDG_ABL_COUNT) == "unknown"
    fused = [abl.esdg_ablation_name(v | abl.ESDG_ABL_FUSE_FLAG) for v in range(abl.ESDG_ABL_COUNT)]
    assert all(n.endswith("fused directions") for n in fused)
    assert fused[abl.ESDG_ABL_FUSED] == names[abl.ESDG_ABL_FUSED]
    assert abl.esdg_ablation_name(abl.ESDG_ABL_COUNT | abl.ESDG_ABL_FUSE_FLAG) == "unknown"


A, B, C, Dp, R = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


def test_argument_errors():
    f = abl.esdg_ablation_volume_rhs_f64
    assert f(-1, A, B, C, Dp, 4, 1, R, 0) == abl.ESDG_ERR_VARIANT
    assert f(abl.ESDG_ABL_COUNT, A, B, C, Dp, 4, 1, R, 0) == abl.ESDG_ERR_VARIANT
    assert f(abl.ESDG_ABL_COUNT | abl.ESDG_ABL_FUSE_FLAG, A, B, C, Dp, 4, 1, R, 0) == abl.ESDG_ERR_VARIANT
    assert f(0x200, A, B, C, Dp, 4, 1, R, 0) == abl.ESDG_ERR_VARIANT
    assert f(abl.ESDG_ABL_FUSE_FLAG, A, B, C, Dp, 5, 1, R, 0) == -2
    for N in (0, 1, 2, 5, 6, 8, 9):
        assert f(0, A, B, C, Dp, N, 1, R, 0) == -2
    assert f(0, A, B, C, Dp, 4, -1, R, 0) == -3
    assert f(0, A, B, C, Dp, 4, 2 ** 40, R, 0) == -3   # more workgroups than one launch holds
    assert f(0, 0, 0, 0, 0, 4, 0, 0, 0) == 0
    for i in range(5):
        args = [A, B, C, Dp, R]
        args[i] = 0
        assert f(0, args[0], args[1], args[2], args[3], 4, 10, args[4], 0) == -1
    assert f(0, A, B, C, Dp, 3, 100, A + 8, 0) == -5
    assert f(0, A, B, C, Dp, 3, 100, Dp, 0) == -5
