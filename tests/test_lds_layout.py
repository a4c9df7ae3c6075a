"""CPU checks of every launch shape in the launch table: the LDS node grid
(padded or not) stays inside the workgroup's LDS and maps nodes one to one,
every line task of a workgroup is taken by exactly one thread (also when the
last workgroup holds fewer elements), a line's slots follow its node
numbering, and the padded shapes cost no more LDS bank cycles than the
unpadded grid in the bank model that chose them."""
import pytest

from tests import lds_layout as L

TABLE = L.parse_launch_table()
CASES = sorted(TABLE)
LDS_PER_CU = 160 * 1024


def test_table_covers_every_order_and_precision():
    assert CASES == sorted((t, n) for t in ("double", "float") for n in range(1, 9))


@pytest.mark.parametrize("dtype,N", CASES)
def test_slots_in_bounds_and_one_to_one(dtype, N):
    s = L.Shape(N, TABLE[(dtype, N)], dtype)
    slots = [s.slot(t) for t in range(s.EPB * s.Np)]
    assert len(set(slots)) == len(slots)
    assert 0 <= min(slots) and max(slots) < s.slots
    assert s.lds_bytes <= LDS_PER_CU
    assert s.task_threads <= s.NT
    if dtype == "float":
        assert L.Shape(N, TABLE[(dtype, N)], dtype, split=True).lds_bytes <= LDS_PER_CU


def test_lds_sizes_match_the_compiled_kernels():
    # LDS bytes per workgroup the compiler reported for these kernels
    # (fp32, whole rhs on perturbation variables: with the split value)
    # and without it (full state variables)
    split = {1: 10240, 2: 15120, 3: 25600, 4: 23040, 5: 25920, 6: 23040, 7: 27648, 8: 34992}
    plain = {1: 9728, 2: 14364, 3: 24320, 4: 23040, 5: 25920, 6: 23040, 7: 25344, 8: 32076}
    for N in split:
        assert L.Shape(N, TABLE[("float", N)], "float", split=True).lds_bytes == split[N], N
        assert L.Shape(N, TABLE[("float", N)], "float").lds_bytes == plain[N], N


@pytest.mark.parametrize("dtype,N", CASES)
def test_every_line_once_also_in_a_ragged_workgroup(dtype, N):
    s = L.Shape(N, TABLE[(dtype, N)], dtype)
    for nvalid in range(1, s.EPB + 1):
        seen = []
        for thread in range(s.NT):
            if s.active(thread, nvalid):
                e, k, line = s.task(thread)
                assert 0 <= k <= 2 and 0 <= line < s.Nq2 and 0 <= e < nvalid
                seen.append((e, k, line, s.half(thread)))
        # each line once per lane, the lanes of a line adjacent
        assert sorted(seen) == sorted((e, k, line, h) for e in range(nvalid) for k in range(3)
                                      for line in range(s.Nq2) for h in range(s.lanes))
        if s.lanes == 2:
            for thread in range(0, s.task_threads, 2):
                assert s.task(thread) == s.task(thread + 1)


@pytest.mark.parametrize("dtype,N", CASES)
def test_line_slots_follow_node_numbering(dtype, N):
    s = L.Shape(N, TABLE[(dtype, N)], dtype)
    covered = set()
    for e in range(s.EPB):
        for k in range(3):
            for line in range(s.Nq2):
                nodes, slots = s.line_nodes(e, k, line)
                assert slots == [s.slot(n) for n in nodes]
                covered.update((k, n) for n in nodes)
    # each direction's lines pass through every node exactly once
    assert len(covered) == 3 * s.EPB * s.Np


@pytest.mark.parametrize("dtype,N", [c for c in CASES if any(
    TABLE[c][f] for f in ("row_pad", "plane_pad", "elem_pad"))])
def test_pads_cost_no_more_bank_cycles(dtype, N):
    cfg = TABLE[(dtype, N)]
    words = 2 if dtype == "double" else 1
    padded = L.Shape(N, cfg, dtype)
    plain = L.Shape(N, dict(cfg, row_pad=0, plane_pad=0, elem_pad=0), dtype)
    for banks in (32, 64):
        assert L.bank_cost(padded, words, banks)[0] <= L.bank_cost(plain, words, banks)[0]


def test_bank_model_sees_the_power_of_two_conflict():
    # N = 7, one element, direction-major: unpadded, direction-1 lines start
    # 64 bytes apart, so a 64-bank wave pays several times the
    # conflict-free cycles; one pad value per row brings it near one
    cfg = dict(zip(L.FIELDS, (1, 192, 0, 0, 0, 1, 1, 1, 1, 0, 0, 0, 0, 1)))
    plain = L.bank_cost(L.Shape(7, cfg), 2, 64)
    padded = L.bank_cost(L.Shape(7, dict(cfg, row_pad=1)), 2, 64)
    assert plain[0] >= 4 * plain[1]
    assert padded[0] <= 1.5 * padded[1]
