"""Host side of the timeline probe: the phase summary of a known synthetic
timeline (no GPU)."""
import numpy as np

from entropy_stable_dg_amd import probe


def test_timeline_phases_of_a_two_round_schedule():
    # 4 workgroups on a 100 MHz clock: two start at 0 and load 5 us, compute
    # 3 us, store 1 us; two start when those end (9 us) and load 2 us,
    # compute 3 us, store 1 us
    tick = 100  # ticks per us
    rows = []
    for w, (t0, a, b, c) in enumerate([(0, 5, 3, 1), (0.2, 5, 3, 1), (9, 2, 3, 1), (9.1, 2, 3, 1)]):
        t = np.cumsum([t0, a, b, c]) * tick
        rows.append([int(round(x)) + 1000 for x in t] + [w % 2, w])
    m = np.array(rows, dtype=np.int64)
    ph = probe.timeline_phases(m, 100e6, bins=30)
    assert ph["workgroups"] == 4 and ph["first_round"] == 2 and ph["compute_units"] == 2
    assert abs(ph["span_us"] - 15.1) < 1e-9
    assert abs(ph["first"]["load_stage_us"] - 5) < 1e-9
    assert abs(ph["later"]["load_stage_us"] - 2) < 1e-9
    assert abs(ph["first"]["pairs_us"] - 3) < 1e-9 and abs(ph["later"]["store_us"] - 1) < 1e-9
    assert abs(ph["later_starts_us"][0] - 9) < 1e-9
    # the last nodes are staged at 9.1 + 2 us; the span ends at 15.1 us
    assert abs(ph["drain_us"] - (15.1 - 11.1)) < 1e-9
    occ = {round(x, 6): (a, b, c) for x, a, b, c in ph["occupancy"]}
    # at 6.04 us both first workgroups compute; at 10.07 both later ones load
    x = [k for k in occ if 6.0 < k < 6.6][0]
    assert occ[x] == (0, 2, 0)
    x = [k for k in occ if 10.0 < k < 10.6][0]
    assert occ[x] == (2, 0, 0)
