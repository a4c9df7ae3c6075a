"""The analytic work model: the per-pair and per-node FLOP tallies are the
sums of their itemised steps under the stated weights, and the figures the
benchmark reports follow from them."""
from entropy_stable_dg_amd import perfmodel as P


def test_weights_of_the_convention():
    assert P.WEIGHT == {"add": 1, "mul": 1, "fma": 2, "rcp": 1, "log": 1}


def test_pair_tally():
    by_op = {}
    for _, ops in P.PAIR_STEPS:
        for op, n in ops.items():
            by_op[op] = by_op.get(op, 0) + n
    # series form of the pair: 12 adds, 20 multiplies, 31 fused multiply-adds, 1 reciprocal
    assert by_op == {"add": 12, "mul": 20, "fma": 31, "rcp": 1}
    assert P.FLOP_PER_PAIR == 12 + 20 + 2 * 31 + 1 == 95


def test_node_tally():
    assert P.FLOP_PER_NODE == 44
    assert P.FLOP_PER_PARTNER_NODE == 44 - 1 - 10 - 5


def test_per_dof_figures():
    # pairs per element 3 Nq^2 Nq N/2; per DOF 3N/2
    for N in range(1, 9):
        assert P.pairs_per_element(N) == 3 * (N + 1) ** 3 * N // 2
        assert abs(P.flops_per_dof(N) - (1.5 * N * 95 + 44)) < 1e-12
    assert P.flops_per_dof(4) == 614.0
    assert abs(P.arithmetic_intensity(4, "f64") - 614.0 / 168.0) < 1e-12
    assert P.bytes_per_dof("f64") == 168 and P.bytes_per_dof("f32") == 84


def test_phase_floors():
    from entropy_stable_dg_amd import perfmodel as P

    # the issue model reproduces the published fp64 vector peak: 1024 SIMDs
    # x 16 lanes per cycle x 2 FLOP per FMA x 2.4 GHz
    lanes_per_cycle = 64 / P.CYCLES_PER_WAVE_VALU
    assert abs(P.SIMDS * lanes_per_cycle * 2 * P.CLOCK_GHZ / 1e3 - P.PEAK_FP64_VECTOR_TFLOPS) < 0.1
    f = P.phase_floors(86.016e6, 5.65e6, 5000.0, 25.0)
    assert abs(f["hbm_us"] - 17.2032) < 1e-9
    assert abs(f["valu_us"] - 5.65e6 * 4 / (1024 * 2.4e9) * 1e6) < 1e-9
    assert f["sum_us"] == f["hbm_us"] + f["valu_us"] and f["max_us"] == f["hbm_us"]
    assert abs(f["measured_over_sum"] - 25.0 / f["sum_us"]) < 1e-12
