"""GPU parity of every optimisation-ladder variant (libesdg_ablation) against
the CPU oracle, at each order the ladder covers, with one launch per
direction and with the directions fused, to the production kernel's fp64 bar (per field, max |rhs - oracle| / max |oracle| <= 1e-11)."""
import numpy as np
import pytest

import oracle
from entropy_stable_dg_amd import ablation as abl
from entropy_stable_dg_amd import inputs as I
from tests.test_gpu_parity import TOL, check, dev, random_workload, to_gpu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

VARIANTS = list(range(abl.ESDG_ABL_COUNT)) + [v | abl.ESDG_ABL_FUSE_FLAG for v in range(abl.ESDG_ABL_COUNT - 1)]


def ablation_rhs(variant, q, phi, geom, D):
    tq, tp, tg, tD = to_gpu(q, phi, geom, D)
    out = abl.volume_rhs(variant, tq, tp, tg, tD)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.fixture(scope="module")
def cases():
    return {}


def case(cases, N):
    if N not in cases:
        q, phi, geom, D = random_workload(N, nelem_xyz=(3, 2, 2), seed=40 + N)
        cases[N] = (q, phi, geom, D, oracle.volume_rhs(q, phi, geom, D, N))
    return cases[N]


@pytest.mark.parametrize("N", abl.ORDERS)
@pytest.mark.parametrize("variant", VARIANTS)
def test_variant_parity(cases, variant, N):
    q, phi, geom, D, ref = case(cases, N)
    print(f"[ablation] variant {variant} ({abl.esdg_ablation_name(variant)}) N={N}", flush=True)
    got = ablation_rhs(variant, q, phi, geom, D)
    check(got, ref, TOL[np.float64], f"ablation {variant:#x} N={N}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_variant_bubble(variant):
    """The bubble workload (N = 4, 4096 elements), against the oracle."""
    wl = I.make("bubble")
    print(f"[ablation] variant {variant} bubble", flush=True)
    got = ablation_rhs(variant, wl.q, wl.phi, wl.geom, wl.D)
    ref = oracle.volume_rhs(wl.q, wl.phi, wl.geom, wl.D, wl.N)
    check(got, ref, TOL[np.float64], f"ablation {variant:#x} bubble")


def test_variant_rejected():
    wl = I.make("tiny")
    tq, tp, tg, tD = to_gpu(wl.q, wl.phi, wl.geom, wl.D)
    with pytest.raises(Exception, match="status -6"):
        abl.volume_rhs(abl.ESDG_ABL_COUNT, tq, tp, tg, tD)


def test_ladder_at_the_timed_size():
    """The configuration bench.py times the ladder on: the bubble workload
    tiled 64 times (N = 4, 262,144 elements).  The kernels are element-local
    and free of atomics, so every tile must reproduce the single bubble's
    result bitwise; the single bubble is checked against the oracle in
    test_variant_bubble.  A sample of tiles (first, middle, last) is compared."""
    wl = I.make("bubble")
    tq, tp, tg, tD = to_gpu(wl.q, wl.phi, wl.geom, wl.D)
    reps = 64
    big = (tq.repeat(1, reps, 1), tp.repeat(reps, 1), tg.repeat(1, reps, 1))
    ne = wl.nelem
    for variant in [abl.ESDG_ABL_BASELINE, abl.ESDG_ABL_CONTRA, abl.ESDG_ABL_SYM_UPPER,
                    abl.ESDG_ABL_SYM_WEIGHTED | abl.ESDG_ABL_FUSE_FLAG, abl.ESDG_ABL_FUSED]:
        print(f"[ablation] variant {variant:#x} at 262,144 elements", flush=True)
        small = abl.volume_rhs(variant, tq, tp, tg, tD)
        out = abl.volume_rhs(variant, big[0], big[1], big[2], tD)
        torch.cuda.synchronize()
        for t in (0, reps // 2, reps - 1):
            assert torch.equal(out[:, t * ne:(t + 1) * ne], small), (variant, t)
        del out
    del big
    torch.cuda.empty_cache()


@pytest.mark.parametrize("N", abl.TWO_LANE_ORDERS)
def test_two_lane_variant_parity(N):
    """Two lanes per line with the cross-lane exchange (N = 5, 7): every
    order it covers on a random warped mesh, a ragged count and the N = 7
    high-order workload, against the oracle."""
    q, phi, geom, D = random_workload(N, nelem_xyz=(3, 2, 2), seed=90 + N)
    tq, tp, tg, tD = to_gpu(q, phi, geom, D)
    got = abl.two_lane_volume_rhs(tq, tp, tg, tD)
    torch.cuda.synchronize()
    check(got.cpu().numpy(), oracle.volume_rhs(q, phi, geom, D, N), TOL[np.float64],
          f"two lanes N={N}")
    ne = 5
    got = abl.two_lane_volume_rhs(tq[:, :ne].contiguous(), tp[:ne].contiguous(),
                                  tg[:, :ne].contiguous(), tD)
    torch.cuda.synchronize()
    check(got.cpu().numpy(), oracle.volume_rhs(q[:, :ne], phi[:ne], geom[:, :ne], D, N),
          TOL[np.float64], f"two lanes N={N} {ne} elements")


def test_two_lane_variant_high_order_workload():
    wl = I.make("high_order")
    tq, tp, tg, tD = to_gpu(wl.q, wl.phi, wl.geom, wl.D)
    got = abl.two_lane_volume_rhs(tq, tp, tg, tD)
    torch.cuda.synchronize()
    check(got.cpu().numpy(), oracle.volume_rhs(wl.q, wl.phi, wl.geom, wl.D, wl.N),
          TOL[np.float64], "two lanes, high order")
