"""Accuracy of the volume kernel's per-node logarithm, against the error bound
its construction gives.

The log means of the two-point flux (page: GPU Performance of an
Entropy-Stable DG Euler Solver with Non-Conservative Terms, section on the
entropy-conservative flux; the log mean and its series branch) take the
difference of two node logs when the states differ by more than the series
threshold.  The fp64 kernel uses its own log (a frexp range reduction and an
odd atanh series with one Newton-refined reciprocal); its absolute error is
bounded by about 1.1e-15 from the reciprocal (relative 3e-15 on t, |t| <=
0.1716, ln m ~ 2t) plus the rounding of the final sum, i.e. a couple of ulp
of |ln x|.  The test allows 2e-15 + 2 ulp(|ln x|) against an 80-bit
extended-precision log over the whole normal range.

The fp32 kernel uses the hardware base-2 log scaled by ln 2; it is held to
2e-7 absolute + 4 ulp(|ln x|): differences of logs only enter where the
states differ by more than 10 percent (log difference at least 0.2), so a
2e-7 error there is 1e-6 relative, far inside the fp32 parity tolerance.
"""
import numpy as np
import pytest

from entropy_stable_dg_amd import probe

torch = pytest.importorskip("torch")


def _inputs(dtype, n, seed):
    rng = np.random.default_rng(seed)
    fi = np.finfo(dtype)
    lo, hi = np.log2(fi.tiny), np.log2(fi.max) - 1e-3
    parts = [
        np.exp2(rng.uniform(lo, hi, n)),                      # whole normal range
        rng.uniform(0.5, 2.0, n),                              # around 1
        np.sqrt(2.0) * (1.0 + rng.uniform(-1e-6, 1e-6, n)),   # the reduction's switch point
        1.0 + rng.uniform(-1e-9, 1e-9, n),                     # very close to 1
        rng.uniform(1e-3, 1e3, n),                             # the kernel's range (rho, scaled b)
        np.exp2(np.arange(int(lo) + 1, int(hi))),              # exact powers of two
        np.array([1.0, fi.tiny, 0.5, 2.0]),
    ]
    x = np.concatenate(parts).astype(dtype)
    x = x[np.isfinite(x) & (x >= fi.tiny)]
    return x


def _run(x, entry, dtype):
    dev = torch.device("cuda:0")
    xd = torch.from_numpy(x).to(dev)
    yd = torch.full_like(xd, float("nan"))
    h = torch.cuda.current_stream(dev).cuda_stream
    assert entry(xd.data_ptr(), yd.data_ptr(), x.size, h) == 0
    torch.cuda.synchronize()
    return yd.cpu().numpy()


@pytest.mark.gpu
def test_node_log_f64():
    assert torch.cuda.is_available()
    x = _inputs(np.float64, 200_000, 11)
    y = _run(x, probe.esdg_probe_node_log_f64, np.float64)
    ref = np.log(x.astype(np.longdouble))
    err = np.abs(y.astype(np.longdouble) - ref).astype(np.float64)
    bound = 2e-15 + 2.0 * np.spacing(np.abs(ref.astype(np.float64)))
    worst = int(np.argmax(err / bound))
    print(f"[node_log f64] n={x.size} max abs err {err.max():.3e}, worst err/bound "
          f"{err[worst] / bound[worst]:.3f} at x={x[worst]!r}", flush=True)
    assert np.all(err <= bound)
    assert y[x == 1.0].tolist() == [0.0] * int((x == 1.0).sum())


@pytest.mark.gpu
def test_node_log_f32():
    assert torch.cuda.is_available()
    x = _inputs(np.float32, 200_000, 12)
    y = _run(x, probe.esdg_probe_node_log_f32, np.float32)
    ref = np.log(x.astype(np.longdouble))
    err = np.abs(y.astype(np.longdouble) - ref).astype(np.float64)
    bound = 2e-7 + 4.0 * np.spacing(np.abs(ref.astype(np.float32))).astype(np.float64)
    worst = int(np.argmax(err / bound))
    print(f"[node_log f32] n={x.size} max abs err {err.max():.3e}, worst err/bound "
          f"{err[worst] / bound[worst]:.3f} at x={x[worst]!r}", flush=True)
    assert np.all(err <= bound)


def test_node_log_host_checks():
    """Argument checks run on the host before any launch (no GPU needed)."""
    for entry in (probe.esdg_probe_node_log_f64, probe.esdg_probe_node_log_f32):
        assert entry(0, 0, 4, 0) == -1          # null pointers with work to do
        assert entry(0, 0, -1, 0) == -3         # negative size
        assert entry(0, 0, 0, 0) == 0           # empty: nothing launched
