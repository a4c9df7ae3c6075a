"""The HBM streaming probes compute what they claim (the bandwidth they report
is only meaningful if they move the bytes they count)."""
import pytest

from entropy_stable_dg_amd import probe

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [1, 2, 6, 1000, 262145, 262146])
def test_stream81_and_copy(n):
    assert torch.cuda.is_available()
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(n)
    src = torch.rand(8 * n, generator=g, dtype=torch.float64).to(dev)
    dst = torch.full((n,), -1.0, dtype=torch.float64, device=dev)
    h = torch.cuda.current_stream(dev).cuda_stream
    assert probe.esdg_probe_stream81_f64(src.data_ptr(), dst.data_ptr(), n, h) == 0
    torch.cuda.synchronize()
    ref = src.view(8, n).cpu()
    expect = ref[0].clone()
    for j in range(1, 8):
        expect += ref[j]          # same summation order as the kernel
    assert torch.equal(dst.cpu(), expect)
    if n % 2 == 0:   # the 32-byte-lane form (even n, aligned arrays)
        wide = torch.full((n,), -1.0, dtype=torch.float64, device=dev)
        assert probe.esdg_probe_stream81_wide_f64(src.data_ptr(), wide.data_ptr(), n, h) == 0
        torch.cuda.synchronize()
        assert torch.equal(wide.cpu(), expect)
    out = torch.empty(n, dtype=torch.float64, device=dev)
    assert probe.esdg_probe_copy_f64(src.data_ptr(), out.data_ptr(), n, h) == 0
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), ref[0])


def test_stream81_bandwidth_is_positive():
    bw = probe.stream81_bandwidth(n=1 << 22, reps=5)
    print(f"[probe] stream 8:1 fp64 at 4M doubles per array: {bw:.0f} GB/s", flush=True)
    assert 100.0 < bw < 20000.0
    bw = probe.stream81_bandwidth(n=1 << 22, reps=5, wide=True)
    print(f"[probe] same, 32-byte lanes: {bw:.0f} GB/s", flush=True)
    assert 100.0 < bw < 20000.0


@pytest.mark.parametrize("name,whole", [("tiny", False), ("bubble", False), ("bubble_f32", False),
                                        ("bubble", True), ("high_order", False)])
def test_timeline_is_the_library_kernel_with_ordered_marks(name, whole):
    """The timeline probe runs the library's kernel: its output equals the
    library's bitwise; every workgroup's marks are in phase order, every batch
    is taken once, and the first round fills every compute unit."""
    import numpy as np

    from entropy_stable_dg_amd import esdg, inputs

    dev = torch.device("cuda:0")
    wl = inputs.make(name)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    q, phi, geom, D, nbr = t(wl.q), t(wl.phi), t(wl.geom), t(wl.D), t(wl.nbr)
    print(f"[probe] timeline {name} whole={whole}", flush=True)
    want = esdg.rhs(q, phi, geom, D, nbr) if whole else esdg.volume_rhs(q, phi, geom, D)
    got, marks = probe.timeline(q, phi, geom, D, nbr if whole else None)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    m = marks.cpu().numpy()
    nwg = probe.esdg_probe_timeline_workgroups(wl.N, wl.nelem, int(wl.q.dtype == np.float64))
    assert m.shape == (nwg, probe.MARK_VALUES)
    assert np.all(np.diff(m[:, :4], axis=1) >= 0)
    assert sorted(m[:, 5].tolist()) == list(range(nwg))
    khz = probe.esdg_probe_wall_clock_khz()
    assert khz > 0
    ph = probe.timeline_phases(m, khz * 1e3)
    print(f"[probe] {name}: {nwg} workgroups, span {ph['span_us']:.1f} us, first round "
          f"{ph['first_round']}, compute units {ph['compute_units']}", flush=True)
    if nwg >= 768:   # more workgroups than one round: every compute unit takes some
        assert ph["compute_units"] == 256
