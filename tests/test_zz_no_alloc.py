"""The allocation-free integrals (esdg_integrals_noalloc_f64), called through
the C ABI, against the workspace entry point (esdg_integrals_f64) on the same
inputs: two calls in a row, the second on a smaller mesh, with full and with
perturbation variables, and under HIP graph capture.  The two entry points
run the same kernels with the same partition, so the sums agree bitwise."""
import numpy as np
import pytest

from entropy_stable_dg_amd import esdg
from entropy_stable_dg_amd import inputs as I

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def on_gpu(*arrays):
    return [torch.from_numpy(np.ascontiguousarray(a)).to(dev()) for a in arrays]


def both(q, phi, geom, w, ref=None):
    """(workspace entry, allocation-free entry) results, through the C ABI."""
    work = torch.empty(esdg.esdg_integrals_workspace_bytes() // 8, dtype=torch.float64,
                       device=dev())
    a = torch.full((3,), float("nan"), dtype=torch.float64, device=dev())
    b = torch.full((3,), float("nan"), dtype=torch.float64, device=dev())
    N = w.shape[0] - 1
    nelem = q.shape[1]
    h = torch.cuda.current_stream().cuda_stream
    rp = ref.data_ptr() if ref is not None else None
    assert esdg.esdg_integrals_f64(q.data_ptr(), rp, phi.data_ptr(), geom.data_ptr(), w.data_ptr(),
                                   N, nelem, work.data_ptr(), a.data_ptr(), h) == esdg.ESDG_OK
    assert esdg.esdg_integrals_noalloc_f64(q.data_ptr(), rp, phi.data_ptr(), geom.data_ptr(),
                                           w.data_ptr(), N, nelem, b.data_ptr(), h) == esdg.ESDG_OK
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy()


def test_two_calls_in_a_row_second_smaller():
    for name, ne in (("bubble", None), ("tiny", 5)):
        wl = I.make(name)
        q, phi, geom = wl.q, wl.phi, wl.geom
        if ne is not None:
            q, phi, geom = q[:, :ne], phi[:ne], geom[:, :ne]
        _, w = I.lgl(wl.N)
        tq, tp, tg, tw = on_gpu(q, phi, geom, w)
        a, b = both(tq, tp, tg, tw)
        print(f"[no-alloc] {name} ({tq.shape[1]} elements): {a} / {b}", flush=True)
        assert np.all(np.isfinite(a)) and np.array_equal(a, b), (name, a, b)


def test_perturbation_variables_two_calls():
    for name in ("baroclinic", "tiny"):
        wl, qp, ref = I.make_perturbed(name)
        _, w = I.lgl(wl.N)
        tq, tr, tp, tg, tw = on_gpu(qp, ref, wl.phi, wl.geom, w)
        a, b = both(tq, tp, tg, tw, ref=tr)
        assert np.all(np.isfinite(a)) and np.array_equal(a, b), (name, a, b)


def test_argument_errors_before_any_launch():
    p = 0x10000000
    f = esdg.esdg_integrals_noalloc_f64
    assert f(p, 0, p, p, p, 0, 1, p + 0x1000000, 0) == esdg.ESDG_ERR_ORDER
    assert f(p, 0, p, p, p, 4, -1, p + 0x1000000, 0) == esdg.ESDG_ERR_NELEM
    assert f(p, 0, p, p, p, 4, 10, 0, 0) == esdg.ESDG_ERR_NULL


def test_under_graph_capture():
    """Captured once and replayed with eager work in between: every replay
    equals an eager call of the workspace entry point on the updated state."""
    wl = I.make("tiny")
    _, w = I.lgl(wl.N)
    tq, tp, tg, tw = on_gpu(wl.q, wl.phi, wl.geom, w)
    out = torch.zeros(3, dtype=torch.float64, device=dev())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        esdg.integrals_noalloc(tq, tp, tg, tw, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        esdg.integrals_noalloc(tq, tp, tg, tw, out)
    base = tq.clone()
    for rep in range(4):
        tq.copy_(base)
        tq[0].mul_(1.0 + 1e-3 * rep)
        want = esdg.integrals(tq, tp, tg, tw)
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), (rep, out, want)
