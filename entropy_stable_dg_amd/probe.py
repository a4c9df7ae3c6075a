"""Binding of libesdg_probe.so (HBM streaming probes, measurement only), with
the C functions of include/esdg_probe.h under the same names."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(HERE, "libesdg_probe.so")
_STREAMS = ("esdg_probe_stream81_f64", "esdg_probe_stream81_wide_f64", "esdg_probe_node_log_f64",
            "esdg_probe_node_log_f32", "esdg_probe_copy_f64")
EXPORTS = _STREAMS + ("esdg_probe_timeline_workgroups", "esdg_probe_timeline_f64",
                      "esdg_probe_timeline_f32", "esdg_probe_wall_clock_khz")
MARK_VALUES = 6   # per workgroup: entry, staged, pairs done, stores issued, CU id, batch

_lib = None


def load(path: str = PROBE_LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None and path == PROBE_LIB_PATH:
        return _lib
    try:  # share the HIP runtime torch ships
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m entropy_stable_dg_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    for name in _STREAMS:
        fn = getattr(lib, name)
        fn.restype = ci
        fn.argtypes = [vp, vp, i64, vp]
    lib.esdg_probe_timeline_workgroups.restype = i64
    lib.esdg_probe_timeline_workgroups.argtypes = [ci, i64, ci]
    for name in ("esdg_probe_timeline_f64", "esdg_probe_timeline_f32"):
        fn = getattr(lib, name)
        fn.restype = ci
        fn.argtypes = [vp, vp, vp, vp, vp, ci, i64, vp, vp, vp]
    lib.esdg_probe_wall_clock_khz.restype = ci
    lib.esdg_probe_wall_clock_khz.argtypes = []
    if path == PROBE_LIB_PATH:
        _lib = lib
    return lib


def esdg_probe_stream81_f64(src: int, dst: int, n: int, stream: int = 0) -> int:
    return load().esdg_probe_stream81_f64(src, dst, n, stream)


def esdg_probe_stream81_wide_f64(src: int, dst: int, n: int, stream: int = 0) -> int:
    return load().esdg_probe_stream81_wide_f64(src, dst, n, stream)


def esdg_probe_node_log_f64(x: int, y: int, n: int, stream: int = 0) -> int:
    return load().esdg_probe_node_log_f64(x, y, n, stream)


def esdg_probe_node_log_f32(x: int, y: int, n: int, stream: int = 0) -> int:
    return load().esdg_probe_node_log_f32(x, y, n, stream)


def esdg_probe_copy_f64(src: int, dst: int, n: int, stream: int = 0) -> int:
    return load().esdg_probe_copy_f64(src, dst, n, stream)


def esdg_probe_timeline_workgroups(N: int, nelem: int, fp64: int) -> int:
    return load().esdg_probe_timeline_workgroups(N, nelem, fp64)


def esdg_probe_timeline_f64(q: int, phi: int, geom: int, D: int, nbr, N: int, nelem: int,
                            rhs: int, marks: int, stream: int = 0) -> int:
    return load().esdg_probe_timeline_f64(q, phi, geom, D, nbr, N, nelem, rhs, marks, stream)


def esdg_probe_timeline_f32(q: int, phi: int, geom: int, D: int, nbr, N: int, nelem: int,
                            rhs: int, marks: int, stream: int = 0) -> int:
    return load().esdg_probe_timeline_f32(q, phi, geom, D, nbr, N, nelem, rhs, marks, stream)


def esdg_probe_wall_clock_khz() -> int:
    return load().esdg_probe_wall_clock_khz()


def stream81_bandwidth(n: int = 1 << 25, reps: int = 20, wide: bool = False) -> float:
    """Empirical HBM bandwidth (GB/s) of the 8-read:1-write fp64 stream on
    cuda:0: 9 * 8 * n bytes per launch, reps back-to-back launches; `wide`
    selects the 32-bytes-per-lane form."""
    import torch

    dev = torch.device("cuda:0")
    src = torch.ones(8 * n, dtype=torch.float64, device=dev)
    dst = torch.empty(n, dtype=torch.float64, device=dev)
    h = torch.cuda.current_stream(dev).cuda_stream
    fn = esdg_probe_stream81_wide_f64 if wide else esdg_probe_stream81_f64
    for _ in range(3):
        if fn(src.data_ptr(), dst.data_ptr(), n, h) != 0:
            raise RuntimeError("stream probe launch failed")
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        fn(src.data_ptr(), dst.data_ptr(), n, h)
    t1.record()
    torch.cuda.synchronize()
    sec = t0.elapsed_time(t1) * 1e-3 / reps
    return 9 * 8 * n / sec / 1e9


def timeline(q, phi, geom, D, nbr=None, rhs=None, marks=None, stream=None):
    """One launch of the volume kernel (or, with nbr, the whole right-hand
    side) with phase marks, on device tensors in the library's layouts.
    Returns (rhs, marks [workgroups][6] uint64 as an int64 tensor)."""
    import torch

    N = round(q.shape[2] ** (1.0 / 3.0)) - 1
    nelem = q.shape[1]
    fp64 = q.dtype == torch.float64
    nwg = esdg_probe_timeline_workgroups(N, nelem, int(fp64))
    if nwg < 0:
        raise ValueError(f"no launch shape for N={N}, nelem={nelem}")
    if rhs is None:
        rhs = torch.empty_like(q)
    if marks is None:
        marks = torch.zeros((max(nwg, 1), MARK_VALUES), dtype=torch.int64, device=q.device)
    if marks.numel() < nwg * MARK_VALUES:
        raise ValueError("marks holds fewer than 6 values per workgroup")
    h = (stream or torch.cuda.current_stream(q.device)).cuda_stream
    fn = esdg_probe_timeline_f64 if fp64 else esdg_probe_timeline_f32
    st = fn(q.data_ptr(), phi.data_ptr(), geom.data_ptr(), D.data_ptr(),
            None if nbr is None else nbr.data_ptr(), N, nelem, rhs.data_ptr(), marks.data_ptr(), h)
    if st != 0:
        raise RuntimeError(f"timeline probe failed with status {st}")
    return rhs, marks[:nwg]


def timeline_phases(marks, clock_hz: float, bins: int = 24) -> dict:
    """Phase statistics of one timeline (marks as timeline() returns them,
    numpy [workgroups][6]; times from the device wall clock at clock_hz):
    durations of loading and staging (phase A), the line pairs (B) and the
    partials and stores (C, D) per workgroup, for the workgroups that started
    with the launch (the first resident round: those that entered before any
    workgroup had finished) and for the rest; when the first round's nodes
    were staged; and, at
    `bins` instants over the launch, how many workgroups are in each phase."""
    import numpy as np

    m = np.asarray(marks, dtype=np.int64)
    t = (m[:, :4] - m[:, 0].min()).astype(np.float64) / clock_hz * 1e6   # us
    span = float(t[:, 3].max())
    first = t[:, 0] < t[:, 3].min()
    out = {"workgroups": int(m.shape[0]), "span_us": span, "first_round": int(first.sum()),
           "compute_units": int(np.unique(m[:, 4]).size)}
    for key, sel in (("first", first), ("later", ~first)):
        if sel.any():
            d = t[sel]
            out[key] = {"load_stage_us": float(np.median(d[:, 1] - d[:, 0])),
                        "pairs_us": float(np.median(d[:, 2] - d[:, 1])),
                        "store_us": float(np.median(d[:, 3] - d[:, 2]))}
    out["first_round_staged_us"] = [float(x) for x in np.percentile(t[first, 1], [10, 50, 90])]
    # after the last workgroup's nodes are staged only pairs and stores remain
    out["drain_us"] = span - float(t[:, 1].max())
    out["later_starts_us"] = ([float(x) for x in np.percentile(t[~first, 0], [0, 50, 100])]
                              if (~first).any() else [])
    rows = []
    for x in np.linspace(0.0, span, bins + 1):
        rows.append((float(x), int(((t[:, 0] <= x) & (t[:, 1] > x)).sum()),
                     int(((t[:, 1] <= x) & (t[:, 2] > x)).sum()),
                     int(((t[:, 2] <= x) & (t[:, 3] > x)).sum())))
    out["occupancy"] = rows
    return out


def timeline_runs(name: str, whole: bool = False, runs: int = 5, rotate_bytes: float = 512e6):
    """Phase summaries (timeline_phases) of `runs` launches of the library's
    kernel with marks on a named workload, after buffers rotated over more
    than the Infinity Cache and a pre-roll of library launches, as the
    benchmark times them.  Returns (workload, summaries sorted by span)."""
    import math
    import time

    import numpy as np
    import torch

    from entropy_stable_dg_amd import esdg, inputs

    dev = torch.device("cuda:0")
    wl = inputs.make(name)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    footprint = 2 * wl.q.nbytes + wl.phi.nbytes + wl.geom.nbytes
    nsets = max(2, math.ceil(rotate_bytes / footprint))
    sets = [(t(wl.q), t(wl.phi), t(wl.geom), t(wl.D), t(wl.nbr)) for _ in range(nsets)]
    outs = [torch.empty_like(s[0]) for s in sets]

    def lib_launch(i):
        q, phi, geom, D, nbr = sets[i % nsets]
        if whole:
            esdg.rhs(q, phi, geom, D, nbr, out=outs[i % nsets])
        else:
            esdg.volume_rhs(q, phi, geom, D, out=outs[i % nsets])

    i, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < 0.25:
        lib_launch(i)
        i += 1
    torch.cuda.synchronize()
    clock = esdg_probe_wall_clock_khz() * 1e3
    phases = []
    for r in range(runs):
        lib_launch(i)          # the launch before, as in a stream of launches
        q, phi, geom, D, nbr = sets[(i + 1) % nsets]
        _, marks = timeline(q, phi, geom, D, nbr if whole else None, rhs=outs[(i + 1) % nsets])
        torch.cuda.synchronize()
        phases.append(timeline_phases(marks.cpu().numpy(), clock))
        i += 2
    del sets, outs
    torch.cuda.empty_cache()
    return wl, sorted(phases, key=lambda ph: ph["span_us"])


def timeline_report(name: str, whole: bool = False, runs: int = 5) -> str:
    """Markdown summary of timeline_runs(): the launch with the median span
    is tabulated."""
    import numpy as np

    wl, phases = timeline_runs(name, whole, runs)
    order = list(range(runs))
    ph = phases[runs // 2]
    dt = "fp64" if wl.q.dtype == np.float64 else "fp32"
    lines = [f"Workload `{name}` ({'whole right-hand side' if whole else 'volume term'}, {dt}, "
             f"N={wl.N}, {wl.nelem} elements): {ph['workgroups']} workgroups on "
             f"{ph['compute_units']} compute units, {ph['first_round']} in the first resident round.",
             "",
             f"Kernel span (first entry to last store issued) over {runs} launches: "
             + ", ".join(f"{phases[k]['span_us']:.2f}" for k in order) + " us; the median one below.",
             "",
             "| workgroups | load + stage (A) | line pairs (B) | partials + store (C, D) |",
             "|---|---|---|---|"]
    for key, lab in (("first", "first round"), ("later", "later")):
        if key in ph:
            d = ph[key]
            lines.append(f"| {lab} | {d['load_stage_us']:.2f} | {d['pairs_us']:.2f} | {d['store_us']:.2f} |")
    p10, p50, p90 = ph["first_round_staged_us"]
    lines += ["", f"Medians in us.  First-round nodes staged at {p10:.2f} / {p50:.2f} / {p90:.2f} us "
              "(10th / 50th / 90th percentile of its workgroups)"
              + (f"; later workgroups start from {ph['later_starts_us'][0]:.2f} us, half by "
                 f"{ph['later_starts_us'][1]:.2f} us, the last at {ph['later_starts_us'][2]:.2f} us"
                 if ph["later_starts_us"] else "")
              + f".  After the last workgroup's nodes are staged, {ph['drain_us']:.2f} us of "
                "pairs and stores remain.",
              "", "Workgroups in each phase over the launch:", "",
              "| t (us) | loading + staging | line pairs | partials + store |", "|---|---|---|---|"]
    for x, a, b, c in ph["occupancy"]:
        lines.append(f"| {x:.1f} | {a} | {b} | {c} |")
    return "\n".join(lines)


if __name__ == "__main__":
    import sys

    args = sys.argv[1:]
    if len(args) >= 2 and args[0] == "timeline":
        print(timeline_report(args[1], whole="--whole" in args), flush=True)
    else:
        print("usage: python -m entropy_stable_dg_amd.probe timeline WORKLOAD [--whole]")
        sys.exit(2)
