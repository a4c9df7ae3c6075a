#!/usr/bin/env python3
"""Throughput of the ESDG flux-differencing volume term on one MI355X.

A step is one evaluation of the whole volume term (one kernel launch of
libesdg) over one batch of synthetic input: the rising-bubble-shaped workload
(16^3 affine hexes, N=4, 512,000 DOF) in fp64.  Inputs are resident in HBM
before the timed region; consecutive steps rotate over enough distinct buffer
sets (> 512 MB in total) that no step finds its inputs in the 256 MB
Infinity Cache left behind by the previous one.

Prints ONE JSON line on stdout; progress goes to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HEADLINE = "bubble"
METRIC = "volume-RHS DOF-updates/s and FP64 GFLOP/s (% of FP64 vector peak), N=4, 1 GPU"
SOURCES = ("entropy_stable_dg_amd/csrc/volume_kernel.hpp", "entropy_stable_dg_amd/csrc/esdg_api.hip",
           "entropy_stable_dg_amd/csrc/launch_table.hpp")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code (comments and blank lines removed, so
    editing a comment does not orphan the counters taken on the same code)."""
    import re

    h = hashlib.sha256()
    for rel in SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(code.encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, dtype: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    base = workload.replace("_f32", "")
    rec = data.get(f"{base}_{dtype}")
    if not rec or rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def measured_counter(workload: str, dtype: str, field: str):
    """A per-launch figure from the committed SQ counter summaries
    (profiles/sq_counters.json), if taken on the current kernel code."""
    path = os.path.join(ROOT, "profiles", "sq_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    rec = data.get(f"{workload.replace('_f32', '')}_{dtype}")
    if not rec or rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get(field)


def counted_fp64_flops(workload: str, dtype: str):
    """Counted FP64 FLOPs per launch (ADD + MUL + TRANS + 2 FMA, x 64 lanes:
    SQ_INSTS_VALU_FLOPS_FP64 plus SQ_INSTS_VALU_FLOPS_FP64_TRANS) from the
    committed counter summaries, if taken on the current kernel code."""
    fl = measured_counter(workload, dtype, "fp64_flops_per_launch")
    if not fl:
        return None
    return fl + (measured_counter(workload, dtype, "fp64_trans_flops_per_launch") or 0.0)


PREROLL_S = 0.25


def preroll(run, sync, seconds: float = PREROLL_S) -> int:
    """Untimed passes of `run()` until `seconds` of wall time have passed,
    synchronising after each, so that the timed pass starts on a device that
    has been busy (clocks up, caches and TLBs warm) however long the host
    spent before it.  Returns the passes run."""
    n, t0 = 0, time.perf_counter()
    while True:
        run()
        sync()
        n += 1
        if time.perf_counter() - t0 >= seconds:
            return n


def time_workload(name: str, steps: int, warmup: int, rotate_bytes: float, full: bool = False,
                  graph: bool = False, two_lane: bool = False):
    """Returns (seconds per step rotating cold buffers, seconds per step hot, info).
    With `full`, the whole right-hand side (volume + surface, esdg_rhs_*).
    With `graph`, the steps are captured once in a HIP graph (through torch's
    graph API) and the graph is replayed: the same launches without the
    per-launch host overhead.  Before each timed pass: `warmup` launches and
    a pre-roll of at least PREROLL_S seconds (preroll()).  With `two_lane`,
    the volume term by the two-lanes-per-line variant of the production kernel
    (libesdg_ablation, fp64, N = 5 and 7), for comparison."""
    import torch

    from entropy_stable_dg_amd import esdg, inputs, perfmodel

    wl = inputs.make(name)
    dtype = "f32" if wl.q.dtype.name == "float32" else "f64"
    dev = torch.device("cuda:0")
    footprint = sum(a.nbytes for a in (wl.q, wl.phi, wl.geom)) + wl.q.nbytes
    nsets = max(2, math.ceil(rotate_bytes / footprint))
    log(f"{name}{' (whole rhs)' if full else ''}: N={wl.N} nelem={wl.nelem} dof={wl.dof} "
        f"dtype={dtype} footprint={footprint / 1e6:.1f} MB x {nsets} buffer sets")
    host = [torch.from_numpy(a) for a in (wl.q, wl.phi, wl.geom, wl.D, wl.nbr)]
    sets = []
    for _ in range(nsets):
        q, phi, geom, D, nbr = (t.to(dev) for t in host)
        rhs = torch.empty_like(q)
        sets.append((q, phi, geom, D, nbr, rhs))
    if full:
        fn = esdg.esdg_rhs_f64 if dtype == "f64" else esdg.esdg_rhs_f32
    elif two_lane:
        from entropy_stable_dg_amd import ablation

        if dtype != "f64" or wl.N not in ablation.TWO_LANE_ORDERS:
            raise ValueError("the two-lane variant is fp64 at N = 5, 7")
        fn = ablation.esdg_ablation_two_lane_volume_rhs_f64
    else:
        fn = esdg.esdg_volume_rhs_f64 if dtype == "f64" else esdg.esdg_volume_rhs_f32
    stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream
    ptrs = [(q.data_ptr(), phi.data_ptr(), geom.data_ptr(), D.data_ptr(), nbr.data_ptr(),
             rhs.data_ptr()) for q, phi, geom, D, nbr, rhs in sets]
    N, nelem = wl.N, wl.nelem

    def run(k: int, rotate: bool) -> None:
        for i in range(k):
            p = ptrs[i % nsets] if rotate else ptrs[0]
            if full:
                st = fn(p[0], p[1], p[2], p[3], p[4], None, N, nelem, p[5], handle)
            else:
                st = fn(p[0], p[1], p[2], p[3], N, nelem, p[5], handle)
            if st != 0:
                raise RuntimeError(esdg.esdg_status_string(st))

    results, prerolls = {}, {}
    for rotate in (True, False):
        run(warmup, rotate)
        torch.cuda.synchronize()
        prerolls[rotate] = preroll(lambda: run(nsets, rotate), torch.cuda.synchronize)
        if graph:
            per_graph = min(steps, 100)
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream(dev)
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                handle = side.cuda_stream
                run(2, rotate)                      # warm-up on the capture stream
            stream.wait_stream(side)
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=side):
                handle = side.cuda_stream
                run(per_graph, rotate)
            handle = stream.cuda_stream
            replays = max(1, steps // per_graph)
            g.replay()
            torch.cuda.synchronize()
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            start.record(stream)
            for _ in range(replays):
                g.replay()
            end.record(stream)
            torch.cuda.synchronize()
            results[rotate] = start.elapsed_time(end) * 1e-3 / (replays * per_graph)
            del g
        else:
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            start.record(stream)
            run(steps, rotate)
            end.record(stream)
            torch.cuda.synchronize()
            results[rotate] = start.elapsed_time(end) * 1e-3 / steps
        log(f"{name}{' (graph replay)' if graph else ''}: {'rotating' if rotate else 'hot'} {results[rotate] * 1e6:.2f} us/step")
    info = dict(N=N, nelem=nelem, dof=wl.dof, dtype=dtype, description=wl.description,
                seed=wl.seed, buffer_sets=nsets,
                preroll={"seconds": PREROLL_S, "passes_rotating": prerolls[True],
                         "passes_hot": prerolls[False], "launches_per_pass": nsets},
                bytes=perfmodel.algorithmic_bytes(N, nelem, dtype),
                flops=perfmodel.flops_per_element(N) * nelem)
    if full:
        info["bytes"] = perfmodel.algorithmic_bytes_rhs(N, nelem, dtype)
        info["bytes_with_face_partners"] = info["bytes"] + perfmodel.face_partner_bytes(N, wl.nbr, dtype)
        info["flops"] += perfmodel.surface_flops(N, wl.nbr)
    del sets
    torch.cuda.empty_cache()
    return results[True], results[False], info, wl


# Time steps near the acoustic limit (0.5 x the smallest LGL node spacing over
# the sound speed): bubble 62.5 m elements, N=4, smallest gap 10.8 m;
# baroclinic 3.75 km tall elements, smallest vertical gap 650 m.
STEP_DT = {"bubble": 7.0e-3, "bubble_f32": 7.0e-3, "baroclinic": 0.5, "baroclinic_f32": 0.5,
           "tiny": 1.0e-4, "high_order": 2.0e-3}


def time_stages(name: str, steps: int, warmup: int, rotate_bytes: float, pert: bool = False):
    """Seconds per fused Runge-Kutta stage (whole right-hand side + the
    low-storage update in one kernel, esdg_lsrk_steps_*), rotating over
    enough independent states (> rotate_bytes) that no stage finds its inputs
    in the cache.  Each timed call is two steps (ten stages, no final copy).
    With `pert`, the state is carried as perturbation variables."""
    import torch

    from entropy_stable_dg_amd import esdg, inputs

    if pert:
        wl, qp, ref = inputs.make_perturbed(name)
    else:
        wl, qp, ref = inputs.make(name), None, None
    dtype = "f32" if wl.q.dtype.name == "float32" else "f64"
    dev = torch.device("cuda:0")
    footprint = (3 * wl.q.nbytes + wl.phi.nbytes + wl.geom.nbytes
                 + (ref.nbytes if ref is not None else 0))
    nsets = max(2, math.ceil(rotate_bytes / footprint))
    log(f"{name} stages{' (perturbation variables)' if pert else ''}: footprint "
        f"{footprint / 1e6:.1f} MB x {nsets} sets")
    sets = []
    for _ in range(nsets):
        q = torch.from_numpy(qp if pert else wl.q).to(dev)
        sets.append(dict(q=q, q_tmp=torch.empty_like(q), dq=torch.empty_like(q),
                         phi=torch.from_numpy(wl.phi).to(dev), geom=torch.from_numpy(wl.geom).to(dev),
                         D=torch.from_numpy(wl.D).to(dev), nbr=torch.from_numpy(wl.nbr).to(dev),
                         ref=torch.from_numpy(ref).to(dev) if pert else None))
    stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream
    fn = esdg.esdg_lsrk_steps_f64 if dtype == "f64" else esdg.esdg_lsrk_steps_f32
    dt = STEP_DT[name]

    def run(k: int) -> None:
        for i in range(k):
            t = sets[i % nsets]
            st = fn(t["q"].data_ptr(), t["q_tmp"].data_ptr(), t["dq"].data_ptr(),
                    t["ref"].data_ptr() if pert else None, t["phi"].data_ptr(),
                    t["geom"].data_ptr(), t["D"].data_ptr(), t["nbr"].data_ptr(), None, dt, 2,
                    wl.N, wl.nelem, handle)
            if st != 0:
                raise RuntimeError(esdg.esdg_status_string(st))

    run(max(1, warmup // 10))
    torch.cuda.synchronize()
    passes = preroll(lambda: run(nsets), torch.cuda.synchronize)
    calls = max(1, steps // 10)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    run(calls)
    t1.record(stream)
    torch.cuda.synchronize()
    sec = t0.elapsed_time(t1) * 1e-3 / (10 * calls)
    finite = all(bool(torch.isfinite(t["q"]).all()) for t in sets)
    log(f"{name} stage{' (perturbation variables)' if pert else ''}: {sec * 1e6:.2f} us/stage")
    del sets
    torch.cuda.empty_cache()
    from entropy_stable_dg_amd import perfmodel

    nbytes = perfmodel.algorithmic_bytes_stage(wl.N, wl.nelem, dtype)
    if pert:
        nbytes += 2 * wl.dof * (8 if dtype == "f64" else 4)
    return sec, {"N": wl.N, "nelem": wl.nelem, "dof": wl.dof, "dtype": dtype, "dt": dt,
                 "stages_timed": 10 * calls, "buffer_sets": nsets, "preroll_passes": passes,
                 "state_finite_after": finite, "bytes_per_stage": nbytes,
                 "hbm_gbs_algorithmic": nbytes / sec / 1e9}


def conservation_drift(name: str, nsteps: int, pert: bool = False) -> dict:
    """Relative change of the sums of the integrals of rho, E and the entropy
    over nsteps Runge-Kutta steps (esdg_integrals_* before and after
    esdg_lsrk_steps_*): the global diagnostics of the page's baroclinic test."""
    import numpy as np
    import torch

    from entropy_stable_dg_amd import esdg, inputs

    if pert:
        wl, qp, ref = inputs.make_perturbed(name)
    else:
        wl, qp, ref = inputs.make(name), None, None
    dev = torch.device("cuda:0")
    q = torch.from_numpy(qp if pert else wl.q).to(dev)
    phi, geom, D, nbr = (torch.from_numpy(a).to(dev) for a in (wl.phi, wl.geom, wl.D, wl.nbr))
    tref = torch.from_numpy(ref).to(dev) if pert else None
    _, w = inputs.lgl(wl.N)
    tw = torch.from_numpy(w.astype(wl.q.dtype)).to(dev)
    before = esdg.integrals(q, phi, geom, tw, ref=tref).cpu().numpy()
    dt = STEP_DT[name]
    t0 = time.perf_counter()
    esdg.lsrk_steps(q, phi, geom, D, nbr, dt, nsteps, ref=tref)
    after = esdg.integrals(q, phi, geom, tw, ref=tref).cpu().numpy()
    wall = time.perf_counter() - t0
    rel = (after - before) / np.abs(before)
    log(f"conservation {name}{' (perturbation variables)' if pert else ''}: {nsteps} steps of "
        f"{dt} s: relative change mass {rel[0]:.2e} energy {rel[1]:.2e} entropy {rel[2]:.2e}")
    return {"steps": nsteps, "dt": dt, "dtype": "f32" if wl.q.dtype.name == "float32" else "f64",
            "perturbation_variables": pert, "relative_change_mass": float(rel[0]),
            "relative_change_energy": float(rel[1]), "relative_change_entropy": float(rel[2]),
            "initial": before.tolist(), "wall_s": wall}


def profile_pass(steps: int, workload: str = HEADLINE) -> dict:
    """Short run for hardware-counter collection under rocprofv3: one plain
    copy kernel of known size (esdg_probe_copy_f64: 512 MiB read, 512 MiB
    written, the calibration of FETCH_SIZE / WRITE_SIZE), then `steps`
    launches of the headline kernel."""
    import torch

    from entropy_stable_dg_amd import probe

    dev = torch.device("cuda:0")
    n = (512 << 20) // 8
    src = torch.ones(n, dtype=torch.float64, device=dev)
    dst = torch.empty_like(src)
    # plain copy kernel (libesdg_probe): reads n*8 B, writes n*8 B
    if probe.esdg_probe_copy_f64(src.data_ptr(), dst.data_ptr(), n,
                                 torch.cuda.current_stream(dev).cuda_stream) != 0:
        raise RuntimeError("copy probe failed")
    torch.cuda.synchronize()
    del src, dst
    name, _, mode = workload.partition(":")
    if mode in ("stage", "stage_pert"):
        sec, inf = time_stages(name, 10 * steps, 10, 512e6, pert=(mode == "stage_pert"))
        return {"profile_pass": True, "workload": workload, "copy_bytes_each_way": n * 8,
                "us_per_stage": sec * 1e6, "bytes_per_launch": inf["bytes_per_stage"],
                "kernel_source_hash": kernel_source_hash()}
    cold, hot, info, _ = time_workload(name, steps, 2, 512e6, full=(mode == "rhs"),
                                       two_lane=(mode == "two_lane"))
    return {"profile_pass": True, "workload": workload, "copy_bytes_each_way": n * 8,
            "us_per_step": cold * 1e6, "bytes_per_launch": info["bytes"],
            "flops_per_launch": info["flops"], "kernel_source_hash": kernel_source_hash()}


def time_ablation(steps: int, warmup: int) -> dict:
    """The optimisation ladder (libesdg_ablation, thread-per-node kernels, one
    variant per cumulative step) and the production kernel, timed on the
    pages' ladder configuration: N = 4, refinement level 6 (262,144
    elements, 32,768,000 DOF), fp64, the bubble workload tiled 64 times."""
    import torch

    from entropy_stable_dg_amd import ablation, esdg, inputs

    wl = inputs.make(HEADLINE)
    dev = torch.device("cuda:0")
    reps = 64
    q, phi, geom, D = (torch.from_numpy(a).to(dev) for a in (wl.q, wl.phi, wl.geom, wl.D))
    q, phi, geom = q.repeat(1, reps, 1), phi.repeat(reps, 1), geom.repeat(1, reps, 1)
    rhs = torch.empty_like(q)
    nelem, N = q.shape[1], wl.N
    handle = torch.cuda.current_stream(dev).cuda_stream
    args = (q.data_ptr(), phi.data_ptr(), geom.data_ptr(), D.data_ptr(), N, nelem, rhs.data_ptr(), handle)

    def timed(call) -> float:
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            call()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    def check(st):
        if st != 0:
            raise RuntimeError(f"ablation launch failed with status {st}")

    ladder = []
    for v in range(ablation.ESDG_ABL_COUNT):
        ms = timed(lambda: check(ablation.esdg_ablation_volume_rhs_f64(v, *args)))
        vf = v | ablation.ESDG_ABL_FUSE_FLAG
        msf = timed(lambda: check(ablation.esdg_ablation_volume_rhs_f64(vf, *args)))
        ladder.append({"variant": v, "name": ablation.esdg_ablation_name(v), "ms": ms,
                       "ms_fused": msf})
        log(f"ablation {v} ({ladder[-1]['name']}): {ms:.3f} ms; directions fused {msf:.3f} ms")
    prod = timed(lambda: check(esdg.esdg_volume_rhs_f64(*args)))
    log(f"ablation production kernel: {prod:.3f} ms")
    base = ladder[0]["ms"]
    for r in ladder:
        r["speedup_vs_baseline"] = base / r["ms"]
        r["speedup_fused_vs_baseline"] = base / r["ms_fused"]
    dof = nelem * wl.Np
    del q, phi, geom, rhs
    torch.cuda.empty_cache()
    return {"config": f"N={N}, {nelem} elements ({dof} DOF), fp64, bubble tiled {reps}x, hot buffers",
            "steps": steps, "ladder": ladder,
            "production": {"ms": prod, "speedup_vs_baseline": base / prod, "dof_per_s": dof / (prod * 1e-3)}}


def roofline_sweep(levels=(3, 4, 5, 6), orders=range(1, 9), dtypes=("f64", "f32"),
                   steps: int = 20) -> dict:
    """Throughput of the volume term and of the whole right-hand side at every
    order N and refinement level L (N_e = 2^(3L) elements, one base element as
    in the page's Fig. 3 and Fig. 5): the bubble-shaped state on a warped 8^3
    mesh (L = 3; periodic in x and y, slip walls in z) is built on the host
    once per order and tiled on the GPU to reach L = 4..6.  The volume term is
    element-local, so tiling leaves its work and traffic per element
    unchanged; for the whole right-hand side every tile keeps the base mesh's
    connectivity (offset to its own elements), so each tile is a closed mesh
    of its own.  Below 512 MB of footprint, launches rotate over enough copies
    that inputs are not cache-resident."""
    import torch

    from entropy_stable_dg_amd import esdg, inputs, perfmodel

    dev = torch.device("cuda:0")
    handle = torch.cuda.current_stream(dev).cuda_stream
    points = []
    for dtype in dtypes:
        fn = esdg.esdg_volume_rhs_f64 if dtype == "f64" else esdg.esdg_volume_rhs_f32
        fn_rhs = esdg.esdg_rhs_f64 if dtype == "f64" else esdg.esdg_rhs_f32
        for N in orders:
            wl = inputs.build_workload(f"sweep_N{N}", (8, 8, 8), (0, 0, 0), (1000, 1000, 1000), N,
                                       "bubble", seed=600 + N, warp_frac=0.05, dtype=dtype,
                                       periodic=(True, True, False))
            base = [torch.from_numpy(a).to(dev) for a in (wl.q, wl.phi, wl.geom, wl.D)]
            base_nbr = torch.from_numpy(wl.nbr).to(dev)
            for L in levels:
                reps = 8 ** (L - 3)
                q = base[0].repeat(1, reps, 1)
                phi = base[1].repeat(reps, 1)
                geom = base[2].repeat(1, reps, 1)
                D = base[3]
                nelem = q.shape[1]
                footprint = (q.numel() * 2 + phi.numel() + geom.numel()) * q.element_size()
                nsets = max(1, math.ceil(512e6 / footprint)) if footprint < 512e6 else 1
                sets = [(q, phi, geom, torch.empty_like(q))]
                for _ in range(nsets - 1):
                    sets.append((q.clone(), phi.clone(), geom.clone(), torch.empty_like(q)))
                ptrs = [(a.data_ptr(), b.data_ptr(), c.data_ptr(), r.data_ptr()) for a, b, c, r in sets]

                # each tile is a closed mesh of its own: its face neighbours
                # are the base mesh's, offset by the tile's first element
                base_ne = base[0].shape[1]
                nbr = torch.cat([torch.where(base_nbr >= 0, base_nbr + t * base_ne, base_nbr)
                                 for t in range(reps)]).contiguous()
                assert nbr.dtype == torch.int32 and tuple(nbr.shape) == (nelem, 6)
                assert int(nbr.max()) < nelem

                def run(k: int, full: bool = False) -> None:
                    for i in range(k):
                        p = ptrs[i % nsets]
                        if full:
                            st = fn_rhs(p[0], p[1], p[2], D.data_ptr(), nbr.data_ptr(), None, N, nelem,
                                        p[3], handle)
                        else:
                            st = fn(p[0], p[1], p[2], D.data_ptr(), N, nelem, p[3], handle)
                        if st != 0:
                            raise RuntimeError("launch failed")

                def timed(full: bool) -> float:
                    run(3, full)
                    torch.cuda.synchronize()
                    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    t0.record()
                    run(steps, full)
                    t1.record()
                    torch.cuda.synchronize()
                    return t0.elapsed_time(t1) * 1e-3 / steps

                sec = timed(False)
                sec_rhs = timed(True)
                dof = nelem * (N + 1) ** 3
                flops = perfmodel.flops_per_element(N) * nelem
                nbytes = perfmodel.algorithmic_bytes(N, nelem, dtype)
                pt = {"dtype": dtype, "N": N, "L": L, "nelem": nelem, "dof": dof, "us": sec * 1e6,
                      "gdof_s": dof / sec / 1e9, "analytic_tflops": flops / sec / 1e12,
                      "hbm_gbs": nbytes / sec / 1e9,
                      "arithmetic_intensity": perfmodel.arithmetic_intensity(N, dtype)}
                if dtype == "f64":
                    pt["frac_fp64_vector_peak"] = pt["analytic_tflops"] / perfmodel.PEAK_FP64_VECTOR_TFLOPS
                pt["rhs_us"] = sec_rhs * 1e6
                pt["rhs_gdof_s"] = dof / sec_rhs / 1e9
                pt["rhs_hbm_gbs"] = perfmodel.algorithmic_bytes_rhs(N, nelem, dtype) / sec_rhs / 1e9
                points.append(pt)
                log(f"sweep {dtype} N={N} L={L}: {nelem} el., {pt['us']:.1f} us, {pt['gdof_s']:.2f} GDOF/s, "
                    f"{pt['analytic_tflops']:.2f} TF/s, {pt['hbm_gbs']:.0f} GB/s; whole rhs "
                    f"{pt['rhs_us']:.1f} us, {pt['rhs_gdof_s']:.2f} GDOF/s")
                del sets, q, phi, geom
                torch.cuda.empty_cache()
            del base
    return {"sweep": "volume term and whole right-hand side, every order and refinement level "
                     "(N_e = 2^(3L))",
            "steps": steps, "points": points}


def cpu_one_core(wl, seconds: float) -> dict:
    """The oracle's fp64 build on one host thread over a bounded leading slice
    of the workload's elements (element-local work, so DOF/s carries over)."""
    import oracle

    orc = oracle.fp64()
    ne = max(1, min(wl.nelem, 256))
    q, phi, geom = wl.q[:, :ne], wl.phi[:ne], wl.geom[:, :ne]
    reps, t0 = 0, time.perf_counter()
    while True:
        orc.volume_rhs(q, phi, geom, wl.D, wl.N, threads=1)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    value = ne * wl.Np * reps / dt
    log(f"cpu oracle 1 thread: {reps} x {ne} elements in {dt:.1f} s -> {value:.3e} DOF/s")
    return {"value": value, "unit": "DOF-updates/s", "cores": 1,
            "sample": f"{reps} evaluations of the first {ne} elements of {wl.name}"}


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo) and the logical CPUs
    the OS reports."""
    name = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{name} ({os.cpu_count()} logical CPUs reported)"


def cpu_baseline(wl, min_seconds: float, runs: int = 3):
    """The oracle's fp64 build (ordered pairs, OpenMP over elements, every
    host thread) on the whole workload: `runs` timed runs of at least
    `min_seconds` / `runs` each, the median reported."""
    import statistics

    import oracle

    orc = oracle.fp64()
    threads = orc.max_threads()
    orc.volume_rhs(wl.q, wl.phi, wl.geom, wl.D, wl.N)  # warm (library load, pages)
    rates, total = [], 0.0
    for _ in range(runs):
        reps, t0 = 0, time.perf_counter()
        while True:
            orc.volume_rhs(wl.q, wl.phi, wl.geom, wl.D, wl.N, threads=threads)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds / runs:
                break
        rates.append(wl.dof * reps / dt)
        total += dt
    value = statistics.median(rates)
    log(f"cpu oracle: {runs} runs, {total:.1f} s on {threads} threads -> median {value:.3e} DOF/s "
        f"(runs {', '.join(f'{r:.3e}' for r in rates)})")
    return {"value": value, "unit": "DOF-updates/s", "cores": threads, "kind": "oracle",
            "sample": f"median of {runs} timed runs of at least {min_seconds / runs:.1f} s, each "
                      f"repeated evaluations of the whole {wl.name} workload ({wl.dof} DOF each); "
                      f"the oracle's fp64 build, ordered pairs, OpenMP over elements",
            "runs": rates, "cpu": cpu_model()}


def roofline_of(achieved_gbs: float, gflops: float, stream_gbs: float, traffic):
    """The roofline object of the dominant kernel, measured against whichever
    roof this run comes closest to (HBM bytes, or fp64 vector FLOPs by the
    analytic count: the kernel issues no MFMA), and a sentence naming what
    binds, derived from the same figures: a roof binds when the kernel reaches
    at least 70 % of it (of the measured stream for HBM), otherwise neither
    does and the time goes to latency."""
    from entropy_stable_dg_amd import perfmodel

    hbm = achieved_gbs / perfmodel.PEAK_HBM_GBS
    alu = gflops / (perfmodel.PEAK_FP64_VECTOR_TFLOPS * 1e3)
    if hbm >= alu:
        roof = {"bound": "hbm", "achieved": achieved_gbs, "peak": perfmodel.PEAK_HBM_GBS,
                "unit": "GB/s", "frac": hbm, "traffic": traffic}
    else:
        roof = {"bound": "alu", "achieved": gflops / 1e3, "peak": perfmodel.PEAK_FP64_VECTOR_TFLOPS,
                "unit": "TFLOP/s", "frac": alu, "traffic": traffic}
    stream = achieved_gbs / stream_gbs
    if stream >= 0.7:
        what = "HBM binds"
    elif alu >= 0.7:
        what = "the fp64 vector units bind"
    else:
        what = "neither roof binds: latency (the load phase of each workgroup round) takes the rest"
    sentence = (f"{what}: {100 * hbm:.0f} % of nominal HBM ({100 * stream:.0f} % of the measured "
                f"8:1 stream), {100 * alu:.0f} % of the fp64 vector peak by the analytic count")
    return roof, sentence


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--rotate-mb", type=float, default=512.0,
                    help="total size of the rotating buffer sets (MB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--profile-pass", action="store_true",
                    help="short run for rocprofv3 counter passes (copy calibration + kernel)")
    ap.add_argument("--workload", default=HEADLINE,
                    help="workload of the profile pass (tiny, bubble, baroclinic, bubble_f32, "
                         "high_order; a ':rhs' suffix profiles the whole right-hand side, "
                         "':two_lane' the two-lanes-per-line variant, ':stage' the fused "
                         "Runge-Kutta stage, ':stage_pert' the same in perturbation variables)")
    ap.add_argument("--extra", default="bubble_f32,bubble:rhs,bubble_f32:rhs,baroclinic,"
                                       "baroclinic:rhs,high_order,high_order:two_lane",
                    help="comma-separated extra workloads to time (reported under 'extra'); "
                         "a ':rhs' suffix times the whole right-hand side (volume + surface), "
                         "':graph' replays the launches from a captured HIP graph")
    ap.add_argument("--stages", default="bubble,bubble_f32,bubble_f32:pert",
                    help="workloads whose fused Runge-Kutta stage (whole rhs + update) is timed "
                         "(reported under 'stage'); ':pert' for perturbation variables")
    ap.add_argument("--conservation-steps", type=int, default=500,
                    help="steps of the conservation-drift diagnostics (0: none)")
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip the optimisation-ladder timing (N=4, 262,144 elements)")
    ap.add_argument("--ablation-steps", type=int, default=10)
    ap.add_argument("--no-timeline", action="store_true",
                    help="skip the phase timeline of the headline kernel (libesdg_probe)")
    ap.add_argument("--sweep", action="store_true",
                    help="only the all-orders roofline sweep (N = 1..8, L = 3..6, fp64 and fp32); "
                         "prints its own JSON line")
    ap.add_argument("--all", action="store_true",
                    help="time every workload (tiny, baroclinic, bubble_f32, high_order) as extras")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the volume term is element-local: each GPU would run the same kernel on its "
              "own elements with no communication)", file=sys.stderr)
        return 2

    import torch

    from entropy_stable_dg_amd import esdg, perfmodel

    if not os.path.exists(esdg.LIB_PATH):
        from entropy_stable_dg_amd import build as hip_build
        hip_build.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    log(f"device: {torch.cuda.get_device_name(0)}; kernel source {kernel_source_hash()}")
    if args.profile_pass:
        print(json.dumps(profile_pass(args.steps, args.workload)), flush=True)
        return 0
    if args.sweep:
        from entropy_stable_dg_amd import probe
        out = roofline_sweep()
        out["hbm_stream81_gbs"] = max(probe.stream81_bandwidth(), probe.stream81_bandwidth(wide=True))
        out["kernel_source_hash"] = kernel_source_hash()
        print(json.dumps(out), flush=True)
        return 0

    t_cold, t_hot, info, wl = time_workload(HEADLINE, args.steps, args.warmup, args.rotate_mb * 1e6)
    value = info["dof"] / t_cold
    achieved_gbs = info["bytes"] / t_cold / 1e9
    gflops = info["flops"] / t_cold / 1e9
    traffic = measured_traffic(HEADLINE, info["dtype"])
    counted_flops = counted_fp64_flops(HEADLINE, info["dtype"])

    extra = {}
    names = [x for x in args.extra.split(",") if x]
    if args.all:
        names = ["tiny", "tiny:graph", "baroclinic", "bubble_f32", "high_order", "bubble:rhs",
                 "bubble_f32:rhs", "baroclinic:rhs", "high_order:rhs"]
    for key in names:
        name, _, mode = key.partition(":")
        full = mode == "rhs"
        c, h, inf, _ = time_workload(name, args.steps, args.warmup, args.rotate_mb * 1e6, full=full,
                                     graph=(mode == "graph"), two_lane=(mode == "two_lane"))
        extra[key] = {
            "dof_per_s": inf["dof"] / c, "us_per_step": c * 1e6, "hot_us_per_step": h * 1e6,
            "hbm_gbs_algorithmic": inf["bytes"] / c / 1e9, "gflops_analytic": inf["flops"] / c / 1e9,
            "traffic": measured_traffic(key.replace(":", "_"), inf["dtype"]),
            "gflops_counted_fp64": (lambda fl: fl / c / 1e9 if fl else None)(
                counted_fp64_flops(key.replace(":", "_"), inf["dtype"])),
            "dtype": inf["dtype"], "N": inf["N"], "nelem": inf["nelem"], "preroll": inf["preroll"],
            "hbm_frac": inf["bytes"] / c / 1e9 / perfmodel.PEAK_HBM_GBS,
            "frac_fp64_vector_peak": (inf["flops"] / c / 1e12 / perfmodel.PEAK_FP64_VECTOR_TFLOPS
                                      if inf["dtype"] == "f64" else None),
        }
        if inf["dtype"] == "f32":
            fl32 = measured_counter(key.replace(":", "_"), inf["dtype"], "fp32_flops_per_launch")
            extra[key]["frac_fp32_vector_peak"] = (inf["flops"] / c / 1e12
                                                   / perfmodel.PEAK_FP32_VECTOR_TFLOPS)
            extra[key]["gflops_counted_fp32"] = fl32 / c / 1e9 if fl32 else None
            extra[key]["frac_fp32_vector_peak_counted"] = (
                fl32 / c / 1e12 / perfmodel.PEAK_FP32_VECTOR_TFLOPS if fl32 else None)
        if mode == "graph":
            extra[key]["what"] = "the same launches captured once in a HIP graph and replayed"
        if mode == "two_lane":
            extra[key]["what"] = ("the production kernel with two lanes per grid line and a "
                                  "cross-lane exchange (libesdg_ablation), for comparison")
        if full:
            extra[key]["hbm_gbs_with_face_partners"] = inf["bytes_with_face_partners"] / c / 1e9
            extra[key]["what"] = "whole right-hand side: volume + entropy-conservative surface term"
        if (inf["dtype"] == "f32" and not full and inf["N"] == info["N"]
                and inf["nelem"] == info["nelem"]):
            extra[key]["speedup_over_fp64"] = (inf["dof"] / c) / value

    stage = {}
    for key in [x for x in args.stages.split(",") if x]:
        name, _, mode = key.partition(":")
        sec, inf = time_stages(name, args.steps, args.warmup, args.rotate_mb * 1e6, pert=(mode == "pert"))
        stage[key] = dict(inf, us_per_stage=sec * 1e6, dof_stage_updates_per_s=inf["dof"] / sec,
                          what="one fused launch: whole right-hand side (volume + surface) and the "
                               "low-storage Runge-Kutta update of the register and the state")
    if "bubble" in stage and "bubble_f32" in stage:
        stage["bubble_f32"]["speedup_over_fp64"] = (stage["bubble"]["us_per_stage"]
                                                    / stage["bubble_f32"]["us_per_stage"])

    conservation = {}
    if args.conservation_steps > 0:
        for key in ("bubble", "bubble_f32", "bubble_f32:pert", "baroclinic", "baroclinic_f32",
                    "baroclinic_f32:pert"):
            name, _, mode = key.partition(":")
            conservation[key] = conservation_drift(name, args.conservation_steps, pert=(mode == "pert"))

    ablation = None
    if not args.no_ablation:
        ablation = time_ablation(args.ablation_steps, 2)

    from entropy_stable_dg_amd import probe
    stream_narrow = probe.stream81_bandwidth()
    stream_wide = probe.stream81_bandwidth(wide=True)
    stream_gbs = max(stream_narrow, stream_wide)
    log(f"HBM stream probe (8 reads : 1 write, fp64): {stream_narrow:.0f} GB/s with 8-byte lanes, "
        f"{stream_wide:.0f} GB/s with 32-byte lanes")

    roofline, binding = roofline_of(achieved_gbs, gflops, stream_gbs, traffic)

    # lower bounds from this run's stream bandwidth and the committed VALU
    # counts (same kernel code): near their sum when load and compute serialise
    def floors_of(key, dtype, nbytes, us):
        v = measured_counter(key.replace(":", "_"), dtype, "valu_wave_instructions_per_launch")
        return perfmodel.phase_floors(nbytes, v, stream_gbs, us) if v else None

    phase_floors = floors_of(HEADLINE, info["dtype"], info["bytes"], t_cold * 1e6)
    if phase_floors and binding.startswith("neither"):
        binding += (f"; the launch takes {phase_floors['measured_over_sum']:.2f} of the sum of its "
                    f"HBM floor ({phase_floors['hbm_us']:.1f} us at the measured stream) and VALU "
                    f"issue floor ({phase_floors['valu_us']:.1f} us): its load and compute phases "
                    + ("barely overlap" if phase_floors["measured_over_sum"] >= 0.9
                       else "overlap in part"))
    for key, e in extra.items():
        if ":" not in key or key.endswith(":rhs"):
            nbytes = e["hbm_gbs_algorithmic"] * e["us_per_step"] * 1e3
            e["phase_floors"] = floors_of(key, e["dtype"], nbytes, e["us_per_step"])

    # where the headline launch's time goes: phase marks of the same kernel
    # (libesdg_probe), the launch with the median span of five
    timeline = None
    if not args.no_timeline:
        _, runs = probe.timeline_runs(HEADLINE, runs=5, rotate_bytes=args.rotate_mb * 1e6)
        ph = runs[len(runs) // 2]
        timeline = {k: ph[k] for k in ("workgroups", "compute_units", "first_round", "span_us",
                                       "first", "later", "first_round_staged_us",
                                       "later_starts_us", "drain_us") if k in ph}
        timeline["spans_us"] = [r["span_us"] for r in runs]
        log(f"phase timeline: span {ph['span_us']:.2f} us; first round loads {ph['first']['load_stage_us']:.2f} us "
            f"(median), pairs {ph['first']['pairs_us']:.2f} us; drain {ph['drain_us']:.2f} us")
        if binding.startswith("neither"):
            binding += (f"; phase timeline of the same kernel: the first round's {ph['first_round']} "
                        f"workgroups load and stage for a median {ph['first']['load_stage_us']:.1f} us "
                        f"before their pairs, and {ph['drain_us']:.1f} us of pairs and stores remain "
                        f"after the last workgroup's loads")

    cpu = None
    cpu1 = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_seconds)
        cpu1 = cpu_one_core(wl, max(1.0, args.cpu_seconds / 3))

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "DOF-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_cold * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": info["dtype"],
        "data": "synthetic",
        "config": {
            "workload": "rising-bubble-shaped 16x16x16 affine hexes on [0,1000]^3 m, N=4, "
                        "512000 DOF, fp64",
            "N": info["N"], "nelem": info["nelem"], "dof": info["dof"], "seed": info["seed"],
            "buffer_sets": info["buffer_sets"], "parallelism": "single GPU",
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "gflops_analytic_fp64": gflops,
        "frac_fp64_vector_peak": gflops / (perfmodel.PEAK_FP64_VECTOR_TFLOPS * 1e3),
        # hardware-counted figures: per-launch counter values (profiles/, same kernel code)
        # over this run's measured launch time
        "gflops_counted_fp64": counted_flops / t_cold / 1e9 if counted_flops else None,
        "frac_fp64_vector_peak_counted": (counted_flops / t_cold / 1e12 / perfmodel.PEAK_FP64_VECTOR_TFLOPS
                                          if counted_flops else None),
        "hbm_gbs_counted": traffic / t_cold / 1e9 if traffic else None,
        "binding_roof": binding,
        "phase_floors": phase_floors,
        "phase_timeline": timeline,
        "arithmetic_intensity": perfmodel.arithmetic_intensity(info["N"], info["dtype"]),
        "hot_ms_per_step": t_hot * 1e3,
        "hot_dof_per_s": info["dof"] / t_hot,
        # untimed launches run before each timed pass (warm device whatever the host did before)
        "preroll": info["preroll"],
        "kernel_source_hash": kernel_source_hash(),
        "hbm_stream81_gbs": stream_gbs,
        "hbm_stream81_gbs_by_lane_width": {"8B": stream_narrow, "32B": stream_wide},
        "frac_of_measured_stream": achieved_gbs / stream_gbs,
        "cpu_oracle_one_core": cpu1,
        "extra": extra,
        "stage": stage,
        "conservation": conservation,
        "ablation": ablation,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
