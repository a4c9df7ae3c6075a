"""Binding of libesdg_probe.so (HBM streaming probes, measurement only), with
the C functions of include/esdg_probe.h under the same names."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(HERE, "libesdg_probe.so")
EXPORTS = ("esdg_probe_stream81_f64", "esdg_probe_stream81_wide_f64", "esdg_probe_node_log_f64",
           "esdg_probe_node_log_f32", "esdg_probe_copy_f64")

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
    for name in EXPORTS:
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
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
