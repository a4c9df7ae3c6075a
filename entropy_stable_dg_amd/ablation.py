"""Binding of libesdg_ablation.so (the optimisation-ladder variants of the
volume term, measurement only), with the C functions of
include/esdg_ablation.h under the same names.  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

from .esdg import ESDG_OK, EsdgError, esdg_status_string

HERE = os.path.dirname(os.path.abspath(__file__))
ABLATION_LIB_PATH = os.path.join(HERE, "libesdg_ablation.so")
EXPORTS = ("esdg_ablation_volume_rhs_f64", "esdg_ablation_two_lane_volume_rhs_f64",
           "esdg_ablation_name")
TWO_LANE_ORDERS = (5, 7)

ESDG_ABL_BASELINE = 0
ESDG_ABL_HOIST = 1
ESDG_ABL_LOGMEAN = 2
ESDG_ABL_CONTRA = 3
ESDG_ABL_SYM_UPPER = 4
ESDG_ABL_SYM_INDEXED = 5
ESDG_ABL_SYM_WEIGHTED = 6
ESDG_ABL_FUSED = 7
ESDG_ABL_COUNT = 8
ESDG_ABL_FUSE_FLAG = 0x100
ESDG_ERR_VARIANT = -6
ORDERS = (3, 4, 7)

_lib = None


def load(path: str = ABLATION_LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None and path == ABLATION_LIB_PATH:
        return _lib
    try:  # share the HIP runtime torch ships
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m entropy_stable_dg_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.esdg_ablation_volume_rhs_f64.restype = ci
    lib.esdg_ablation_volume_rhs_f64.argtypes = [ci, vp, vp, vp, vp, ci, i64, vp, vp]
    lib.esdg_ablation_two_lane_volume_rhs_f64.restype = ci
    lib.esdg_ablation_two_lane_volume_rhs_f64.argtypes = [vp, vp, vp, vp, ci, i64, vp, vp]
    lib.esdg_ablation_name.restype = ctypes.c_char_p
    lib.esdg_ablation_name.argtypes = [ci]
    if path == ABLATION_LIB_PATH:
        _lib = lib
    return lib


def esdg_ablation_volume_rhs_f64(variant: int, q: int, phi: int, geom: int, D: int, N: int,
                                 nelem: int, rhs: int, stream: int = 0) -> int:
    return load().esdg_ablation_volume_rhs_f64(variant, q, phi, geom, D, N, nelem, rhs, stream)


def esdg_ablation_two_lane_volume_rhs_f64(q: int, phi: int, geom: int, D: int, N: int, nelem: int,
                                          rhs: int, stream: int = 0) -> int:
    return load().esdg_ablation_two_lane_volume_rhs_f64(q, phi, geom, D, N, nelem, rhs, stream)


def esdg_ablation_name(variant: int) -> str:
    return load().esdg_ablation_name(variant).decode()


def volume_rhs(variant, q, phi, geom, D, out=None, stream=None):
    """The volume term by ladder variant `variant` on float64 GPU tensors
    (shapes as esdg.volume_rhs; N must be 3, 4 or 7)."""
    import torch

    for name, t in (("q", q), ("phi", phi), ("geom", geom), ("D", D)):
        if t.dtype != torch.float64:
            raise TypeError(f"{name} must be float64")
        if not t.is_cuda or t.device != q.device or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor on {q.device}")
    N = D.shape[0] - 1
    Np = (N + 1) ** 3
    nelem = q.shape[1]
    if (tuple(q.shape) != (5, nelem, Np) or tuple(phi.shape) != (nelem, Np)
            or tuple(geom.shape) != (10, nelem, Np) or tuple(D.shape) != (N + 1, N + 1)):
        raise ValueError("shapes must be q [5][nelem][Np], phi [nelem][Np], geom [10][nelem][Np], D [N+1][N+1]")
    if out is None:
        out = torch.empty_like(q)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        st = esdg_ablation_volume_rhs_f64(variant, q.data_ptr(), phi.data_ptr(), geom.data_ptr(),
                                          D.data_ptr(), N, nelem, out.data_ptr(), handle)
    if st != ESDG_OK:
        msg = "unknown ablation variant" if st == ESDG_ERR_VARIANT else esdg_status_string(st)
        raise EsdgError(st, msg)
    return out


def two_lane_volume_rhs(q, phi, geom, D, out=None, stream=None):
    """The production volume kernel with two lanes per grid line (N = 5, 7),
    on float64 GPU tensors shaped as for esdg.volume_rhs."""
    import torch

    N = D.shape[0] - 1
    if out is None:
        out = torch.empty_like(q)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    for name, t in (("q", q), ("phi", phi), ("geom", geom), ("D", D), ("out", out)):
        if t.dtype != torch.float64 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float64 GPU tensor")
    with torch.cuda.device(q.device):
        st = esdg_ablation_two_lane_volume_rhs_f64(q.data_ptr(), phi.data_ptr(), geom.data_ptr(),
                                                   D.data_ptr(), N, q.shape[1], out.data_ptr(),
                                                   handle)
    if st != ESDG_OK:
        raise EsdgError(st, esdg_status_string(st))
    return out
