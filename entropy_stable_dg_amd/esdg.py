"""Python binding of libesdg (ctypes).  Argument marshalling only: every step of
the volume term runs in the HIP kernels of libesdg.so; there is no CPU path.

Two levels:
  * esdg_volume_rhs_f64 / esdg_volume_rhs_f32 / esdg_rhs_f64 / esdg_rhs_f32 /
    esdg_status_string / esdg_min_order / esdg_max_order -- the C functions of
    include/esdg.h under the same names (device pointers as Python ints, a
    status code returned);
  * volume_rhs(q, phi, geom, D, out=None, stream=None) and
    rhs(q, phi, geom, D, nbr, omega=None, out=None, stream=None) -- the same calls on
    torch tensors resident on the GPU, raising EsdgError on a bad status.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libesdg.so")

ESDG_OK = 0
ESDG_ERR_NULL = -1
ESDG_ERR_ORDER = -2
ESDG_ERR_NELEM = -3
ESDG_ERR_LAUNCH = -4
ESDG_ERR_ALIAS = -5

# every symbol include/esdg.h declares
EXPORTS = ("esdg_volume_rhs_f64", "esdg_volume_rhs_f32", "esdg_rhs_f64", "esdg_rhs_f32",
           "esdg_status_string", "esdg_min_order", "esdg_max_order")


class EsdgError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"esdg status {status}: {message}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libesdg.so; fails loudly if it has not been built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    try:  # bind to the HIP runtime torch ships, so one runtime serves both
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m entropy_stable_dg_amd.build`"
                           " (there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    for name in ("esdg_volume_rhs_f64", "esdg_volume_rhs_f32"):
        fn = getattr(lib, name)
        fn.restype = ci
        fn.argtypes = [vp, vp, vp, vp, ci, i64, vp, vp]
    for name in ("esdg_rhs_f64", "esdg_rhs_f32"):
        fn = getattr(lib, name)
        fn.restype = ci
        fn.argtypes = [vp, vp, vp, vp, vp, vp, ci, i64, vp, vp]
    lib.esdg_status_string.restype = ctypes.c_char_p
    lib.esdg_status_string.argtypes = [ci]
    lib.esdg_min_order.restype = ci
    lib.esdg_min_order.argtypes = []
    lib.esdg_max_order.restype = ci
    lib.esdg_max_order.argtypes = []
    if path == LIB_PATH:
        _lib = lib
    return lib


# --- C functions under their own names ----------------------------------------
def esdg_volume_rhs_f64(q: int, phi: int, geom: int, D: int, N: int, nelem: int, rhs: int,
                        stream: int = 0) -> int:
    return load().esdg_volume_rhs_f64(q, phi, geom, D, N, nelem, rhs, stream)


def esdg_volume_rhs_f32(q: int, phi: int, geom: int, D: int, N: int, nelem: int, rhs: int,
                        stream: int = 0) -> int:
    return load().esdg_volume_rhs_f32(q, phi, geom, D, N, nelem, rhs, stream)


def _host_vec3(omega, ctype):
    """omega as a host array of 3 values (or None -> NULL)."""
    if omega is None:
        return None
    vals = [float(x) for x in omega]
    if len(vals) != 3:
        raise ValueError("omega must have 3 components")
    return (ctype * 3)(*vals)


def esdg_rhs_f64(q: int, phi: int, geom: int, D: int, nbr: int, omega, N: int, nelem: int,
                 rhs: int, stream: int = 0) -> int:
    """omega: None or 3 numbers (host values)."""
    return load().esdg_rhs_f64(q, phi, geom, D, nbr, _host_vec3(omega, ctypes.c_double), N, nelem,
                               rhs, stream)


def esdg_rhs_f32(q: int, phi: int, geom: int, D: int, nbr: int, omega, N: int, nelem: int,
                 rhs: int, stream: int = 0) -> int:
    return load().esdg_rhs_f32(q, phi, geom, D, nbr, _host_vec3(omega, ctypes.c_float), N, nelem,
                               rhs, stream)


def esdg_status_string(status: int) -> str:
    return load().esdg_status_string(status).decode()


def esdg_min_order() -> int:
    return load().esdg_min_order()


def esdg_max_order() -> int:
    return load().esdg_max_order()


# --- tensor-level call ------------------------------------------------------------
def volume_rhs(q, phi, geom, D, out=None, stream=None):
    """rhs[5][nelem][Np] = volume term of (q, phi, geom, D) on the GPU.

    q [5][nelem][Np], phi [nelem][Np], geom [10][nelem][Np], D [N+1][N+1]:
    contiguous torch tensors of one dtype (float64 or float32) on one GPU.
    The call is asynchronous on `stream` (default: torch's current stream).
    """
    return _call(q, phi, geom, D, None, out, stream)


def rhs(q, phi, geom, D, nbr, omega=None, out=None, stream=None):
    """rhs[5][nelem][Np] = volume + entropy-conservative surface term (+ the
    Coriolis source -omega x U when omega, 3 numbers, is given) on the GPU;
    nbr [nelem][6] int32 face neighbours on the same GPU (-1 = slip wall),
    the rest as volume_rhs."""
    import torch

    if nbr is None or nbr.dtype != torch.int32:
        raise TypeError("nbr must be an int32 tensor")
    return _call(q, phi, geom, D, nbr, out, stream, omega)


def _call(q, phi, geom, D, nbr, out, stream, omega=None):
    import torch

    dtype = q.dtype
    if dtype not in (torch.float64, torch.float32):
        raise TypeError("q must be float64 or float32")
    named = (("q", q), ("phi", phi), ("geom", geom), ("D", D))
    for name, t in named:
        if t.dtype != dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    for name, t in named:
        if not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU (no CPU path)")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, expected {q.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if D.dim() != 2 or D.shape[0] != D.shape[1]:
        raise ValueError("D must be square [N+1][N+1]")
    N = D.shape[0] - 1
    Np = (N + 1) ** 3
    if q.dim() != 3 or q.shape[0] != 5 or q.shape[2] != Np:
        raise ValueError(f"q must be [5][nelem][{Np}]")
    nelem = q.shape[1]
    if tuple(phi.shape) != (nelem, Np):
        raise ValueError(f"phi must be [{nelem}][{Np}]")
    if tuple(geom.shape) != (10, nelem, Np):
        raise ValueError(f"geom must be [10][{nelem}][{Np}]")
    if nbr is not None:
        if not nbr.is_cuda or nbr.device != q.device or not nbr.is_contiguous():
            raise ValueError(f"nbr must be a contiguous GPU tensor on {q.device}")
        if tuple(nbr.shape) != (nelem, 6):
            raise ValueError(f"nbr must be [{nelem}][6]")
    if out is None:
        out = torch.empty_like(q)
    elif (out.dtype != dtype or out.device != q.device or tuple(out.shape) != tuple(q.shape)
          or not out.is_contiguous()):
        raise ValueError("out must match q in dtype, device, shape and be contiguous")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        if nbr is None:
            fn = esdg_volume_rhs_f64 if dtype == torch.float64 else esdg_volume_rhs_f32
            st = fn(q.data_ptr(), phi.data_ptr(), geom.data_ptr(), D.data_ptr(), N, nelem,
                    out.data_ptr(), handle)
        else:
            fn = esdg_rhs_f64 if dtype == torch.float64 else esdg_rhs_f32
            st = fn(q.data_ptr(), phi.data_ptr(), geom.data_ptr(), D.data_ptr(), nbr.data_ptr(),
                    omega, N, nelem, out.data_ptr(), handle)
    if st != ESDG_OK:
        raise EsdgError(st, esdg_status_string(st))
    return out
