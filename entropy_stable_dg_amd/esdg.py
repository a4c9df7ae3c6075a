"""Python binding of libesdg (ctypes).  Argument marshalling only: every step of
the volume term runs in the HIP kernels of libesdg.so; there is no CPU path.

Two levels:
  * every C function of include/esdg.h under its own name (device pointers as
    Python ints, host arrays as sequences, a status code returned);
  * volume_rhs, rhs, rhs_pert, lsrk_stage, lsrk_steps, integrals -- the same
    calls on torch tensors resident on the GPU, raising EsdgError on a bad
    status.
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
ESDG_ERR_DEVICE = -7

# every symbol include/esdg.h declares
EXPORTS = ("esdg_volume_rhs_f64", "esdg_volume_rhs_f32", "esdg_rhs_f64", "esdg_rhs_f32",
           "esdg_rhs_pert_f64", "esdg_rhs_pert_f32", "esdg_lsrk_stage_f64", "esdg_lsrk_stage_f32",
           "esdg_lsrk_steps_f64", "esdg_lsrk_steps_f32", "esdg_lsrk_stages",
           "esdg_lsrk_coefficients", "esdg_integrals_workspace_bytes", "esdg_integrals_f64",
           "esdg_integrals_f32", "esdg_integrals_noalloc_f64", "esdg_status_string",
           "esdg_min_order", "esdg_max_order")


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
    for name in ("esdg_rhs_pert_f64", "esdg_rhs_pert_f32"):
        fn = getattr(lib, name)
        fn.restype = ci
        fn.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, i64, vp, vp]
    for name, real in (("esdg_lsrk_stage_f64", ctypes.c_double), ("esdg_lsrk_stage_f32", ctypes.c_float)):
        fn = getattr(lib, name)
        fn.restype = ci
        fn.argtypes = [vp, vp, vp, vp, vp, vp, vp, real, real, real, ci, i64, vp, vp, vp]
    for name, real in (("esdg_lsrk_steps_f64", ctypes.c_double), ("esdg_lsrk_steps_f32", ctypes.c_float)):
        fn = getattr(lib, name)
        fn.restype = ci
        fn.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, real, ci, ci, i64, vp]
    lib.esdg_lsrk_stages.restype = ci
    lib.esdg_lsrk_stages.argtypes = []
    lib.esdg_lsrk_coefficients.restype = ci
    lib.esdg_lsrk_coefficients.argtypes = [ctypes.POINTER(ctypes.c_double)] * 2
    lib.esdg_integrals_workspace_bytes.restype = i64
    lib.esdg_integrals_workspace_bytes.argtypes = []
    for name in ("esdg_integrals_f64", "esdg_integrals_f32"):
        fn = getattr(lib, name)
        fn.restype = ci
        fn.argtypes = [vp, vp, vp, vp, vp, ci, i64, vp, vp, vp]
    lib.esdg_integrals_noalloc_f64.restype = ci
    lib.esdg_integrals_noalloc_f64.argtypes = [vp, vp, vp, vp, vp, ci, i64, vp, vp]
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


def esdg_rhs_pert_f64(qp: int, ref: int, phi: int, geom: int, D: int, nbr: int, omega, N: int,
                      nelem: int, rhs: int, stream: int = 0) -> int:
    return load().esdg_rhs_pert_f64(qp, ref, phi, geom, D, nbr, _host_vec3(omega, ctypes.c_double),
                                    N, nelem, rhs, stream)


def esdg_rhs_pert_f32(qp: int, ref: int, phi: int, geom: int, D: int, nbr: int, omega, N: int,
                      nelem: int, rhs: int, stream: int = 0) -> int:
    return load().esdg_rhs_pert_f32(qp, ref, phi, geom, D, nbr, _host_vec3(omega, ctypes.c_float),
                                    N, nelem, rhs, stream)


def esdg_lsrk_stage_f64(q_in: int, ref: int, phi: int, geom: int, D: int, nbr: int, omega,
                        a: float, b: float, dt: float, N: int, nelem: int, dq: int, q_out: int,
                        stream: int = 0) -> int:
    return load().esdg_lsrk_stage_f64(q_in, ref, phi, geom, D, nbr,
                                      _host_vec3(omega, ctypes.c_double), a, b, dt, N, nelem, dq,
                                      q_out, stream)


def esdg_lsrk_stage_f32(q_in: int, ref: int, phi: int, geom: int, D: int, nbr: int, omega,
                        a: float, b: float, dt: float, N: int, nelem: int, dq: int, q_out: int,
                        stream: int = 0) -> int:
    return load().esdg_lsrk_stage_f32(q_in, ref, phi, geom, D, nbr,
                                      _host_vec3(omega, ctypes.c_float), a, b, dt, N, nelem, dq,
                                      q_out, stream)


def esdg_lsrk_steps_f64(q: int, q_tmp: int, dq: int, ref: int, phi: int, geom: int, D: int,
                        nbr: int, omega, dt: float, nsteps: int, N: int, nelem: int,
                        stream: int = 0) -> int:
    return load().esdg_lsrk_steps_f64(q, q_tmp, dq, ref, phi, geom, D, nbr,
                                      _host_vec3(omega, ctypes.c_double), dt, nsteps, N, nelem,
                                      stream)


def esdg_lsrk_steps_f32(q: int, q_tmp: int, dq: int, ref: int, phi: int, geom: int, D: int,
                        nbr: int, omega, dt: float, nsteps: int, N: int, nelem: int,
                        stream: int = 0) -> int:
    return load().esdg_lsrk_steps_f32(q, q_tmp, dq, ref, phi, geom, D, nbr,
                                      _host_vec3(omega, ctypes.c_float), dt, nsteps, N, nelem,
                                      stream)


def esdg_lsrk_stages() -> int:
    return load().esdg_lsrk_stages()


def esdg_lsrk_coefficients():
    """(A, B): the library's stage coefficients as two lists (host values)."""
    n = esdg_lsrk_stages()
    A, B = (ctypes.c_double * n)(), (ctypes.c_double * n)()
    st = load().esdg_lsrk_coefficients(A, B)
    if st != ESDG_OK:
        raise EsdgError(st, esdg_status_string(st))
    return list(A), list(B)


def esdg_integrals_workspace_bytes() -> int:
    return load().esdg_integrals_workspace_bytes()


def esdg_integrals_f64(q: int, ref: int, phi: int, geom: int, w: int, N: int, nelem: int,
                       work: int, out: int, stream: int = 0) -> int:
    return load().esdg_integrals_f64(q, ref, phi, geom, w, N, nelem, work, out, stream)


def esdg_integrals_f32(q: int, ref: int, phi: int, geom: int, w: int, N: int, nelem: int,
                       work: int, out: int, stream: int = 0) -> int:
    return load().esdg_integrals_f32(q, ref, phi, geom, w, N, nelem, work, out, stream)


def esdg_integrals_noalloc_f64(q: int, ref: int, phi: int, geom: int, w: int, N: int,
                               nelem: int, out: int, stream: int = 0) -> int:
    return load().esdg_integrals_noalloc_f64(q, ref, phi, geom, w, N, nelem, out, stream)


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


def _check(status: int) -> None:
    if status != ESDG_OK:
        raise EsdgError(status, esdg_status_string(status))


def _validate(q, phi, geom, D, nbr=None, ref=None):
    """Checks the tensors of one call; returns (N, nelem)."""
    import torch

    dtype = q.dtype
    if dtype not in (torch.float64, torch.float32):
        raise TypeError("q must be float64 or float32")
    named = [("q", q), ("phi", phi), ("geom", geom), ("D", D)]
    if ref is not None:
        named.append(("ref", ref))
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
    if ref is not None and tuple(ref.shape) != (2, nelem, Np):
        raise ValueError(f"ref must be [2][{nelem}][{Np}]")
    if nbr is not None:
        if nbr.dtype != torch.int32:
            raise TypeError("nbr must be an int32 tensor")
        if not nbr.is_cuda or nbr.device != q.device or not nbr.is_contiguous():
            raise ValueError(f"nbr must be a contiguous GPU tensor on {q.device}")
        if tuple(nbr.shape) != (nelem, 6):
            raise ValueError(f"nbr must be [{nelem}][6]")
    return N, nelem


def _like(t, q, name):
    """A caller's buffer shaped like q (allocated when None)."""
    import torch

    if t is None:
        return torch.empty_like(q)
    if (t.dtype != q.dtype or t.device != q.device or tuple(t.shape) != tuple(q.shape)
            or not t.is_contiguous()):
        raise ValueError(f"{name} must match q in dtype, device, shape and be contiguous")
    return t


def _stream_handle(stream, device):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def rhs_pert(qp, ref, phi, geom, D, nbr, omega=None, out=None, stream=None):
    """Whole right-hand side of the state carried as perturbation variables qp
    [5][nelem][Np] about the reference at rest ref [2][nelem][Np] (density,
    pressure); the rest as rhs()."""
    import torch

    N, nelem = _validate(qp, phi, geom, D, nbr, ref)
    out = _like(out, qp, "out")
    fn = esdg_rhs_pert_f64 if qp.dtype == torch.float64 else esdg_rhs_pert_f32
    with torch.cuda.device(qp.device):
        _check(fn(qp.data_ptr(), ref.data_ptr(), phi.data_ptr(), geom.data_ptr(), D.data_ptr(),
                  nbr.data_ptr(), omega, N, nelem, out.data_ptr(), _stream_handle(stream, qp.device)))
    return out


def lsrk_stage(q_in, phi, geom, D, nbr, a, b, dt, dq, q_out=None, ref=None, omega=None,
               stream=None):
    """One fused Runge-Kutta stage: dq <- a dq + dt rhs(q_in) (in place),
    q_out <- q_in + b dq (returned; allocated when None)."""
    import torch

    N, nelem = _validate(q_in, phi, geom, D, nbr, ref)
    dq = _like(dq, q_in, "dq")
    q_out = _like(q_out, q_in, "q_out")
    fn = esdg_lsrk_stage_f64 if q_in.dtype == torch.float64 else esdg_lsrk_stage_f32
    with torch.cuda.device(q_in.device):
        _check(fn(q_in.data_ptr(), ref.data_ptr() if ref is not None else None, phi.data_ptr(),
                  geom.data_ptr(), D.data_ptr(), nbr.data_ptr(), omega, float(a), float(b),
                  float(dt), N, nelem, dq.data_ptr(), q_out.data_ptr(),
                  _stream_handle(stream, q_in.device)))
    return q_out


def lsrk_steps(q, phi, geom, D, nbr, dt, nsteps, ref=None, omega=None, q_tmp=None, dq=None,
               stream=None):
    """nsteps Runge-Kutta steps of size dt on q, in place (returned); q_tmp and
    dq are workspaces (allocated when None)."""
    import torch

    N, nelem = _validate(q, phi, geom, D, nbr, ref)
    q_tmp = _like(q_tmp, q, "q_tmp")
    dq = _like(dq, q, "dq")
    fn = esdg_lsrk_steps_f64 if q.dtype == torch.float64 else esdg_lsrk_steps_f32
    with torch.cuda.device(q.device):
        _check(fn(q.data_ptr(), q_tmp.data_ptr(), dq.data_ptr(),
                  ref.data_ptr() if ref is not None else None, phi.data_ptr(), geom.data_ptr(),
                  D.data_ptr(), nbr.data_ptr(), omega, float(dt), int(nsteps), N, nelem,
                  _stream_handle(stream, q.device)))
    return q


def integrals(q, phi, geom, w, ref=None, work=None, out=None, stream=None):
    """Device float64 tensor [3]: the sums of the integrals of rho, E and the
    entropy -rho s/(gamma-1) over the mesh; w [N+1] the LGL weights (same
    dtype and device as q)."""
    import torch

    Nq = w.shape[0]
    D_dummy = torch.empty((Nq, Nq), dtype=q.dtype, device=q.device)
    N, nelem = _validate(q, phi, geom, D_dummy, None, ref)
    if w.dtype != q.dtype or w.device != q.device or not w.is_contiguous() or w.dim() != 1:
        raise ValueError("w must be a contiguous 1-D tensor like q")
    if work is None:
        work = torch.empty(esdg_integrals_workspace_bytes() // 8, dtype=torch.float64,
                           device=q.device)
    if out is None:
        out = torch.empty(3, dtype=torch.float64, device=q.device)
    fn = esdg_integrals_f64 if q.dtype == torch.float64 else esdg_integrals_f32
    with torch.cuda.device(q.device):
        _check(fn(q.data_ptr(), ref.data_ptr() if ref is not None else None, phi.data_ptr(),
                  geom.data_ptr(), w.data_ptr(), N, nelem, work.data_ptr(), out.data_ptr(),
                  _stream_handle(stream, q.device)))
    return out


def integrals_noalloc(q, phi, geom, w, out, ref=None, stream=None):
    """integrals() of a float64 state through the allocation-free entry point:
    `out` (device float64 [3]) is the caller's; the partial sums use the
    library's own device array."""
    import torch

    Nq = w.shape[0]
    D_dummy = torch.empty((Nq, Nq), dtype=q.dtype, device=q.device)
    N, nelem = _validate(q, phi, geom, D_dummy, None, ref)
    if q.dtype != torch.float64:
        raise TypeError("the allocation-free integrals take float64 states")
    if w.dtype != q.dtype or w.device != q.device or not w.is_contiguous() or w.dim() != 1:
        raise ValueError("w must be a contiguous 1-D tensor like q")
    if (out.dtype != torch.float64 or out.device != q.device or out.numel() != 3
            or not out.is_contiguous()):
        raise ValueError("out must be a contiguous float64 tensor of 3 values on q's device")
    with torch.cuda.device(q.device):
        _check(esdg_integrals_noalloc_f64(q.data_ptr(), ref.data_ptr() if ref is not None else None,
                                          phi.data_ptr(), geom.data_ptr(), w.data_ptr(), N, nelem,
                                          out.data_ptr(), _stream_handle(stream, q.device)))
    return out


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
