"""CPU oracle of the ESDG flux-differencing volume term (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls it, and shares no code with it.

The arithmetic lives in ``esdg_oracle.c`` (plain C99, fp64, OpenMP over
elements); this module compiles it with gcc and calls it through ctypes.
Inputs in fp32 are promoted exactly to fp64 before the call.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "esdg_oracle.c")
_LIB = os.path.join(_HERE, "libesdg_oracle.so")

_P = ctypes.POINTER(ctypes.c_double)


def compile_library(src: str, out: str) -> str:
    """gcc -O2, OpenMP, no fast-math, no FMA contraction."""
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle into oracle/libesdg_oracle.so."""
    if force or not os.path.exists(_LIB):
        compile_library(_SRC, _LIB)
    return _LIB


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_P)


class Oracle:
    """ctypes handle on one build of the oracle library (the default build, or
    another path, e.g. a deliberately broken copy in a mutation test)."""

    def __init__(self, path: str | None = None):
        if path is None:
            if not os.path.exists(_LIB):
                build()
            path = _LIB
        lib = ctypes.CDLL(path)
        lib.oracle_volume_rhs.restype = ctypes.c_int
        lib.oracle_volume_rhs.argtypes = [_P, _P, _P, _P, ctypes.c_int, ctypes.c_int64, _P, _P,
                                          ctypes.c_int]
        lib.oracle_ec_flux.restype = None
        lib.oracle_ec_flux.argtypes = [_P, _P, _P, _P, ctypes.c_int, ctypes.c_int64, _P]
        lib.oracle_node_state.restype = None
        lib.oracle_node_state.argtypes = [_P, _P, ctypes.c_int64, _P]
        lib.oracle_surface_rhs.restype = ctypes.c_int
        lib.oracle_surface_rhs.argtypes = [_P, _P, _P, ctypes.POINTER(ctypes.c_int32), ctypes.c_int,
                                           ctypes.c_int64, _P, _P, ctypes.c_int]
        lib.oracle_add_coriolis.restype = None
        lib.oracle_add_coriolis.argtypes = [_P, _P, ctypes.c_int64, _P]
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        self.lib = lib
        self.path = path

    def volume_rhs(self, q, phi, geom, D, N: int, *, with_magnitude: bool = False,
                   threads: int = 0):
        """Volume term rhs[5][nelem][Np] of the semi-discrete ESDG form.

        With ``with_magnitude`` also returns mag[5][nelem][Np], the per-node sum
        of the absolute values of the summands of rhs (the scale of its
        round-off)."""
        q, phi, geom, D = _f64(q), _f64(phi), _f64(geom), _f64(D)
        Nq = N + 1
        Np = Nq ** 3
        if D.shape != (Nq, Nq):
            raise ValueError("D must be (N+1) x (N+1)")
        nelem = phi.size // Np
        if q.size != 5 * nelem * Np or phi.size != nelem * Np or geom.size != 10 * nelem * Np:
            raise ValueError("array sizes do not match N and nelem")
        rhs = np.empty((5, nelem, Np))
        mag = np.empty((5, nelem, Np)) if with_magnitude else None
        rc = self.lib.oracle_volume_rhs(_ptr(q), _ptr(phi), _ptr(geom), _ptr(D), N, nelem,
                                        _ptr(rhs), _ptr(mag) if mag is not None else None,
                                        int(threads))
        if rc != 0:
            raise ValueError(f"oracle_volume_rhs failed ({rc})")
        return (rhs, mag) if with_magnitude else rhs

    def surface_rhs(self, q, phi, geom, nbr, N: int, *, rhs=None, mag=None, threads: int = 0):
        """Surface term of the semi-discrete ESDG form with the entropy-
        conservative flux, added to ``rhs`` (zeros when None) and returned;
        ``mag`` (optional) accumulates its absolute values.  nbr [nelem][6]
        int32 face neighbours, -1 = slip wall."""
        q, phi, geom = _f64(q), _f64(phi), _f64(geom)
        nbr = np.ascontiguousarray(nbr, dtype=np.int32)
        Np = (N + 1) ** 3
        nelem = phi.size // Np
        if q.size != 5 * nelem * Np or geom.size != 10 * nelem * Np or nbr.shape != (nelem, 6):
            raise ValueError("array sizes do not match N and nelem")
        if rhs is None:
            rhs = np.zeros((5, nelem, Np))
        if rhs.dtype != np.float64 or not rhs.flags.c_contiguous or rhs.size != 5 * nelem * Np:
            raise ValueError("rhs must be a contiguous float64 [5][nelem][Np] array")
        if mag is not None and (mag.dtype != np.float64 or not mag.flags.c_contiguous
                                or mag.size != 5 * nelem * Np):
            raise ValueError("mag must be a contiguous float64 [5][nelem][Np] array")
        rc = self.lib.oracle_surface_rhs(_ptr(q), _ptr(phi), _ptr(geom),
                                         nbr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), N, nelem,
                                         _ptr(rhs), _ptr(mag) if mag is not None else None,
                                         int(threads))
        if rc != 0:
            raise ValueError(f"oracle_surface_rhs failed ({rc})")
        return rhs

    def rhs(self, q, phi, geom, D, nbr, N: int, *, omega=None, with_magnitude: bool = False,
            threads: int = 0):
        """Whole semi-discrete right-hand side: volume + entropy-conservative
        surface term + the Coriolis source -omega x U (omega None: h = 0)."""
        out = self.volume_rhs(q, phi, geom, D, N, with_magnitude=with_magnitude, threads=threads)
        rhs, mag = out if with_magnitude else (out, None)
        self.surface_rhs(q, phi, geom, nbr, N, rhs=rhs, mag=mag, threads=threads)
        if omega is not None:
            self.add_coriolis(q, omega, rhs)
            if mag is not None:
                h = np.zeros_like(rhs)
                self.add_coriolis(q, omega, h)
                mag += np.abs(h)
        return (rhs, mag) if with_magnitude else rhs

    def add_coriolis(self, q, omega, rhs):
        """rhs[1:4] -= omega x U at every node (in place); q, rhs [5][...]."""
        q = _f64(q)
        om = _f64(omega).reshape(3)
        if rhs.dtype != np.float64 or not rhs.flags.c_contiguous or rhs.shape != q.shape:
            raise ValueError("rhs must be a contiguous float64 array shaped like q")
        self.lib.oracle_add_coriolis(_ptr(q), _ptr(om), q.size // 5, _ptr(rhs))
        return rhs

    def ec_flux(self, qi, phii, ql, phil, j: int) -> np.ndarray:
        """Two-point flux F_j(q_i, q_l) for a batch of pairs: qi, ql [n][5]
        conserved states, phii, phil [n]; returns [n][5]."""
        qi, ql = _f64(qi).reshape(-1, 5), _f64(ql).reshape(-1, 5)
        phii, phil = _f64(phii).reshape(-1), _f64(phil).reshape(-1)
        n = qi.shape[0]
        if not (ql.shape[0] == phii.size == phil.size == n):
            raise ValueError("batch sizes differ")
        F = np.empty((n, 5))
        self.lib.oracle_ec_flux(_ptr(qi), _ptr(phii), _ptr(ql), _ptr(phil), int(j), n, _ptr(F))
        return F

    def node_state(self, q, phi) -> np.ndarray:
        """Per-node (rho, u1, u2, u3, p, b) for conserved states q [n][5]."""
        q = _f64(q).reshape(-1, 5)
        phi = _f64(phi).reshape(-1)
        out = np.empty((q.shape[0], 6))
        self.lib.oracle_node_state(_ptr(q), _ptr(phi), q.shape[0], _ptr(out))
        return out

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())


_default = None


def default() -> Oracle:
    """The oracle built from oracle/esdg_oracle.c (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def volume_rhs(*args, **kwargs):
    return default().volume_rhs(*args, **kwargs)


def ec_flux(*args, **kwargs):
    return default().ec_flux(*args, **kwargs)


def surface_rhs(*args, **kwargs):
    return default().surface_rhs(*args, **kwargs)


def rhs(*args, **kwargs):
    return default().rhs(*args, **kwargs)


def node_state(*args, **kwargs):
    return default().node_state(*args, **kwargs)


def max_threads() -> int:
    return default().max_threads()
