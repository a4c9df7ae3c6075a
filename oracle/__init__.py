"""CPU oracle of the ESDG right-hand side and its time stepping (test
infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls it, and shares no code with it.

The arithmetic lives in ``esdg_oracle.c`` (plain C99, OpenMP over elements);
this module compiles it with gcc twice and calls it through ctypes:

  * ``libesdg_oracle.so``      -- long double arithmetic (64-bit significand):
                                  the reference every GPU result is compared
                                  with (``default()`` and the module-level
                                  functions);
  * ``libesdg_oracle_f64.so``  -- double arithmetic: the variant timed as the
                                  CPU baseline (``fp64()``).

Inputs and outputs are float64 arrays; fp32 inputs are promoted exactly.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "esdg_oracle.c")
_LIB = os.path.join(_HERE, "libesdg_oracle.so")          # long double
_LIB_F64 = os.path.join(_HERE, "libesdg_oracle_f64.so")  # double

_P = ctypes.POINTER(ctypes.c_double)
_ODE_FN = ctypes.CFUNCTYPE(None, _P, _P, ctypes.c_int64)


def compile_library(src: str, out: str, long_double: bool = True) -> str:
    """gcc -O2, OpenMP, no fast-math, no FMA contraction; long double
    arithmetic unless `long_double` is False."""
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-Wextra"]
    if long_double:
        cmd.append("-DORACLE_LONG_DOUBLE")
    cmd += ["-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile both builds of the oracle (long double and double)."""
    if force or not os.path.exists(_LIB_F64):
        compile_library(_SRC, _LIB_F64, long_double=False)
    if force or not os.path.exists(_LIB):
        compile_library(_SRC, _LIB, long_double=True)
    return _LIB


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_P)


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _nodes(N: int) -> int:
    return (N + 1) ** 3


class Oracle:
    """ctypes handle on one build of the oracle library (the default build, the
    fp64 build, or another path, e.g. a deliberately broken copy in a mutation
    test)."""

    def __init__(self, path: str | None = None):
        if path is None:
            if not os.path.exists(_LIB):
                build(force=False)
            path = _LIB
        lib = ctypes.CDLL(path)
        i64, ci, cd = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        i32p = ctypes.POINTER(ctypes.c_int32)
        lib.oracle_volume_rhs.restype = ci
        lib.oracle_volume_rhs.argtypes = [_P, _P, _P, _P, ci, i64, _P, _P, ci]
        lib.oracle_ec_flux.restype = None
        lib.oracle_ec_flux.argtypes = [_P, _P, _P, _P, ci, i64, _P]
        lib.oracle_surface_rhs.restype = ci
        lib.oracle_surface_rhs.argtypes = [_P, _P, _P, i32p, ci, i64, _P, _P, ci]
        lib.oracle_add_coriolis.restype = None
        lib.oracle_add_coriolis.argtypes = [_P, _P, i64, _P]
        lib.oracle_lsrk_coefficients.restype = None
        lib.oracle_lsrk_coefficients.argtypes = [_P, _P]
        lib.oracle_lsrk_ode.restype = ci
        lib.oracle_lsrk_ode.argtypes = [_P, i64, cd, ci, _ODE_FN]
        lib.oracle_lsrk_esdg.restype = ci
        lib.oracle_lsrk_esdg.argtypes = [_P, _P, _P, _P, i32p, _P, ci, i64, cd, ci, ci]
        lib.oracle_integrals.restype = ci
        lib.oracle_integrals.argtypes = [_P, _P, _P, _P, ci, i64, _P]
        lib.oracle_full_state.restype = None
        lib.oracle_full_state.argtypes = [_P, _P, _P, i64, _P]
        lib.oracle_mantissa_bits.restype = ci
        lib.oracle_mantissa_bits.argtypes = []
        lib.oracle_max_threads.restype = ci
        lib.oracle_max_threads.argtypes = []
        self.lib = lib
        self.path = path

    @property
    def mantissa_bits(self) -> int:
        """Significand bits of the build's arithmetic (64 long double, 53 double)."""
        return int(self.lib.oracle_mantissa_bits())

    def volume_rhs(self, q, phi, geom, D, N: int, *, with_magnitude: bool = False,
                   threads: int = 0):
        """Volume term rhs[5][nelem][Np] of the semi-discrete ESDG form.

        With ``with_magnitude`` also returns mag[5][nelem][Np], the per-node sum
        of the absolute values of the summands of rhs (the scale of its
        round-off)."""
        q, phi, geom, D = _f64(q), _f64(phi), _f64(geom), _f64(D)
        Nq = N + 1
        Np = _nodes(N)
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
        Np = _nodes(N)
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
        rc = self.lib.oracle_surface_rhs(_ptr(q), _ptr(phi), _ptr(geom), _i32p(nbr), N, nelem,
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

    # --- time stepping ----------------------------------------------------------
    def lsrk_coefficients(self):
        """(A[5], B[5]) of the five-stage fourth-order 2N-storage scheme."""
        A, B = np.empty(5), np.empty(5)
        self.lib.oracle_lsrk_coefficients(_ptr(A), _ptr(B))
        return A, B

    def lsrk_ode(self, f, y0, dt: float, nsteps: int) -> np.ndarray:
        """nsteps steps of the oracle's stepper on dy/dt = f(y), f a Python
        function of a float64 vector returning one of the same size."""
        y = _f64(y0).reshape(-1).copy()
        n = y.size

        def cb(yp, dyp, m):
            yy = np.ctypeslib.as_array(yp, shape=(m,))
            out = np.asarray(f(yy.copy()), dtype=np.float64).reshape(m)
            np.ctypeslib.as_array(dyp, shape=(m,))[:] = out

        fn = _ODE_FN(cb)
        rc = self.lib.oracle_lsrk_ode(_ptr(y), n, float(dt), int(nsteps), fn)
        if rc != 0:
            raise ValueError(f"oracle_lsrk_ode failed ({rc})")
        return y

    def lsrk(self, q, phi, geom, D, nbr, N: int, dt: float, nsteps: int, *, omega=None,
             threads: int = 0) -> np.ndarray:
        """The state after nsteps steps of size dt of dq/dt = rhs(q), the whole
        right-hand side (volume + surface + the Coriolis source for omega)."""
        out = _f64(q).copy()
        phi, geom, D = _f64(phi), _f64(geom), _f64(D)
        nbr = np.ascontiguousarray(nbr, dtype=np.int32)
        Np = _nodes(N)
        nelem = phi.size // Np
        if out.size != 5 * nelem * Np or geom.size != 10 * nelem * Np or nbr.shape != (nelem, 6):
            raise ValueError("array sizes do not match N and nelem")
        om = _f64(omega).reshape(3) if omega is not None else None
        rc = self.lib.oracle_lsrk_esdg(_ptr(out), _ptr(phi), _ptr(geom), _ptr(D), _i32p(nbr),
                                       _ptr(om) if om is not None else None, N, nelem, float(dt),
                                       int(nsteps), int(threads))
        if rc != 0:
            raise ValueError(f"oracle_lsrk_esdg failed ({rc})")
        return out

    def integrals(self, q, phi, geom, w, N: int) -> np.ndarray:
        """[sum of integrals of rho, of E, of the entropy -rho s/(gamma-1)]."""
        q, phi, geom, w = _f64(q), _f64(phi), _f64(geom), _f64(w)
        Np = _nodes(N)
        nelem = phi.size // Np
        if q.size != 5 * nelem * Np or geom.size != 10 * nelem * Np or w.size != N + 1:
            raise ValueError("array sizes do not match N and nelem")
        out = np.empty(3)
        rc = self.lib.oracle_integrals(_ptr(q), _ptr(phi), _ptr(geom), _ptr(w), N, nelem, _ptr(out))
        if rc != 0:
            raise ValueError(f"oracle_integrals failed ({rc})")
        return out

    def full_state(self, qp, ref, phi) -> np.ndarray:
        """Full conserved state from perturbation variables about a reference
        at rest: qp [5][...], ref [2][...] (reference density, pressure),
        phi [...] -> q [5][...]."""
        qp, ref, phi = _f64(qp), _f64(ref), _f64(phi)
        n = phi.size
        if qp.size != 5 * n or ref.size != 2 * n:
            raise ValueError("array sizes differ")
        q = np.empty_like(qp)
        self.lib.oracle_full_state(_ptr(qp), _ptr(ref), _ptr(phi), n, _ptr(q))
        return q

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())


_default = None
_fp64 = None


def default() -> Oracle:
    """The long double reference build (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def fp64() -> Oracle:
    """The double build, timed as the CPU baseline (built on first use)."""
    global _fp64
    if _fp64 is None:
        if not os.path.exists(_LIB_F64):
            build(force=False)
        _fp64 = Oracle(_LIB_F64)
    return _fp64


def volume_rhs(*args, **kwargs):
    return default().volume_rhs(*args, **kwargs)


def ec_flux(*args, **kwargs):
    return default().ec_flux(*args, **kwargs)


def surface_rhs(*args, **kwargs):
    return default().surface_rhs(*args, **kwargs)


def rhs(*args, **kwargs):
    return default().rhs(*args, **kwargs)


def lsrk(*args, **kwargs):
    return default().lsrk(*args, **kwargs)


def integrals(*args, **kwargs):
    return default().integrals(*args, **kwargs)


def full_state(*args, **kwargs):
    return default().full_state(*args, **kwargs)


def max_threads() -> int:
    return default().max_threads()
