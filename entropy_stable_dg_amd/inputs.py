"""Seeded synthetic inputs for the ESDG volume term: LGL nodes, the SBP
differentiation matrix, hexahedral meshes (affine or smoothly warped),
curl-form metric terms, and atmospheric states.

This module builds inputs only.  It holds none of the volume-term arithmetic
(no pressure recovery, no two-point flux, no log mean): both the CPU oracle
and the HIP library receive the arrays it returns and nothing else from it.

Page cited: "GPU Performance of an Entropy-Stable Discontinuous Galerkin Euler
Solver with Non-Conservative Terms" (arXiv 2605.16684v2), written [ESDG-GPU].

Array layouts (the library's contract):
  node index  n = a + Nq*(b + Nq*c), a along xi_1, b along xi_2, c along xi_3
  q     [5][nelem][Np]   rho, rho*u1, rho*u2, rho*u3, E  (E includes rho*phi)
  phi   [nelem][Np]      geopotential g*z
  geom  [10][nelem][Np]  Ja^1_1, Ja^1_2, Ja^1_3, Ja^2_1, ..., Ja^3_3, J
                         with Ja^k_j = J * d(xi_k)/d(x_j)
  D     [Nq][Nq]         D[a][l] = l_l'(xi_a)
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# Physical constants.  The pages give none; these are the usual dry-air
# values for the atmospheric workloads of [ESDG-GPU §5].
GAMMA = 1.4
R_GAS = 287.0
CP = GAMMA * R_GAS / (GAMMA - 1.0)  # 1004.5
CV = R_GAS / (GAMMA - 1.0)
GRAV = 9.81
P0 = 1.0e5


# ---------------------------------------------------------------------------
# 1D Legendre-Gauss-Lobatto operators (textbook; [ESDG-GPU §3] uses LGL
# collocation with an N_q x N_q differentiation matrix per direction).
# ---------------------------------------------------------------------------
def legendre(n: int, x: np.ndarray) -> np.ndarray:
    """P_n(x) by the three-term recurrence (n+1)P_{n+1} = (2n+1)xP_n - nP_{n-1}."""
    x = np.asarray(x, dtype=np.float64)
    if n == 0:
        return np.ones_like(x)
    p0, p1 = np.ones_like(x), x.copy()
    for k in range(1, n):
        p0, p1 = p1, ((2 * k + 1) * x * p1 - k * p0) / (k + 1)
    return p1


def lgl(N: int) -> tuple[np.ndarray, np.ndarray]:
    """Nodes and weights of the (N+1)-point LGL rule on [-1, 1].

    The nodes are the roots of q(x) = P_{N+1}(x) - P_{N-1}(x), which is a
    multiple of (1 - x^2) P_N'(x); q'(x) = (2N+1) P_N(x).  Newton's method is
    started from the Chebyshev-Gauss-Lobatto points.  Weights are
    w_j = 2 / (N (N+1) P_N(x_j)^2).
    """
    if N < 1:
        raise ValueError("LGL rule needs N >= 1")
    x = -np.cos(np.pi * np.arange(N + 1) / N)
    for _ in range(100):
        q = legendre(N + 1, x) - legendre(N - 1, x)
        dq = (2 * N + 1) * legendre(N, x)
        step = q / dq
        x = x - step
        if np.max(np.abs(step)) < 1e-16:
            break
    x[0], x[-1] = -1.0, 1.0
    x = 0.5 * (x - x[::-1])  # exact antisymmetry about 0
    w = 2.0 / (N * (N + 1) * legendre(N, x) ** 2)
    return x, w


def diff_matrix(N: int) -> np.ndarray:
    """Lagrange differentiation matrix on the LGL nodes, D[a][l] = l_l'(x_a).

    Off-diagonal: P_N(x_a) / (P_N(x_l) (x_a - x_l)).  Diagonal: minus the
    off-diagonal row sum, so that D annihilates constants to round-off
    (analytically -N(N+1)/4, 0, ..., 0, N(N+1)/4).
    """
    x, _ = lgl(N)
    pn = legendre(N, x)
    Nq = N + 1
    D = np.zeros((Nq, Nq))
    for a in range(Nq):
        for l in range(Nq):
            if a != l:
                D[a, l] = pn[a] / (pn[l] * (x[a] - x[l]))
    for a in range(Nq):
        D[a, a] = -np.sum(D[a, :])
    return D


# ---------------------------------------------------------------------------
# Hexahedral meshes and metric terms
# ---------------------------------------------------------------------------
def _apply_d(D: np.ndarray, f: np.ndarray, axis: int) -> np.ndarray:
    """Apply D along reference direction axis (0 -> xi_1, 1 -> xi_2, 2 -> xi_3)
    of an array shaped (..., Nq_c, Nq_b, Nq_a)."""
    if axis == 0:
        return np.einsum("ij,...cbj->...cbi", D, f)
    if axis == 1:
        return np.einsum("ij,...cja->...cia", D, f)
    return np.einsum("ij,...jba->...iba", D, f)


def box_mesh(K, lo, hi, N: int, warp_frac: float = 0.0, seed: int = 0,
             warp_wavelength=None) -> np.ndarray:
    """Node coordinates X[3][nelem][Nq][Nq][Nq] (indexed [d][e][c][b][a]).

    K = (Kx, Ky, Kz) elements on the box [lo, hi]; element e = ex + Kx*(ey + Ky*ez).
    With warp_frac > 0 each coordinate is displaced by
        warp_frac * h_d * prod_e sin(2 pi x_e / lambda_e + theta_{d,e})
    with seeded phases theta, evaluated at the LGL nodes (lambda defaults to
    the box length, so the map stays periodic and smooth).
    """
    Kx, Ky, Kz = K
    lo = np.asarray(lo, dtype=np.float64)
    hi = np.asarray(hi, dtype=np.float64)
    h = (hi - lo) / np.array([Kx, Ky, Kz], dtype=np.float64)
    xi, _ = lgl(N)
    Nq = N + 1
    t = 0.5 * (xi + 1.0)  # [0, 1] within an element
    ex = np.arange(Kx)
    ey = np.arange(Ky)
    ez = np.arange(Kz)
    # element order: ex fastest
    EZ, EY, EX = np.meshgrid(ez, ey, ex, indexing="ij")
    EX, EY, EZ = EX.ravel(), EY.ravel(), EZ.ravel()
    nelem = EX.size
    X = np.empty((3, nelem, Nq, Nq, Nq))
    X[0] = (lo[0] + h[0] * (EX[:, None, None, None] + t[None, None, None, :]))
    X[1] = (lo[1] + h[1] * (EY[:, None, None, None] + t[None, None, :, None]))
    X[2] = (lo[2] + h[2] * (EZ[:, None, None, None] + t[None, :, None, None]))
    if warp_frac:
        rng = np.random.default_rng(seed)
        theta = rng.uniform(0.0, 2.0 * np.pi, size=(3, 3))
        lam = (hi - lo) if warp_wavelength is None else np.asarray(warp_wavelength, dtype=np.float64)
        A = X.copy()
        for d in range(3):
            s = np.ones_like(A[0])
            for e in range(3):
                s = s * np.sin(2.0 * np.pi * (A[e] - lo[e]) / lam[e] + theta[d, e])
            X[d] = A[d] + warp_frac * h[d] * s
    return X


def metrics(X: np.ndarray, D: np.ndarray) -> np.ndarray:
    """geom[10][nelem][Np]: curl-form metric terms Ja^k_j and the Jacobian J.

    Ja^k_n = -xhat_k . curl_xi( X_l grad_xi X_m ), (n, m, l) cyclic
    (Kopriva, J. Sci. Comput. 26 (2006), conservative curl form), built with
    the same D so that sum_k D^k Ja^k_n = 0 holds to round-off (the metric
    identities).  J = det(dX/dxi) from the nodal derivatives.
    """
    nelem = X.shape[1]
    Nq = X.shape[2]
    dX = np.empty((3, 3) + X.shape[1:])  # dX[d][j] = dX_d / dxi_j
    for d in range(3):
        for j in range(3):
            dX[d, j] = _apply_d(D, X[d], j)
    # The curl form is unchanged by a per-element shift of X_l (the discrete
    # curl of a discrete gradient vanishes); element-centred coordinates keep
    # the products small and the metric identities tight in floating point.
    Xc = X - X.mean(axis=(2, 3, 4), keepdims=True)
    geom = np.empty((10, nelem, Nq, Nq, Nq))
    for n in range(3):
        m, l = (n + 1) % 3, (n + 2) % 3
        V = [Xc[l] * dX[m, j] for j in range(3)]  # V_j = X_l d_j X_m
        curl = [
            _apply_d(D, V[2], 1) - _apply_d(D, V[1], 2),
            _apply_d(D, V[0], 2) - _apply_d(D, V[2], 0),
            _apply_d(D, V[1], 0) - _apply_d(D, V[0], 1),
        ]
        for k in range(3):
            geom[3 * k + n] = -curl[k]
    A = np.moveaxis(dX, (0, 1), (-2, -1))
    geom[9] = np.linalg.det(A)
    if np.any(geom[9] <= 0.0):
        raise ValueError("mesh has non-positive Jacobian")
    return geom.reshape(10, nelem, Nq ** 3)


# ---------------------------------------------------------------------------
# Atmospheric states (Eq. 1 of [ESDG-GPU §2]: e = c_v T + |u|^2/2 + phi,
# E = rho e, phi = g z).  The workloads take their shapes from the rising
# thermal bubble ([ESDG-GPU §5.1, Eq. 9]) and the baroclinic channel
# ([ESDG-GPU §5.2]); base states are builder-defined since the pages cite
# them without formulas.
# ---------------------------------------------------------------------------
def conserved(rho, u, p, phi) -> np.ndarray:
    """q from primitives via the energy definition E = p/(gamma-1) + rho|u|^2/2 + rho phi."""
    E = p / (GAMMA - 1.0) + 0.5 * rho * (u[0] ** 2 + u[1] ** 2 + u[2] ** 2) + rho * phi
    return np.stack([rho, rho * u[0], rho * u[1], rho * u[2], E])


def state_isothermal(X, T0=300.0, u_noise=0.0, rho_noise=0.0, rng=None):
    """Isothermal hydrostatic atmosphere p = p0 exp(-g z/(R T0)), rho = p/(R T0),
    plus optional seeded uniform velocity noise (m/s) and relative density
    noise (pressure kept hydrostatic).  Returns (q, phi) shaped like X[0]."""
    z = X[2]
    phi = GRAV * z
    p = P0 * np.exp(-phi / (R_GAS * T0))
    rho = p / (R_GAS * T0)
    if rho_noise:
        rho = rho * (1.0 + rng.uniform(-rho_noise, rho_noise, size=rho.shape))
    u = np.zeros((3,) + z.shape)
    if u_noise:
        u = rng.uniform(-u_noise, u_noise, size=u.shape)
    return conserved(rho, u, p, phi), phi


def state_bubble(X, theta0=300.0, amp=0.5, rc=250.0, centre=(500.0, 500.0, 350.0),
                 u_noise=1e-3, rng=None):
    """Isentropic hydrostatic base (Exner pi = 1 - g z/(c_p theta0),
    p = p0 pi^(c_p/R)) with the smooth cosine potential-temperature bubble
    dtheta = amp (1 + cos(pi r/rc))/2 for r <= rc ([ESDG-GPU §5.1, Eq. 9]),
    T = theta pi, rho = p/(R T), seeded uniform velocity noise."""
    z = X[2]
    phi = GRAV * z
    pi_ex = 1.0 - GRAV * z / (CP * theta0)
    p = P0 * pi_ex ** (CP / R_GAS)
    r = np.sqrt((X[0] - centre[0]) ** 2 + (X[1] - centre[1]) ** 2 + (X[2] - centre[2]) ** 2)
    dtheta = np.where(r <= rc, amp * 0.5 * (1.0 + np.cos(np.pi * r / rc)), 0.0)
    T = (theta0 + dtheta) * pi_ex
    rho = p / (R_GAS * T)
    u = np.zeros((3,) + z.shape)
    if u_noise:
        u = rng.uniform(-u_noise, u_noise, size=u.shape)
    return conserved(rho, u, p, phi), phi


def state_channel(X, L, T0=300.0, T_noise=1.0, u_max=35.0, rng=None):
    """Stratified isothermal base with seeded +-T_noise K temperature noise
    (p hydrostatic for T0, rho = p/(R T)) and a zonal jet
    u1 = u_max sin^2(pi y/L_y) sin(pi z/L_z) (builder-defined stand-in for the
    balanced jet of the baroclinic channel, [ESDG-GPU §5.2])."""
    y, z = X[1], X[2]
    phi = GRAV * z
    p = P0 * np.exp(-phi / (R_GAS * T0))
    T = T0 + rng.uniform(-T_noise, T_noise, size=z.shape)
    rho = p / (R_GAS * T)
    u = np.zeros((3,) + z.shape)
    u[0] = u_max * np.sin(np.pi * y / L[1]) ** 2 * np.sin(np.pi * z / L[2])
    return conserved(rho, u, p, phi), phi


def reference_at_rest(state: str, X, theta0=300.0, T0=300.0):
    """The hydrostatic state at rest a workload's perturbation variables are
    taken about: the isentropic base of the bubble (without the bubble), the
    isothermal base of the other states.  Returns (rbar, pbar) shaped like
    X[0]."""
    z = X[2]
    phi = GRAV * z
    if state == "bubble":
        pi_ex = 1.0 - GRAV * z / (CP * theta0)
        p = P0 * pi_ex ** (CP / R_GAS)
        return p / (R_GAS * theta0 * pi_ex), p
    p = P0 * np.exp(-phi / (R_GAS * T0))
    return p / (R_GAS * T0), p


def perturbation_variables(q, phi, rbar, pbar):
    """q' = q - qbar with qbar = (rbar, 0, 0, 0, pbar/(gamma-1) + rbar phi),
    the reference at rest (fp64)."""
    qbar = conserved(rbar, np.zeros((3,) + np.shape(rbar)), pbar, phi)
    return q - qbar


# ---------------------------------------------------------------------------
# Named workloads
# ---------------------------------------------------------------------------
# Face order of the connectivity array: -xi1, +xi1, -xi2, +xi2, -xi3, +xi3.
FACE_WALL = -1


def box_connectivity(K, periodic=(True, True, True)) -> np.ndarray:
    """Face neighbours nbr[nelem][6] (int32) of the box mesh of box_mesh():
    element e = ex + Kx*(ey + Ky*ez); face 2k is the -xi_(k+1) face, 2k+1 the
    +xi_(k+1) face; the neighbour across a face holds the matching nodes on
    its opposite face with the same tangential indices.  Faces on the box
    boundary wrap around where `periodic` says so, else are FACE_WALL."""
    Kx, Ky, Kz = K
    Ks = (Kx, Ky, Kz)
    EZ, EY, EX = np.meshgrid(np.arange(Kz), np.arange(Ky), np.arange(Kx), indexing="ij")
    idx = [EX.ravel(), EY.ravel(), EZ.ravel()]
    nbr = np.empty((idx[0].size, 6), dtype=np.int32)
    for k in range(3):
        for side, step in ((0, -1), (1, 1)):
            c = [i.copy() for i in idx]
            c[k] = c[k] + step
            out = (c[k] < 0) | (c[k] >= Ks[k])
            c[k] = np.mod(c[k], Ks[k])
            e = c[0] + Kx * (c[1] + Ky * c[2])
            if not periodic[k]:
                e = np.where(out, FACE_WALL, e)
            nbr[:, 2 * k + side] = e
    return nbr


@dataclasses.dataclass
class Workload:
    name: str
    N: int
    nelem: int
    q: np.ndarray      # [5][nelem][Np]
    phi: np.ndarray    # [nelem][Np]
    geom: np.ndarray   # [10][nelem][Np]
    D: np.ndarray      # [Nq][Nq]
    X: np.ndarray      # [3][nelem][Np] node coordinates (tests only)
    seed: int
    dtype: str
    description: str
    nbr: np.ndarray = None          # [nelem][6] face neighbours (FACE_WALL = slip wall)
    periodic: tuple = (True, True, True)

    @property
    def Np(self) -> int:
        return (self.N + 1) ** 3

    @property
    def dof(self) -> int:
        return self.nelem * self.Np


def build_workload(name: str, K, lo, hi, N: int, state: str, seed: int,
                   warp_frac: float = 0.0, dtype: str = "f64", description: str = "",
                   warp_wavelength=None, state_kwargs=None,
                   periodic=(True, True, True)) -> Workload:
    """Mesh + metrics + state for an arbitrary box; the named configs below use it."""
    rng = np.random.default_rng(seed)
    D = diff_matrix(N)
    X = box_mesh(K, lo, hi, N, warp_frac=warp_frac, seed=seed + 7919,
                 warp_wavelength=warp_wavelength)
    geom = metrics(X, D)
    nelem = X.shape[1]
    Np = (N + 1) ** 3
    kw = dict(state_kwargs or {})
    if state == "isothermal":
        q, phi = state_isothermal(X, rng=rng, **kw)
    elif state == "bubble":
        q, phi = state_bubble(X, rng=rng, **kw)
    elif state == "channel":
        L = np.asarray(hi, dtype=np.float64) - np.asarray(lo, dtype=np.float64)
        q, phi = state_channel(X, L, rng=rng, **kw)
    else:
        raise ValueError(f"unknown state {state!r}")
    q = np.ascontiguousarray(q.reshape(5, nelem, Np))
    phi = np.ascontiguousarray(phi.reshape(nelem, Np))
    Xf = np.ascontiguousarray(X.reshape(3, nelem, Np))
    if dtype == "f32":
        q, phi, geom, D = (a.astype(np.float32) for a in (q, phi, geom, D))
    elif dtype != "f64":
        raise ValueError(dtype)
    return Workload(name, N, nelem, q, phi, np.ascontiguousarray(geom), np.ascontiguousarray(D),
                    Xf, seed, dtype, description, box_connectivity(K, periodic), tuple(periodic))


# The five workloads: sizes and state recipes.
CONFIGS = {
    "tiny": dict(K=(4, 4, 4), lo=(0, 0, 0), hi=(1, 1, 1), N=3, state="isothermal", seed=101,
                 state_kwargs=dict(u_noise=1.0, rho_noise=1e-3), periodic=(True, True, False),
                 description="4x4x4 affine hexes on the unit cube, N=3, isothermal hydrostatic "
                             "(T0=300 K) + U(-1,1) m/s velocity and 1e-3 relative density noise"),
    "bubble": dict(K=(16, 16, 16), lo=(0, 0, 0), hi=(1000, 1000, 1000), N=4, state="bubble",
                   seed=202, periodic=(True, True, False),
                   description="16^3 affine hexes on [0,1000]^3 m, N=4, isentropic base "
                               "theta0=300 K + cosine bubble (0.5 K, r=250 m, centre "
                               "(500,500,350)) + U(-1e-3,1e-3) m/s velocity noise"),
    "baroclinic": dict(K=(80, 16, 8), lo=(0, 0, 0), hi=(4.0e7, 6.0e6, 3.0e4), N=4,
                       state="channel", seed=303, warp_frac=0.05, periodic=(True, False, False),
                       description="80x16x8 hexes on a 40000x6000x30 km channel, N=4, "
                                   "isothermal 300 K base + U(-1,1) K noise, zonal jet 35 m/s, "
                                   "seeded sinusoidal warp of 5% of the element size"),
    "baroclinic_f32": dict(K=(80, 16, 8), lo=(0, 0, 0), hi=(4.0e7, 6.0e6, 3.0e4), N=4,
                           state="channel", seed=303, warp_frac=0.05, dtype="f32",
                           periodic=(True, False, False),
                           description="the baroclinic-channel workload rounded to fp32"),
    "bubble_f32": dict(K=(16, 16, 16), lo=(0, 0, 0), hi=(1000, 1000, 1000), N=4, state="bubble",
                       seed=202, dtype="f32", periodic=(True, True, False),
                       description="the rising-bubble workload rounded to fp32"),
    "high_order": dict(K=(24, 24, 24), lo=(0, 0, 0), hi=(1000, 1000, 1000), N=7, state="bubble",
                       seed=505, warp_frac=0.05, periodic=(True, True, False),
                       description="24^3 warped hexes on [0,1000]^3 m, N=7, rising-bubble "
                                   "state, 5% sinusoidal warp"),
}


def make(name: str, **override) -> Workload:
    """Build a named workload (seeded, deterministic)."""
    cfg = dict(CONFIGS[name])
    cfg.update(override)
    return build_workload(name, **cfg)


def make_perturbed(name: str, **override):
    """A named workload with its state as perturbation variables about its
    reference at rest (reference_at_rest).  Returns (wl, qp, ref): wl as
    make() returns it, qp [5][nelem][Np] and ref [2][nelem][Np] (rbar, pbar)
    in the workload's dtype, qp formed in fp64 from the fp64 state before
    rounding."""
    cfg = dict(CONFIGS[name])
    cfg.update(override)
    dtype = cfg.get("dtype", "f64")
    wl64 = build_workload(name, **dict(cfg, dtype="f64"))
    X = wl64.X
    rbar, pbar = reference_at_rest(cfg["state"], X)
    qp = perturbation_variables(wl64.q, wl64.phi, rbar, pbar)
    ref = np.stack([rbar, pbar])
    wl = wl64 if dtype == "f64" else build_workload(name, **cfg)
    npdt = np.float64 if dtype == "f64" else np.float32
    return wl, np.ascontiguousarray(qp.astype(npdt)), np.ascontiguousarray(ref.astype(npdt))


def dof_count(N: int, K=(1, 1, 1), L: int = 0) -> int:
    """Nodes of a mesh of K base elements refined L times: N_e = K 2^(3L),
    N_p = N_e (N+1)^3 ([ESDG-GPU §4.1 and §5.1])."""
    Kx, Ky, Kz = K
    return Kx * Ky * Kz * (2 ** (3 * L)) * (N + 1) ** 3
