"""Work and traffic model of the volume term, and MI355X peak figures.

Algorithmic traffic per node (DOF): the kernel must read 5 conserved fields,
the geopotential and 10 geometry values (9 metric terms and J) and write 5
fields: 21 values = 168 B in fp64, 84 B in fp32.  The differentiation matrix
(N+1)^2 values per launch is added once.

FLOP counting convention (counted from the kernel's arithmetic; the method's
work, not the ordered-pair work the symmetric evaluation avoids):
  +, -, x, / and reciprocal = 1 FLOP, fused multiply-add = 2, log = 1;
  comparisons and selects = 0; the log means are counted on their series
  branch; quantities hoisted per node are counted once per node.
  per unordered pair on a line ........ 120
  per node (primitives, p, b, 2 logs,
            1/b, direction sum, -1/J) ...  38
Unordered pairs per element: 3 (N+1)^2 (N+1) N / 2.

Whole right-hand side (volume + entropy-conservative surface term, one fused
kernel): the algorithmic traffic adds only the connectivity, 6 int32 per
element; the kernel also re-reads each face partner's 5 fields and phi from
the neighbouring element (48 B per face node in fp64 with a neighbour, none at
a slip wall), which the cache may or may not serve.  Work per face node: one
pair (120) plus the partner's per-node values (38) with a neighbour; one pair
and the mirror state (12) at a slip wall.
"""
from __future__ import annotations

FLOP_PER_PAIR = 120
FLOP_PER_NODE = 38

# MI355X (gfx950) published peaks
PEAK_HBM_GBS = 8000.0          # HBM3E, GB/s
PEAK_FP64_VECTOR_TFLOPS = 78.6
PEAK_FP32_VECTOR_TFLOPS = 157.3
CU_COUNT = 256
CLOCK_GHZ = 2.4


def pairs_per_element(N: int) -> int:
    Nq = N + 1
    return 3 * Nq * Nq * (Nq * (Nq - 1) // 2)


def flops_per_element(N: int) -> int:
    return pairs_per_element(N) * FLOP_PER_PAIR + (N + 1) ** 3 * FLOP_PER_NODE


def flops_per_dof(N: int) -> float:
    return flops_per_element(N) / (N + 1) ** 3


def bytes_per_dof(dtype: str) -> int:
    return 21 * (8 if dtype == "f64" else 4)


def algorithmic_bytes(N: int, nelem: int, dtype: str) -> int:
    size = 8 if dtype == "f64" else 4
    return nelem * (N + 1) ** 3 * bytes_per_dof(dtype) + (N + 1) ** 2 * size


def arithmetic_intensity(N: int, dtype: str) -> float:
    return flops_per_dof(N) / bytes_per_dof(dtype)


FLOP_PER_MIRROR = 12


def face_nodes_per_element(N: int) -> int:
    return 6 * (N + 1) ** 2


def surface_flops(N: int, nbr) -> int:
    """FLOP of the surface term over a mesh with connectivity nbr [nelem][6]."""
    import numpy as np

    nbr = np.asarray(nbr)
    walls = int((nbr < 0).sum())
    faces = int(nbr.size)
    per_face = (N + 1) ** 2
    return ((faces - walls) * per_face * (FLOP_PER_PAIR + FLOP_PER_NODE)
            + walls * per_face * (FLOP_PER_PAIR + FLOP_PER_MIRROR))


def face_partner_bytes(N: int, nbr, dtype: str) -> int:
    """Bytes of the face partners' states the fused kernel reads (6 values per
    face node with a neighbour)."""
    import numpy as np

    size = 8 if dtype == "f64" else 4
    return int((np.asarray(nbr) >= 0).sum()) * (N + 1) ** 2 * 6 * size


def algorithmic_bytes_rhs(N: int, nelem: int, dtype: str) -> int:
    return algorithmic_bytes(N, nelem, dtype) + 24 * nelem
