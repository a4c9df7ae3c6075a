"""Work and traffic model of the volume term, and MI355X peak figures.

Algorithmic traffic per node (DOF): the kernel must read 5 conserved fields,
the geopotential and 10 geometry values (9 metric terms and J) and write 5
fields: 21 values = 168 B in fp64, 84 B in fp32.  The differentiation matrix
(N+1)^2 values per launch is added once.

FLOP counting convention (the method's work, not the ordered-pair work the
symmetric evaluation avoids): +, -, x, reciprocal and log = 1 FLOP, fused
multiply-add = 2; comparisons, selects and negations = 0; the log means are
counted on their series branch (the branch smooth flows take); quantities
hoisted per node are counted once per node.  The tallies below follow the
kernel's pair and node arithmetic step by step (pair_update and node_values
of csrc/volume_kernel.hpp, series form):

  per unordered pair on a line ........ 95   (PAIR_STEPS)
  per node ............................ 44   (NODE_STEPS)

Unordered pairs per element: 3 (N+1)^2 (N+1) N / 2.

Whole right-hand side (volume + entropy-conservative surface term, one fused
kernel): the algorithmic traffic adds only the connectivity, 6 int32 per
element; the kernel also re-reads each face partner's 5 fields and phi from
the neighbouring element (48 B per face node in fp64 with a neighbour, none at
a slip wall), which the cache may or may not serve.  Work per face node: one
pair plus the partner's per-node values (its primitives, p, b, 2 logs, 1/b,
w: NODE_STEPS without the -1/J and the directional sum) with a neighbour; one
pair and the mirror state at a slip wall.
"""
from __future__ import annotations

# (step, {operation: count}) with operation in add (also sub), mul, fma, rcp, log
PAIR_STEPS = (
    ("sums and jumps of rho and b", {"add": 4}),
    ("one reciprocal for 1/(rho_a+rho_l) and 1/(b_a+b_l)", {"mul": 1, "rcp": 1}),
    ("1/(rho_a+rho_l), 1/(b_a+b_l)", {"mul": 2}),
    ("log mean of rho: s, s^2, cubic series in s^2, scale", {"mul": 3, "fma": 3}),
    ("inverse log mean of b: s, s^2, cubic series in s^2, scale", {"mul": 3, "fma": 3}),
    ("{{rho}}/(2{{b}}): density sum over the staged-2b sum", {"mul": 1}),
    ("pair metric Ja^k(a) + Ja^k(l)", {"add": 3}),
    ("2{{u}}", {"add": 3}),
    ("contravariant density flux", {"mul": 2, "fma": 2}),
    ("symmetric momentum flux", {"mul": 3, "fma": 3}),
    ("energy-flux coefficient", {"add": 1, "fma": 1}),
    ("energy flux", {"mul": 1, "fma": 3}),
    ("gravity term g", {"add": 1, "mul": 2}),
    ("gravity for each node: g/b_a, -g/b_l", {"mul": 2}),
    ("density and energy contributions to both nodes", {"fma": 4}),
    ("momentum contributions with gravity to both nodes", {"fma": 12}),
)
NODE_STEPS = (
    ("1/rho, 1/(2 rho)", {"rcp": 1, "mul": 1}),
    ("u/2", {"mul": 3}),
    ("|u|^2/4", {"mul": 1, "fma": 2}),
    ("E - U.u/2... - rho phi", {"mul": 1, "fma": 3, "add": 1}),
    ("p", {"mul": 1}),
    ("staged 2b = rho/p", {"rcp": 1, "mul": 1}),
    ("1/(2b) = p/rho", {"mul": 1}),
    ("ln rho, ln b (the log of 2^16 x 2b)", {"log": 2, "mul": 1}),
    ("phi/4", {"mul": 1}),
    ("w/2 = (phi - |u|^2/2)/2", {"fma": 1}),
    ("-1/J", {"rcp": 1}),
    ("sum of the three directional partials", {"add": 10}),
    ("scale by -1/J", {"mul": 5}),
)
WEIGHT = {"add": 1, "mul": 1, "fma": 2, "rcp": 1, "log": 1}


def tally(steps) -> int:
    return sum(WEIGHT[op] * n for _, ops in steps for op, n in ops.items())


FLOP_PER_PAIR = tally(PAIR_STEPS)
FLOP_PER_NODE = tally(NODE_STEPS)
# a face partner's node values: NODE_STEPS without -1/J, the directional sum and the scaling
FLOP_PER_PARTNER_NODE = FLOP_PER_NODE - tally(NODE_STEPS[-3:])

# MI355X (gfx950) published peaks
PEAK_HBM_GBS = 8000.0          # HBM3E, GB/s
PEAK_FP64_VECTOR_TFLOPS = 78.6
PEAK_FP32_VECTOR_TFLOPS = 157.3
CU_COUNT = 256
CLOCK_GHZ = 2.4
# VALU issue: 256 CUs x 4 SIMDs, 2.4 GHz; a wave64 fp64 or (unpacked) fp32
# VALU instruction occupies its SIMD for 4 cycles (16 lanes per cycle), which
# is where the vector peaks come from (78.6 TF/s = 1024 x 16 x 2 x 2.4 GHz)
SIMDS = 4 * CU_COUNT
CYCLES_PER_WAVE_VALU = 4


def phase_floors(bytes_per_launch: float, valu_wave_instructions: float, stream_gbs: float,
                 measured_us: float) -> dict:
    """Two lower bounds on a launch: moving its algorithmic bytes at the
    measured stream bandwidth, and issuing its counted VALU wave-instructions
    on every SIMD back to back (4 cycles each, transcendentals counted as one
    issue).  A kernel whose load and compute phases overlap perfectly runs
    near the larger; one whose phases serialise, near their sum."""
    hbm = bytes_per_launch / (stream_gbs * 1e9) * 1e6
    valu = valu_wave_instructions * CYCLES_PER_WAVE_VALU / (SIMDS * CLOCK_GHZ * 1e9) * 1e6
    return {"hbm_us": hbm, "valu_us": valu, "max_us": max(hbm, valu), "sum_us": hbm + valu,
            "measured_us": measured_us, "measured_over_sum": measured_us / (hbm + valu),
            "measured_over_max": measured_us / max(hbm, valu)}


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
    return ((faces - walls) * per_face * (FLOP_PER_PAIR + FLOP_PER_PARTNER_NODE)
            + walls * per_face * (FLOP_PER_PAIR + FLOP_PER_MIRROR))


def face_partner_bytes(N: int, nbr, dtype: str) -> int:
    """Bytes of the face partners' states the fused kernel reads (6 values per
    face node with a neighbour)."""
    import numpy as np

    size = 8 if dtype == "f64" else 4
    return int((np.asarray(nbr) >= 0).sum()) * (N + 1) ** 2 * 6 * size


def algorithmic_bytes_rhs(N: int, nelem: int, dtype: str) -> int:
    return algorithmic_bytes(N, nelem, dtype) + 24 * nelem


def algorithmic_bytes_stage(N: int, nelem: int, dtype: str) -> float:
    """Bytes of one fused Runge-Kutta stage, averaged over the five stages of
    a step: the whole right-hand side's inputs (16 values per node and the
    connectivity), the register dq read (by four of the five stages: the
    first does not read it) and written, and the next state written: 16 +
    4/5 x 5 + 10 = 30 values per node."""
    size = 8 if dtype == "f64" else 4
    return nelem * (N + 1) ** 3 * 30 * size + (N + 1) ** 2 * size + 24 * nelem
