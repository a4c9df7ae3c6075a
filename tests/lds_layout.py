"""Host-side model of the kernel's launch shapes and LDS layout, for checking
a launch table on the CPU before it runs on a GPU.

It reads the `Launch<T, N>` table of csrc/launch_table.hpp and derives, for each
shape, what the kernel derives from its `LaunchCfg`: the LDS slot of every
node of a workgroup (node grid x + R y + P z + E e with the row, plane and
element pads), the line task of every thread (element-major, direction-major,
or direction-major with each direction on a 32-lane boundary) and the slot
of each node of a line (first slot + a * stride).  `bank_cost` is the bank
model used to choose the pads: for one LDS read in which every active lane
reads one value of its own line, the cycles of a wave when the LDS has
`banks` 4-byte banks and serves banks / words lanes at a time, a group's
cycles being the number of distinct addresses on its most-loaded bank.

Nothing here runs on the GPU or is used by the library at run time.
"""
from __future__ import annotations

import os
import re
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
API_SOURCE = os.path.join(os.path.dirname(HERE), "entropy_stable_dg_amd", "csrc", "launch_table.hpp")

# LaunchCfg<EPB, NT, WAVES, METRIC_LDS, CACHE, KMAJOR, FIN, SERIES, SERIES_SURF,
#           ROW_PAD, PLANE_PAD, ELEM_PAD, WAVES_SURF, LANES, DISTINCT, SLOTS64> and its defaults
FIELDS = ("epb", "nt", "waves", "metric_lds", "cache", "kmajor", "fin", "series", "series_surf",
          "row_pad", "plane_pad", "elem_pad", "waves_surf", "lanes", "distinct", "slots64")
DEFAULTS = (None, None, 0, 1, 0, 0, 0, 0, 0, 0, 0, 0, 0, 1, 0, 0)

# staged values per node (without / with the metric) and partial sums per node
STAGED_NO_METRIC, STAGED_WITH_METRIC = 10, 19
PARTIALS, PARTIALS_FIN = 15, 10


def _value(tok: str) -> int:
    tok = tok.strip()
    return {"true": 1, "false": 0}[tok] if tok in ("true", "false") else int(tok)


def parse_launch_table(path: str = API_SOURCE) -> dict:
    """{("double"|"float", N): {field: value}} from the Launch<> specialisations."""
    text = open(path).read()
    pat = re.compile(r"struct Launch<(double|float),\s*(\d+)>\s*\{\s*using C = LaunchCfg<([^>]*)>;")
    table = {}
    for dtype, n, args in pat.findall(text):
        vals = [_value(a) for a in args.split(",")]
        if len(vals) < 2 or len(vals) > len(FIELDS):
            raise ValueError(f"LaunchCfg of {dtype} N={n}: {len(vals)} arguments")
        full = list(vals) + list(DEFAULTS[len(vals):])
        table[(dtype, int(n))] = dict(zip(FIELDS, full))
    return table


@dataclass
class Shape:
    N: int
    cfg: dict
    dtype: str = "double"
    split: bool = False   # the fp32 perturbation kernels stage b (p - P) too

    def __post_init__(self):
        c = self.cfg
        self.Nq = self.N + 1
        self.Nq2 = self.Nq * self.Nq
        self.Np = self.Nq2 * self.Nq
        self.EPB, self.NT = c["epb"], c["nt"]
        self.R = self.Nq + c["row_pad"]
        self.P = self.Nq * self.R + c["plane_pad"]
        self.E = self.Nq * self.P + c["elem_pad"]
        self.slots = self.EPB * self.E
        if c.get("slots64"):   # value arrays 64 slots apart
            self.slots = (self.slots + 63) // 64 * 64
        self.lines = 3 * self.EPB * self.Nq2
        lines_per_dir = self.EPB * self.Nq2
        self.dir_stride = (lines_per_dir + 31) // 32 * 32 if c["kmajor"] == 2 else lines_per_dir
        self.lanes = c.get("lanes", 1)
        self.task_threads = self.lanes * (3 * self.dir_stride if c["kmajor"] else self.lines)
        staged = STAGED_WITH_METRIC if c["metric_lds"] else STAGED_NO_METRIC
        partials = PARTIALS_FIN if c["fin"] else PARTIALS
        self.region = max(staged, partials) + (1 if c["fin"] else 0)
        # the extra value sits in the shared region when the partials leave it free
        self.values = self.region + (1 if self.split and staged >= partials else 0)
        self.lds_bytes = self.values * self.slots * (8 if self.dtype == "double" else 4)

    def slot(self, t: int) -> int:
        """LDS slot of node t of the workgroup (t = e Np + x + Nq y + Nq^2 z)."""
        e, r = divmod(t, self.Np)
        z, r2 = divmod(r, self.Nq2)
        y, x = divmod(r2, self.Nq)
        return e * self.E + z * self.P + y * self.R + x

    def half(self, thread: int) -> int:
        """Which half of its line a thread owns (0 with one lane per line)."""
        return thread % self.lanes

    def task(self, thread: int):
        """(e, k, line) of a thread's line task, as the kernel derives it."""
        Nq2, EPB = self.Nq2, self.EPB
        thread //= self.lanes
        if self.cfg["kmajor"]:
            k, r = divmod(thread, self.dir_stride)
            e, line = divmod(r, Nq2)
            if k > 2:
                k, e = 2, EPB
        else:
            e, r3 = divmod(thread, 3 * Nq2)
            k, line = divmod(r3, Nq2)
        return e, k, line

    def active(self, thread: int, nvalid_elements: int) -> bool:
        e, _, _ = self.task(thread)
        return thread < self.task_threads and e * self.Np < nvalid_elements * self.Np

    def line_nodes(self, e: int, k: int, line: int):
        """Node numbers (within the workgroup) and LDS slots of the line's nodes."""
        Nq, Nq2 = self.Nq, self.Nq2
        p1, p2 = line % Nq, line // Nq
        n0 = (Nq * (p1 + Nq * p2), p1 + Nq2 * p2, p1 + Nq * p2)[k]
        nstep = (1, Nq, Nq2)[k]
        s0 = (self.R * p1 + self.P * p2, p1 + self.P * p2, p1 + self.R * p2)[k]
        sstep = (1, self.R, self.P)[k]
        nodes = [e * self.Np + n0 + a * nstep for a in range(Nq)]
        slots = [e * self.E + s0 + a * sstep for a in range(Nq)]
        return nodes, slots


def bank_cost(shape: Shape, words: int, banks: int) -> tuple:
    """(cycles, conflict-free cycles) of one pair-loop read over a workgroup's
    waves (the same for every node a of the lines)."""
    group = banks // words
    total = ideal = 0
    for w0 in range(0, shape.NT, 64):
        for g0 in range(w0, w0 + 64, group):
            per_bank = {}
            n = 0
            for thread in range(g0, g0 + group):
                if thread >= shape.NT or not shape.active(thread, shape.EPB):
                    continue
                n += 1
                slots = shape.line_nodes(*shape.task(thread))[1]
                s = slots[-1] if shape.half(thread) else slots[0]
                for d in range(words * s, words * s + words):
                    per_bank.setdefault(d % banks, set()).add(d)
            if n:
                total += max(len(v) for v in per_bank.values())
                ideal += 1
    return total, ideal
