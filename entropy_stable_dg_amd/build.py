"""Build libesdg.so, libesdg_probe.so and libesdg_ablation.so (HIP, gfx950)
in-tree with hipcc.

    python -m entropy_stable_dg_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libesdg.so")
SOURCES = [os.path.join(CSRC, "esdg_api.hip")]
DEPENDS = SOURCES + [os.path.join(CSRC, "volume_kernel.hpp"), os.path.join(CSRC, "launch_table.hpp"),
                     os.path.join(INCLUDE, "esdg.h")]
# HBM streaming probes (measurement only), a library of their own
PROBE_LIB = os.path.join(HERE, "libesdg_probe.so")
PROBE_SOURCES = [os.path.join(CSRC, "stream_probe.hip")]
# the optimisation-ladder variants of the volume term (measurement only)
ABLATION_LIB = os.path.join(HERE, "libesdg_ablation.so")
ABLATION_SOURCES = [os.path.join(CSRC, "ablation.hip")]
ABLATION_DEPENDS = ABLATION_SOURCES + [os.path.join(CSRC, "volume_kernel.hpp"),
                                       os.path.join(INCLUDE, "esdg_ablation.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    # no packed-fp32 instructions (v_pk_*_f32) anywhere in the library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _compile(sources, out, verbose):
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I" + INCLUDE, "-I" + CSRC, "-o", tmp] + sources
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile the HIP sources: libesdg.so (the volume term),
    libesdg_probe.so (HBM streaming probes) and libesdg_ablation.so (the
    optimisation-ladder variants)."""
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    _compile(ABLATION_SOURCES, ABLATION_LIB, verbose)
    return _compile(SOURCES, LIB, verbose)


def is_stale() -> bool:
    """True when the library is missing or older than one of its sources."""
    probe_deps = PROBE_SOURCES + [os.path.join(CSRC, "volume_kernel.hpp"),
                                  os.path.join(CSRC, "launch_table.hpp"),
                                  os.path.join(INCLUDE, "esdg_probe.h")]
    for lib, deps in ((LIB, DEPENDS), (PROBE_LIB, probe_deps), (ABLATION_LIB, ABLATION_DEPENDS)):
        if not os.path.exists(lib):
            return True
        t = os.path.getmtime(lib)
        if any(os.path.getmtime(p) > t for p in deps):
            return True
    return False


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
