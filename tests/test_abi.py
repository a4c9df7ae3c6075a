"""The C-ABI library loads on a machine without a GPU, exports every function
include/esdg.h declares, and rejects bad arguments synchronously, before any
HIP call (nothing here launches a kernel)."""
import ctypes
import os
import re

import pytest

from entropy_stable_dg_amd import esdg, probe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "esdg.h")
PROBE_HEADER = os.path.join(ROOT, "include", "esdg_probe.h")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(esdg_\w+)\s*\(", text)))


def test_probe_library_exports_its_header():
    assert declared_functions(PROBE_HEADER) == sorted(probe.EXPORTS)
    lib = probe.load()
    out = os.popen(f"nm -D --defined-only {probe.PROBE_LIB_PATH}").read()
    syms = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for name in probe.EXPORTS:
        assert hasattr(lib, name) and name in syms


def test_probe_argument_errors():
    # validation before any HIP call: no launch happens here
    for fn in (probe.esdg_probe_stream81_f64, probe.esdg_probe_stream81_wide_f64,
               probe.esdg_probe_copy_f64):
        assert fn(0x1000, 0x2000, -1, 0) == -3
        assert fn(0, 0x2000, 10, 0) == -1
        assert fn(0x1000, 0, 10, 0) == -1
        assert fn(0, 0, 0, 0) == 0
    # the wide form needs 16-byte alignment and an even length
    assert probe.esdg_probe_stream81_wide_f64(0x1008, 0x2000, 10, 0) == -2
    assert probe.esdg_probe_stream81_wide_f64(0x1000, 0x2008, 10, 0) == -2
    assert probe.esdg_probe_stream81_wide_f64(0x1000, 0x2000, 11, 0) == -2


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(esdg.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = esdg.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_exported_symbols_are_c_linkage():
    out = os.popen(f"nm -D --defined-only {esdg.LIB_PATH}").read()
    syms = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for name in declared_functions():
        assert name in syms, name


def test_order_range_and_status_strings():
    assert esdg.esdg_min_order() == 1
    assert esdg.esdg_max_order() == 8
    for st in (esdg.ESDG_OK, esdg.ESDG_ERR_NULL, esdg.ESDG_ERR_ORDER, esdg.ESDG_ERR_NELEM,
               esdg.ESDG_ERR_LAUNCH, esdg.ESDG_ERR_ALIAS, esdg.ESDG_ERR_DEVICE):
        s = esdg.esdg_status_string(st)
        assert s and s != "unknown status"
    assert esdg.esdg_status_string(12345) == "unknown status"


# Fake, never-dereferenced addresses: every call below fails validation (or is
# the nelem == 0 no-op) before the library touches the HIP runtime.
A, B, C, Dp, R = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


@pytest.mark.parametrize("fn", [esdg.esdg_volume_rhs_f64, esdg.esdg_volume_rhs_f32])
def test_argument_errors(fn):
    assert fn(A, B, C, Dp, 0, 1, R, 0) == esdg.ESDG_ERR_ORDER
    assert fn(A, B, C, Dp, 9, 1, R, 0) == esdg.ESDG_ERR_ORDER
    assert fn(A, B, C, Dp, -1, 1, R, 0) == esdg.ESDG_ERR_ORDER
    assert fn(A, B, C, Dp, 4, -1, R, 0) == esdg.ESDG_ERR_NELEM
    assert fn(A, B, C, Dp, 4, 2 ** 62, R, 0) == esdg.ESDG_ERR_NELEM
    # nelem == 0: OK without reading any pointer
    assert fn(0, 0, 0, 0, 4, 0, 0, 0) == esdg.ESDG_OK
    for i in range(5):
        args = [A, B, C, Dp, R]
        args[i] = 0
        assert fn(args[0], args[1], args[2], args[3], 4, 10, args[4], 0) == esdg.ESDG_ERR_NULL
    # the order check comes first, then nelem, then pointers
    assert fn(0, 0, 0, 0, 0, -1, 0, 0) == esdg.ESDG_ERR_ORDER
    assert fn(0, 0, 0, 0, 3, -1, 0, 0) == esdg.ESDG_ERR_NELEM


@pytest.mark.parametrize("fn", [esdg.esdg_volume_rhs_f64, esdg.esdg_volume_rhs_f32])
def test_grid_limit(fn):
    # more workgroups than a launch grid holds (2^31 - 1 at 16 elements per
    # workgroup for N = 1): refused before any HIP call; the fake arrays lie
    # 2^45 bytes apart so that they do not overlap
    big = 16 * 2 ** 31 + 16
    far = [(i + 1) << 45 for i in range(5)]
    assert fn(far[0], far[1], far[2], far[3], 1, big, far[4], 0) == esdg.ESDG_ERR_NELEM
    assert esdg.esdg_rhs_f64(far[0], far[1], far[2], far[3], 1 << 40, None, 1, big, far[4],
                             0) == esdg.ESDG_ERR_NELEM


@pytest.mark.parametrize("fn,size", [(esdg.esdg_volume_rhs_f64, 8), (esdg.esdg_volume_rhs_f32, 4)])
def test_alias_errors(fn, size):
    N, nelem = 3, 100
    field = nelem * 64 * size
    # rhs overlapping the last field of q, phi, the geometry, or D
    assert fn(A, B, C, Dp, N, nelem, A + 4 * field, 0) == esdg.ESDG_ERR_ALIAS
    assert fn(A, B, C, Dp, N, nelem, B - 5 * field + size, 0) == esdg.ESDG_ERR_ALIAS
    assert fn(A, B, C, Dp, N, nelem, C + 9 * field, 0) == esdg.ESDG_ERR_ALIAS
    assert fn(A, B, C, Dp, N, nelem, Dp + 8, 0) == esdg.ESDG_ERR_ALIAS


@pytest.mark.parametrize("fn,size", [(esdg.esdg_rhs_f64, 8), (esdg.esdg_rhs_f32, 4)])
def test_rhs_argument_errors(fn, size):
    NB = 0x60000000
    om = (0.0, 0.0, 1e-4)
    for w in (None, om):   # omega is optional (host values), checked after the pointers
        assert fn(A, B, C, Dp, NB, w, 0, 1, R, 0) == esdg.ESDG_ERR_ORDER
        assert fn(A, B, C, Dp, NB, w, 4, -1, R, 0) == esdg.ESDG_ERR_NELEM
        assert fn(0, 0, 0, 0, 0, w, 4, 0, 0, 0) == esdg.ESDG_OK
        for i in range(6):
            args = [A, B, C, Dp, NB, R]
            args[i] = 0
            assert fn(args[0], args[1], args[2], args[3], args[4], w, 4, 10, args[5], 0) == esdg.ESDG_ERR_NULL
    # rhs overlapping the connectivity array
    N, nelem = 3, 100
    assert fn(A, B, C, Dp, NB, None, N, nelem, NB + 6 * nelem * 4 - size, 0) == esdg.ESDG_ERR_ALIAS
    assert fn(A, B, C, Dp, NB, om, N, nelem, NB - 5 * nelem * 64 * size + size, 0) == esdg.ESDG_ERR_ALIAS
    # and the inputs, as for the volume term
    assert fn(A, B, C, Dp, NB, None, N, nelem, A + 4 * nelem * 64 * size, 0) == esdg.ESDG_ERR_ALIAS
    with pytest.raises(ValueError):
        fn(A, B, C, Dp, NB, (1.0, 2.0), N, nelem, R, 0)


def test_tensor_wrapper_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(5, 1, 8, dtype=torch.float64)
    phi = torch.zeros(1, 8, dtype=torch.float64)
    geom = torch.zeros(10, 1, 8, dtype=torch.float64)
    D = torch.zeros(2, 2, dtype=torch.float64)
    with pytest.raises(ValueError, match="GPU"):
        esdg.volume_rhs(q, phi, geom, D)
    with pytest.raises(TypeError):
        esdg.volume_rhs(q.float(), phi, geom, D)
    nbr = torch.zeros(1, 6, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        esdg.rhs(q, phi, geom, D, nbr)
    with pytest.raises(TypeError):
        esdg.rhs(q, phi, geom, D, nbr.long())


def test_missing_library_fails_loudly(tmp_path):
    """No CPU fallback: a binding pointed at a library that is not there raises."""
    from entropy_stable_dg_amd import ablation
    for mod in (esdg, probe, ablation):
        with pytest.raises(RuntimeError, match="missing"):
            mod.load(str(tmp_path / "not_built.so"))


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
