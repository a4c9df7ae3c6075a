"""The library used from plain C on the GPU: a C99 program (HIP runtime C API,
no C++ and no Python at call time) allocates device memory, copies a
workload in, calls esdg_volume_rhs_f64 / esdg_rhs_f64 on its own stream and
copies the result back; the result is held to the oracle (volume term of
the page "GPU Performance of an Entropy-Stable DG Euler Solver with
Non-Conservative Terms", section 3, Eq. 2) at the parity tolerance."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from entropy_stable_dg_amd import inputs as I

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "entropy_stable_dg_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

PROGRAM = r"""
#include <stdio.h>
#include <stdlib.h>
#include <hip/hip_runtime_api.h>
#include "esdg.h"

/* input file: int32 N, int32 whole, int64 nelem, then q, phi, geom, D (double)
   and, when whole != 0, nbr (int32); output file: rhs (double) */
static void *slurp(FILE *f, size_t bytes)
{
    void *p = malloc(bytes);
    if (!p || fread(p, 1, bytes, f) != bytes) { fprintf(stderr, "short read\n"); exit(2); }
    return p;
}

#define CHECK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
    fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); return 3; } } while (0)

int main(int argc, char **argv)
{
    if (argc != 3) return 1;
    FILE *f = fopen(argv[1], "rb");
    if (!f) return 1;
    int N, whole;
    long long nelem;
    if (fread(&N, 4, 1, f) != 1 || fread(&whole, 4, 1, f) != 1 || fread(&nelem, 8, 1, f) != 1) return 2;
    const size_t np = (size_t)(N + 1) * (N + 1) * (N + 1), n = (size_t)nelem * np;
    const size_t bq = 5 * n * 8, bphi = n * 8, bgeom = 10 * n * 8, bD = (size_t)(N + 1) * (N + 1) * 8;
    const size_t bnbr = (size_t)nelem * 6 * 4;
    void *hq = slurp(f, bq), *hphi = slurp(f, bphi), *hgeom = slurp(f, bgeom), *hD = slurp(f, bD);
    void *hnbr = whole ? slurp(f, bnbr) : NULL;
    fclose(f);
    double *q, *phi, *geom, *D, *rhs;
    int32_t *nbr = NULL;
    hipStream_t s;
    CHECK(hipMalloc((void **)&q, bq)); CHECK(hipMalloc((void **)&phi, bphi));
    CHECK(hipMalloc((void **)&geom, bgeom)); CHECK(hipMalloc((void **)&D, bD));
    CHECK(hipMalloc((void **)&rhs, bq));
    CHECK(hipMemcpy(q, hq, bq, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(phi, hphi, bphi, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(geom, hgeom, bgeom, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(D, hD, bD, hipMemcpyHostToDevice));
    if (whole) {
        CHECK(hipMalloc((void **)&nbr, bnbr));
        CHECK(hipMemcpy(nbr, hnbr, bnbr, hipMemcpyHostToDevice));
    }
    CHECK(hipStreamCreate(&s));
    int st = whole ? esdg_rhs_f64(q, phi, geom, D, nbr, NULL, N, nelem, rhs, s)
                   : esdg_volume_rhs_f64(q, phi, geom, D, N, nelem, rhs, s);
    if (st != ESDG_OK) { fprintf(stderr, "esdg: %s\n", esdg_status_string(st)); return 4; }
    CHECK(hipStreamSynchronize(s));
    void *hr = malloc(bq);
    if (!hr) return 5;
    CHECK(hipMemcpy(hr, rhs, bq, hipMemcpyDeviceToHost));
    FILE *o = fopen(argv[2], "wb");
    if (!o || fwrite(hr, 1, bq, o) != bq) return 6;
    fclose(o);
    CHECK(hipStreamDestroy(s));
    CHECK(hipFree(q)); CHECK(hipFree(phi)); CHECK(hipFree(geom)); CHECK(hipFree(D)); CHECK(hipFree(rhs));
    if (nbr) CHECK(hipFree(nbr));
    printf("ok\n");
    return 0;
}
"""


@pytest.fixture(scope="module")
def program(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    if not os.path.exists(os.path.join(LIBDIR, "libesdg.so")):
        pytest.skip("libesdg.so not built")
    d = tmp_path_factory.mktemp("cprog")
    src, exe = d / "run.c", d / "run"
    src.write_text(PROGRAM)
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{ROCM}/include", str(src), "-o", str(exe),
           f"-L{LIBDIR}", "-l:libesdg.so", f"-L{ROCM}/lib", "-lamdhip64",
           f"-Wl,-rpath,{LIBDIR}", f"-Wl,-rpath,{ROCM}/lib"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


@pytest.mark.parametrize("name,whole", [("tiny", False), ("bubble", False), ("tiny", True),
                                        ("bubble", True)])
def test_c_program_on_gpu(program, tmp_path, name, whole):
    wl = I.make(name)
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        np.array([wl.N, int(whole)], dtype=np.int32).tofile(f)
        np.array([wl.nelem], dtype=np.int64).tofile(f)
        for a in (wl.q, wl.phi, wl.geom, wl.D):
            np.ascontiguousarray(a, dtype=np.float64).tofile(f)
        if whole:
            np.ascontiguousarray(wl.nbr, dtype=np.int32).tofile(f)
    print(f"[c-program] {name} {'whole rhs' if whole else 'volume term'} N={wl.N} nelem={wl.nelem}",
          flush=True)
    run = subprocess.run([str(program), str(inp), str(out)], capture_output=True, text=True,
                         timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    got = np.fromfile(out, dtype=np.float64).reshape(wl.q.shape)
    if whole:
        ref, mag = oracle.rhs(wl.q, wl.phi, wl.geom, wl.D, wl.nbr, wl.N, with_magnitude=True)
        scale = np.abs(mag).reshape(5, -1).max(axis=1)
    else:
        ref = oracle.volume_rhs(wl.q, wl.phi, wl.geom, wl.D, wl.N)
        scale = np.abs(ref).reshape(5, -1).max(axis=1)
    err = np.abs(got - ref).reshape(5, -1).max(axis=1) / scale
    print(f"[c-program] max error per field {['%.1e' % e for e in err]}", flush=True)
    assert np.all(np.isfinite(got)) and err.max() <= 1e-11
