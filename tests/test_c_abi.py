"""The boundary is a C ABI: a plain C99 program includes include/*.h, links
the three libraries and calls host-side entry points (status strings, order
range, synchronous argument errors, variant names) -- no GPU needed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "entropy_stable_dg_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "esdg.h"
#include "esdg_ablation.h"
#include "esdg_probe.h"

int main(void)
{
    int fails = 0;
    if (esdg_min_order() != 1 || esdg_max_order() != 8) fails++;
    if (strcmp(esdg_status_string(ESDG_OK), "ok") != 0) fails++;
    /* argument errors come back before any HIP call: fake pointers are never read */
    const double *p = (const double *)0x10000;
    double *r = (double *)0x90000;
    if (esdg_volume_rhs_f64(p, p, p, p, 0, 1, r, 0) != ESDG_ERR_ORDER) fails++;
    if (esdg_volume_rhs_f32((const float *)p, (const float *)p, (const float *)p,
                            (const float *)p, 4, -1, (float *)r, 0) != ESDG_ERR_NELEM) fails++;
    if (esdg_rhs_f64(p, p, p, p, (const int32_t *)0, (const double *)0, 4, 10, r, 0)
        != ESDG_ERR_NULL) fails++;
    if (esdg_volume_rhs_f64(0, 0, 0, 0, 4, 0, 0, 0) != ESDG_OK) fails++;
    if (esdg_ablation_volume_rhs_f64(ESDG_ABL_COUNT, p, p, p, p, 4, 1, r, 0) != ESDG_ERR_VARIANT) fails++;
    if (strcmp(esdg_ablation_name(ESDG_ABL_BASELINE), "baseline") != 0) fails++;
    if (esdg_probe_copy_f64(p, r, -1, 0) != -3) fails++;
    /* the timeline's workgroup count follows the launch table: 3 elements per
       workgroup at N = 4, one at N = 7 */
    if (esdg_probe_timeline_workgroups(4, 4096, 1) != 1366) fails++;
    if (esdg_probe_timeline_workgroups(4, 4096, 0) != 1366) fails++;
    if (esdg_probe_timeline_workgroups(7, 13824, 1) != 13824) fails++;
    if (esdg_probe_timeline_workgroups(9, 10, 1) != -3) fails++;
    if (esdg_probe_timeline_workgroups(4, (int64_t)0x7fffffffffffffffLL, 1) != -3) fails++;
    if (esdg_probe_timeline_f64(p, p, p, p, 0, 9, 1, r, (uint64_t *)r, 0) != -3) fails++;
    if (esdg_probe_timeline_f64(p, p, p, p, 0, 4, 1, r, (uint64_t *)0, 0) != -1) fails++;
    if (esdg_probe_timeline_f32(0, 0, 0, 0, 0, 4, 0, 0, 0, 0) != 0) fails++;
    printf("fails=%d\n", fails);
    return fails;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_plain_c_program_links_and_calls_the_libraries(tmp_path):
    for lib in ("libesdg.so", "libesdg_ablation.so", "libesdg_probe.so"):
        if not os.path.exists(os.path.join(LIBDIR, lib)):
            pytest.skip(f"{lib} not built")
    src = tmp_path / "t.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "t"
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror=implicit-function-declaration",
           "-D__HIP_PLATFORM_AMD__", f"-I{os.path.join(ROOT, 'include')}", f"-I{ROCM}/include",
           str(src), "-o", str(exe), f"-L{LIBDIR}", "-l:libesdg.so", "-l:libesdg_ablation.so",
           "-l:libesdg_probe.so", f"-Wl,-rpath,{LIBDIR}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "fails=0" in run.stdout
