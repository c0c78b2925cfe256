"""The public headers are plain C: gcc compiles a caller, links libred.so, and
the argument checks answer from C (no call reaches a kernel)."""
import os
import subprocess

import pytest

import reduction_libred_amd as rl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_SOURCE = r"""
#include <stdio.h>
#include "libred.h"
#include "libred_ablate.h"
#include "libred_probe.h"

int main(void) {
    float *x = (float *)0x10000, *out = (float *)0x20000;
    int fails = 0;
    fails += red_sum_f32(NULL, 4, out, 0) != RED_ERR_INVALID_ARG;
    fails += red_max_f32(x, 4, NULL, 0) != RED_ERR_INVALID_ARG;
    fails += red_sum_i32_i64((const int32_t *)x, 4, (int64_t *)(out + 1), 0) != RED_ERR_INVALID_ARG;
    fails += red_rows_sum_f32(x, (size_t)1 << 40, (size_t)1 << 40, out, 0) != RED_ERR_INVALID_ARG;
    fails += red_rows_max_f32(NULL, 0, 5, NULL, 0) != RED_OK;
    fails += red_ablate_num_partials(1, 1000) != 4;
    red_flat_policy p;
    red_default_flat_policy((size_t)1 << 28, &p);
    fails += p.layout != 1;
    fails += red_status_string(RED_ERR_HIP) == NULL;
    printf("%s %d\n", red_version(), fails);
    return fails;
}
"""


def test_headers_compile_as_c_and_link(tmp_path):
    src = tmp_path / "caller.c"
    src.write_text(C_SOURCE)
    exe = tmp_path / "caller"
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    libdir = os.path.dirname(rl.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(rocm, 'include')}",
           str(src), "-o", str(exe), f"-L{libdir}", "-l:libred.so", f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "hip_runtime_api.h" in r.stderr:
        pytest.skip("HIP headers not found")
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.startswith("libred")
