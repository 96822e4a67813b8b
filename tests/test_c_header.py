"""The C ABI from C: a C99 program that includes include/optim_step.h (gcc,
-Wall -Wextra -Werror), links the in-tree library and calls the host-only
entry points (workspace sizing, validation errors, the codebook).  Its
struct sizes and results must agree with the Python binding's.  No device
is touched."""
import ctypes
import os
import shutil
import subprocess

import pytest

import optimizer_step_adamw_amd as osa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include "optim_step.h"
#include <stdio.h>
#include <string.h>

int main(void) {
    int64_t numel[2] = {5000, 77};
    /* non-overlapping fake device addresses: never dereferenced on the host */
    uintptr_t base = (uintptr_t)1 << 40;
    void *p[2], *g[2], *m[2], *v[2];
    for (int i = 0; i < 2; ++i) {
        p[i] = (void *)(base + (uintptr_t)(4 * i + 0) * (1u << 20));
        g[i] = (void *)(base + (uintptr_t)(4 * i + 1) * (1u << 20));
        m[i] = (void *)(base + (uintptr_t)(4 * i + 2) * (1u << 20));
        v[i] = (void *)(base + (uintptr_t)(4 * i + 3) * (1u << 20));
    }
    double wd[2] = {0.1, 0.0};
    optim_tensor_list tl;
    memset(&tl, 0, sizeof tl);
    tl.n = 2;
    tl.numel = numel;
    tl.param = p;
    tl.grad = (const void *const *)g;
    tl.m = m;
    tl.v = v;
    tl.weight_decay = wd;
    tl.param_dtype = OPTIM_F32;
    tl.grad_dtype = OPTIM_F32;
    size_t bytes = 0;
    int rc = optim_plan_workspace_size(&tl, OPTIM_ALGO_ADAMW, NULL, &bytes);
    printf("adamw %d %zu\n", rc, bytes);
    optim_plan_opts o;
    memset(&o, 0, sizeof o);
    o.state_layout = 7;
    rc = optim_plan_workspace_size(&tl, OPTIM_ALGO_ADAMW, &o, &bytes);
    printf("bad_layout %d %d\n", rc, (int)(strlen(optim_last_error()) > 0));
    float vals[256], thr[260];
    rc = optim_quant_codebook(8, 1, vals, thr);
    printf("codebook %d %.9g %.9g\n", rc, (double)vals[0], (double)vals[127]);
    printf("sizes %zu %zu %zu\n", sizeof(optim_tensor_list), sizeof(optim_plan_opts), sizeof(optim_adamw_hp));
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_header_compiles_as_c_and_matches_the_binding(tmp_path):
    lib = osa.LIB_PATH
    if not os.path.exists(lib):
        pytest.skip("library not built")
    src = tmp_path / "abi.c"
    exe = tmp_path / "abi"
    src.write_text(PROGRAM)
    libdir = os.path.dirname(lib)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
           "-o", str(exe), "-L", libdir, "-l:liboptim_step.so", f"-Wl,-rpath,{libdir}",
           "-Wl,-rpath-link,/opt/rocm/lib"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=120).stdout.split("\n")
    rows = {r.split()[0]: r.split()[1:] for r in out if r.strip()}
    # the same list through the Python binding
    p = [1 << 40, (1 << 40) + 4 * (1 << 20)]
    tl = osa.TensorList(p, [x + (1 << 20) for x in p], m=[x + 2 * (1 << 20) for x in p],
                        v=[x + 3 * (1 << 20) for x in p], weight_decay=[0.1, 0.0], numel=[5000, 77])
    assert rows["adamw"] == ["0", str(osa.optim_plan_workspace_size(tl, osa.OPTIM_ALGO_ADAMW, None))]
    assert rows["bad_layout"] == [str(osa.OPTIM_EINVAL), "1"]
    assert rows["codebook"][0] == "0"
    assert rows["sizes"] == [str(ctypes.sizeof(osa.optim_tensor_list)), str(ctypes.sizeof(osa.optim_plan_opts)),
                             str(ctypes.sizeof(osa.optim_adamw_hp))]
