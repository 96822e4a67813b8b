"""Build the HIP library liboptim_step.so for gfx950 (in-tree).

Flags: -O3; -ffp-contract=off so every multiply and add in the kernels rounds
as written; IEEE fp32 division and sqrt; fp32 denormals kept; packed-fp32
instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_DIR = os.path.join(HERE, "lib")
LIB_PATH = os.path.join(LIB_DIR, "liboptim_step.so")
SOURCES = [os.path.join(CSRC, f) for f in ("kernels_adam.hip", "kernels_mini.hip", "kernels_blockwise.hip",
                                           "kernels_util.hip", "kernels_lion_lamb.hip", "kernels_scaled.hip", "api.cpp")]
ARCH = os.environ.get("OPTIM_STEP_ARCH", "gfx950")


def hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


def _flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
            "-fno-gpu-flush-denormals-to-zero",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(verbose: bool = False) -> str:
    """Compiles every source to an object (in parallel), then links the
    shared library; always recompiles."""
    from concurrent.futures import ThreadPoolExecutor
    obj_dir = os.path.join(LIB_DIR, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    objs = [os.path.join(obj_dir, os.path.basename(src) + ".o") for src in SOURCES]
    cmds = [[hipcc()] + _flags() + ["-c", src, "-o", obj] for src, obj in zip(SOURCES, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    jobs = max(1, min(len(cmds), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(jobs) as ex:
        for c, rc in zip(cmds, ex.map(lambda c: subprocess.call(c), cmds)):
            if rc != 0:
                raise subprocess.CalledProcessError(rc, c)
    tmp = LIB_PATH + ".tmp"
    link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.check_call(link)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
