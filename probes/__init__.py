"""Access-pattern ceiling probes for the benchmark (stream_probe.hip), and
device checks of the step library's numeric helpers for the test suite
(numerics_check.hip).

A separate library, not part of liboptim_step.so's C ABI.  Each probe
streams one step kernel's exact access pattern (arrays, lane layout, unit
size, access kind) with no arithmetic; bench.py reports each kernel's
bandwidth as a fraction of its pattern's measured ceiling.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "stream_probe.hip"), os.path.join(HERE, "numerics_check.hip")]
LIB_PATH = os.path.join(HERE, "libstream_probe.so")
ARCH = os.environ.get("OPTIM_STEP_ARCH", "gfx950")

_lib = None


def build(verbose: bool = False) -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = ["/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc",
           f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           # the step library's floating-point flags, for the numerics checks
           "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "optimizer_step_adamw_amd", "csrc"),
           "-Wall", "-Wno-unused-command-line-argument", "-o", tmp] + SRCS
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with probes.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        sigs = {
            "probe_adamw": [P, P, P, P, i64, i32, P],
            "probe_ademamix": [P, P, P, P, P, i64, i32, P],
            "probe_mini": [P, P, P, i64, P],
            "probe_bf16r": [P, P, P, P, P, i64, i32, P],
            "probe_blockwise": [P, P, P, P, P, P, i64, i32, i32, i32, P],
            "probe_read": [P, i64, i32, P, P],
            "probe_write": [P, i64, i32, P],
            "probe_copy": [P, P, i64, P],
            "check_recip_rn": [ctypes.c_uint32, ctypes.c_uint32, P, P, P],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        _lib = L
    return _lib


def call(name: str, *args) -> None:
    """Calls a probe (tensors become device pointers; the stream is torch's
    current one) and raises on a launch error."""
    import torch
    conv = [a.data_ptr() if hasattr(a, "data_ptr") else a for a in args]
    rc = getattr(lib(), name)(*conv, torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"{name}: hipError {rc}")
