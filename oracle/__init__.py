"""CPU oracle for the fused AdamW-family optimizer step (test infrastructure).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the product path never does.
It wraps ``oracle.c`` (plain scalar C, fp64, built with gcc) through ctypes and
adds thin numpy drivers that hold per-parameter state.  It shares no code with
the HIP library.

Each function cites the web page (title, section) whose definition it follows;
see the header of ``oracle.c`` for the page list.  Conversions between bit
patterns and numbers here are exact (bf16/fp32 -> float64 widening).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-D_DEFAULT_SOURCE", "-fPIC", "-shared",
            "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
            "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None

_d = ctypes.c_double
_i64 = ctypes.c_int64
_i32 = ctypes.c_int
_p = ctypes.c_void_p


_SIGS = {
    "oracle_adamw_step": [_i64, _p, _p, _p, _p, _d, _d, _d, _d, _d, _i64],
    "mutant_adamw_decay_after_step": [_i64, _p, _p, _p, _p, _d, _d, _d, _d, _d, _i64],
    "oracle_ademamix_step": [_i64, _p, _p, _p, _p, _p, _d, _d, _d, _d, _d, _d, _d, _i64],
    "oracle_adam_mini_step": [_i64, _i64, _p, _p, _p, _p, _d, _d, _d, _d, _d, _i64],
    "oracle_any_nonfinite": [_i64, _p],
    "oracle_cosine_lr": [_i64, _i64, _d, _d],
    "oracle_remainder_split": [_i64, _p, _p, _p],
    "oracle_remainder_reconstruct": [_i64, _p, _p, _p],
    "oracle_remainder_exhaustive": [],
    "oracle_dynamic_map": [_i32, _p],
    "oracle_thresholds": [_i32, _p, _p],
    "oracle_quantize": [_i64, _i64, _i32, _i32, _p, _p, _p, _p],
    "oracle_dequantize": [_i64, _i64, _i32, _i32, _p, _p, _p, _p],
    "oracle_pack_nibbles": [_i64, _p, _p],
    "oracle_unpack_nibbles": [_i64, _p, _p],
    "oracle_blockwise_step": [_i64, _i64, _i32, _p, _p, _p, _p, _p, _p,
                              _d, _d, _d, _d, _d, _i64, _p, _p],
    "oracle_blockwise_ademamix_step": [_i64, _i64, _i32, _p, _p, _p, _p, _p, _p, _p, _p,
                                       _d, _d, _d, _d, _d, _d, _d, _i64, _p, _p, _p],
    "oracle_lion_step": [_i64, _p, _p, _p, _d, _d, _d, _d],
    "oracle_lamb_step": [_i64, _p, _p, _p, _p, _d, _d, _d, _d, _d, _i64, _p],
    "oracle_round_model_copy": [_i64, _i32, _p, _p],
    "oracle_adamw_scaled_step": [_i64, _i32, _p, _p, _p, _p, _p, _p, _d, _d, _d, _d, _d, _i64, _p, _p],
    "oracle_sumsq": [_i64, _p],
    "oracle_clip_coef": [_d, _d],
    "oracle_scaler_update": [_p, _p, _i32, _d, _d, _i32],
}
_RESTYPES = {"oracle_any_nonfinite": _i32, "oracle_cosine_lr": ctypes.c_float,
             "oracle_remainder_exhaustive": _i64, "oracle_dynamic_map": _i32,
             "oracle_sumsq": _d, "oracle_clip_coef": _d}


def load(path: str) -> ctypes.CDLL:
    """A configured handle on a build of oracle.c at `path`."""
    L = ctypes.CDLL(path)
    for name, args in _SIGS.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = _RESTYPES.get(name, None)
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = load(_LIB_PATH)
    return _lib


class use_build:
    """Context manager: route every oracle call to another build of
    oracle.c (the mutation test plants mistakes in copies of it)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = lib()
        _lib = load(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def compile_source(src: str, out_path: str) -> None:
    """gcc a variant of the oracle source with the flags build() uses."""
    c_path = out_path[:-3] + ".c"
    with open(c_path, "w") as f:
        f.write(src)
    subprocess.check_call([
        "gcc", "-O2", "-std=c11", "-D_DEFAULT_SOURCE", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math", "-w", "-o", out_path, c_path, "-lm"])


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# exact widening of stored formats
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f32_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


# --------------------------------------------------------------------------
# per-step functions (in place on float64 state arrays)
def adamw_step(p, m, v, g, lr, beta1, beta2, eps, wd, t):
    """AdamW, Algorithm 2 decay order (bitsandbytes PR #2040, description)."""
    lib().oracle_adamw_step(p.size, _ptr(p), _ptr(m), _ptr(v), _ptr(_f64(g)),
                            lr, beta1, beta2, eps, wd, t)


def mutant_adamw_decay_after_step(p, m, v, g, lr, beta1, beta2, eps, wd, t):
    """TEST MUTANT: the decay-after ordering the bitsandbytes PR removes."""
    lib().mutant_adamw_decay_after_step(p.size, _ptr(p), _ptr(m), _ptr(v),
                                        _ptr(_f64(g)), lr, beta1, beta2, eps, wd, t)


def ademamix_step(p, m1, m2, nu, g, lr, beta1, beta2, beta3, alpha, eps, wd, t):
    """AdEMAMix with constant alpha/beta3, m2 not bias-corrected."""
    lib().oracle_ademamix_step(p.size, _ptr(p), _ptr(m1), _ptr(m2), _ptr(nu),
                               _ptr(_f64(g)), lr, beta1, beta2, beta3, alpha,
                               eps, wd, t)


def adam_mini_step(p, m, V, g, block, lr, beta1, beta2, eps, wd, t):
    """Adam-mini shared-v step for one tensor (block = head_numel or numel)."""
    assert p.size % block == 0 and V.size == p.size // block
    lib().oracle_adam_mini_step(p.size, block, _ptr(p), _ptr(m), _ptr(V),
                                _ptr(_f64(g)), lr, beta1, beta2, eps, wd, t)


def any_nonfinite(x) -> bool:
    x = _f64(x)
    return bool(lib().oracle_any_nonfinite(x.size, _ptr(x)))


def round_model_copy(master_f32: np.ndarray, half: bool) -> np.ndarray:
    """fp32 master -> bf16 or fp16 bit patterns, round to nearest even."""
    u = np.ascontiguousarray(f32_bits(master_f32).ravel())
    out = np.empty(u.size, np.uint16)
    lib().oracle_round_model_copy(u.size, int(bool(half)), _ptr(u), _ptr(out))
    return out


def adamw_scaled_step(p, qm, qv, sm, sv, g_f32, half, lr, beta1, beta2, eps, wd, t):
    """AdamW with per-tensor scaled 16-bit moments (fp16 if half, else bf16):
    qm, qv uint16 patterns and sm, sv float32[1] scales, all in place.
    Returns the fp32 moments before rescaling."""
    for a in (qm, qv):
        assert a.dtype == np.uint16 and a.flags["C_CONTIGUOUS"]
    for a in (sm, sv):
        assert a.dtype == np.float32 and a.size == 1
    g = np.ascontiguousarray(g_f32, np.float32).ravel()
    m32, v32 = np.empty(p.size, np.float32), np.empty(p.size, np.float32)
    lib().oracle_adamw_scaled_step(p.size, int(bool(half)), _ptr(p), _ptr(qm), _ptr(qv), _ptr(sm),
                                   _ptr(sv), _ptr(g), lr, beta1, beta2, eps, wd, t, _ptr(m32),
                                   _ptr(v32))
    return m32, v32


def lion_step(p, m_f32, g_f32, lr, beta1, beta2, wd):
    """Lion (decay before the sign update); m float32 state, in place."""
    assert m_f32.dtype == np.float32 and m_f32.flags["C_CONTIGUOUS"]
    g = np.ascontiguousarray(g_f32, np.float32).ravel()
    lib().oracle_lion_step(p.size, _ptr(p), _ptr(m_f32), _ptr(g), lr, beta1, beta2, wd)


def lamb_step(p, m, v, g, lr, beta1, beta2, eps, wd, t):
    """LAMB on one tensor (per-tensor trust ratio), in place; returns u."""
    u = np.empty(p.size)
    lib().oracle_lamb_step(p.size, _ptr(p), _ptr(m), _ptr(v), _ptr(_f64(g)), lr, beta1, beta2,
                           eps, wd, t, _ptr(u))
    return u


def grad_norm(grads, inv_scale: float = 1.0) -> float:
    """Global L2 norm of the unscaled gradients G*s over the whole list
    (FusedAdam & PyTorch Lightning AMP: clipping folded into the step)."""
    total = 0.0
    for G in grads:
        x = _f64(np.asarray(G, np.float64).ravel() * inv_scale)
        total += lib().oracle_sumsq(x.size, _ptr(x))
    return float(np.sqrt(total))


def clip_coef(norm: float, max_norm: float) -> float:
    return float(lib().oracle_clip_coef(norm, max_norm))


class ScalerState:
    """Dynamic loss scale (fp32) and count of clean steps."""

    def __init__(self, scale: float, tracker: int = 0):
        self.scale = np.array([scale], np.float32)
        self.tracker = np.array([tracker], np.int32)

    def update(self, found_inf: bool, growth: float, backoff: float, interval: int):
        lib().oracle_scaler_update(_ptr(self.scale), _ptr(self.tracker), int(bool(found_inf)),
                                   growth, backoff, interval)


def cosine_lr(k: int, K: int, lr_max: float, lr_min: float = 0.0) -> np.float32:
    return np.float32(lib().oracle_cosine_lr(k, K, lr_max, lr_min))


# --------------------------------------------------------------------------
# bf16 + int16 remainder (TransformerEngine PR #1408, description)
def remainder_split(x_f32: np.ndarray):
    u = np.ascontiguousarray(f32_bits(x_f32).ravel())
    b = np.empty(u.size, np.uint16)
    r = np.empty(u.size, np.int16)
    lib().oracle_remainder_split(u.size, _ptr(u), _ptr(b), _ptr(r))
    return b, r


def remainder_reconstruct(b: np.ndarray, r: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16).ravel()
    r = np.ascontiguousarray(r, dtype=np.int16).ravel()
    u = np.empty(b.size, np.uint32)
    lib().oracle_remainder_reconstruct(b.size, _ptr(b), _ptr(r), _ptr(u))
    return u.view(np.float32)


def remainder_exhaustive_failures() -> int:
    return int(lib().oracle_remainder_exhaustive())


# --------------------------------------------------------------------------
# blockwise quantized states
def dynamic_map(mag_bits: int) -> np.ndarray:
    M = np.zeros(1 << mag_bits, np.float32)
    cnt = lib().oracle_dynamic_map(mag_bits, _ptr(M))
    assert cnt == M.size
    return M


def thresholds(M: np.ndarray) -> np.ndarray:
    T = np.zeros(M.size, np.float32)
    lib().oracle_thresholds(M.size, _ptr(np.ascontiguousarray(M, np.float32)), _ptr(T))
    return T


def quantize(x: np.ndarray, block: int, mag_bits: int, signed: bool):
    x = np.ascontiguousarray(x, np.float32).ravel()
    T = thresholds(dynamic_map(mag_bits))
    codes = np.empty(x.size, np.uint8)
    absmax = np.empty((x.size + block - 1) // block, np.float32)
    lib().oracle_quantize(x.size, block, mag_bits, int(signed), _ptr(x), _ptr(T),
                          _ptr(codes), _ptr(absmax))
    return codes, absmax


def dequantize(codes: np.ndarray, absmax: np.ndarray, block: int, mag_bits: int,
               signed: bool) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8).ravel()
    absmax = np.ascontiguousarray(absmax, np.float32)
    M = dynamic_map(mag_bits)
    x = np.empty(codes.size, np.float32)
    lib().oracle_dequantize(codes.size, block, mag_bits, int(signed), _ptr(codes),
                            _ptr(M), _ptr(absmax), _ptr(x))
    return x


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8).ravel()
    out = np.empty((codes.size + 1) // 2, np.uint8)
    lib().oracle_pack_nibbles(codes.size, _ptr(codes), _ptr(out))
    return out


def unpack_nibbles(packed: np.ndarray, n: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, np.uint8).ravel()
    out = np.empty(n, np.uint8)
    lib().oracle_unpack_nibbles(n, _ptr(packed), _ptr(out))
    return out


def blockwise_step(p, g_f32, qm, qv, am, av, bits, block, lr, beta1, beta2, eps,
                   wd, t):
    """Blockwise 8-bit/4-bit 2-state AdamW step; codes unpacked, in place."""
    n = p.size
    g = np.ascontiguousarray(g_f32, np.float32).ravel()
    sm = np.empty(n, np.float32)
    sv = np.empty(n, np.float32)
    lib().oracle_blockwise_step(n, block, bits, _ptr(p), _ptr(g), _ptr(qm), _ptr(qv),
                                _ptr(am), _ptr(av), lr, beta1, beta2, eps, wd, t,
                                _ptr(sm), _ptr(sv))
    return sm, sv  # the fp32 states before requantization


def blockwise_ademamix_step(p, g_f32, qm, qm2, qv, am, am2, av, bits, block, lr, beta1, beta2,
                            beta3, alpha, eps, wd, t):
    """Blockwise 8-bit/4-bit AdEMAMix step (m1, m2 signed, nu unsigned); codes
    unpacked, in place.  Returns the fp32 states before requantization."""
    n = p.size
    g = np.ascontiguousarray(g_f32, np.float32).ravel()
    sm, sm2, sv = (np.empty(n, np.float32) for _ in range(3))
    lib().oracle_blockwise_ademamix_step(n, block, bits, _ptr(p), _ptr(g), _ptr(qm), _ptr(qm2),
                                         _ptr(qv), _ptr(am), _ptr(am2), _ptr(av), lr, beta1,
                                         beta2, beta3, alpha, eps, wd, t, _ptr(sm), _ptr(sm2),
                                         _ptr(sv))
    return sm, sm2, sv


# --------------------------------------------------------------------------
# Adam-mini partition by parameter name ("Adam-mini <> DTensor", AdamWMini)
MINI_FULL_V, MINI_HEAD, MINI_SCALAR = 0, 1, 2


def adam_mini_kind(name: str) -> int:
    if any(s in name for s in ("embed", "embd", "wte", "lm_head.weight", "output.weight")):
        return MINI_FULL_V
    if any(s in name for s in ("q_proj.weight", "k_proj.weight", "wq.weight", "wk.weight")):
        return MINI_HEAD
    return MINI_SCALAR


def adam_mini_weight_decay(name: str, wd: float) -> float:
    return 0.0 if ("norm" in name or "ln_f" in name) else wd


# --------------------------------------------------------------------------
# error metric: |x - ref| / max(|ref|, tau)
def relerr_tau(x, ref, tau: float) -> np.ndarray:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.abs(x - ref) / np.maximum(np.abs(ref), tau)
