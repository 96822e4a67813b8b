"""Python binding of liboptim_step.so, the fused AdamW-family optimizer step
for AMD Instinct MI355X (gfx950).

Argument marshalling only: torch tensors are turned into device pointers and a
HIP stream handle; every step of the computation runs in the library's HIP
kernels.  Functions keep the C names of ``include/optim_step.h``.  If the
library has not been built, importing the binding works but every call raises
``RuntimeError`` -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

from .build import LIB_PATH, build as build_library

OPTIM_OK = 0
OPTIM_EINVAL, OPTIM_EALIGN, OPTIM_EDTYPE, OPTIM_EWORKSPACE, OPTIM_EUNSUPPORTED, OPTIM_EHIP = range(1, 7)
OPTIM_F32, OPTIM_BF16, OPTIM_F16 = 0, 1, 2
OPTIM_LAYOUT_SEPARATE, OPTIM_LAYOUT_INTERLEAVED = 0, 1
(OPTIM_ALGO_ADAMW, OPTIM_ALGO_ADEMAMIX, OPTIM_ALGO_ADAM_MINI, OPTIM_ALGO_BLOCKWISE,
 OPTIM_ALGO_BLOCKWISE_ADEMAMIX, OPTIM_ALGO_LION, OPTIM_ALGO_LAMB) = range(7)
OPTIM_MINI_FULL_V, OPTIM_MINI_HEAD, OPTIM_MINI_SCALAR = range(3)
OPTIM_SCHED_NONE, OPTIM_SCHED_COSINE = 0, 1

EXPORTED = (
    "optim_last_error", "optim_plan_workspace_size", "optim_plan_create", "optim_plan_destroy",
    "optim_plan_set_schedule", "optim_step_adamw", "optim_step_ademamix", "optim_step_adam_mini",
    "optim_step_8bit_blockwise", "optim_check_finite", "optim_remainder_split",
    "optim_remainder_reconstruct", "optim_quant_codebook", "optim_quantize_blockwise",
    "optim_dequantize_blockwise", "optim_grad_norm", "optim_scaler_update",
    "optim_step_8bit_blockwise_ademamix", "optim_step_lion", "optim_step_lamb",
    "optim_plan_create_static", "optim_plan_trace", "optim_plan_trace_read",
)
# bytes of the library's static per-device workspace (optim_plan_create_static)
OPTIM_STATIC_WORKSPACE_BYTES = 16 << 20


class OptimError(RuntimeError):
    def __init__(self, code: int, fn: str, msg: str):
        super().__init__(f"{fn} failed with code {code}: {msg}")
        self.code = code


_P = ctypes.c_void_p
_PP = ctypes.POINTER(ctypes.c_void_p)


class optim_tensor_list(ctypes.Structure):
    _fields_ = [
        ("n", ctypes.c_int32),
        ("numel", ctypes.POINTER(ctypes.c_int64)),
        ("param", _PP), ("grad", _PP), ("m", _PP), ("v", _PP), ("m2", _PP),
        ("remainder", _PP), ("qm", _PP), ("qv", _PP), ("absmax_m", _PP), ("absmax_v", _PP),
        ("weight_decay", ctypes.POINTER(ctypes.c_double)),
        ("mini_kind", ctypes.POINTER(ctypes.c_int32)),
        ("head_numel", ctypes.POINTER(ctypes.c_int64)),
        ("param_dtype", ctypes.c_int32),
        ("grad_dtype", ctypes.c_int32),
        ("qm2", _PP), ("absmax_m2", _PP), ("master", _PP), ("scale_m", _PP), ("scale_v", _PP),
    ]


class optim_plan_opts(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("block", ctypes.c_int32), ("grid", ctypes.c_int32),
                ("tile", ctypes.c_int32), ("state_dtype", ctypes.c_int32), ("segment_bytes", ctypes.c_int64),
                ("state_layout", ctypes.c_int32)]


class optim_kernel_time(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char_p), ("workgroups", ctypes.c_int64), ("ms", ctypes.c_double)]


class optim_adamw_hp(ctypes.Structure):
    _fields_ = [("beta1", ctypes.c_double), ("beta2", ctypes.c_double), ("eps", ctypes.c_double)]


class optim_lion_hp(ctypes.Structure):
    _fields_ = [("beta1", ctypes.c_double), ("beta2", ctypes.c_double)]


class optim_ademamix_hp(ctypes.Structure):
    _fields_ = [("beta1", ctypes.c_double), ("beta2", ctypes.c_double), ("beta3", ctypes.c_double),
                ("alpha", ctypes.c_double), ("eps", ctypes.c_double)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree library; raise if it was never built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with optimizer_step_adamw_amd.build_library() "
                "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, f64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_size_t
        tl = ctypes.POINTER(optim_tensor_list)
        opts = ctypes.POINTER(optim_plan_opts)
        sigs = {
            "optim_last_error": ([], ctypes.c_char_p),
            "optim_plan_workspace_size": ([tl, i32, opts, ctypes.POINTER(sz)], i32),
            "optim_plan_create": ([tl, i32, opts, _P, sz, _P, ctypes.POINTER(_P)], i32),
            "optim_plan_destroy": ([_P], i32),
            "optim_plan_create_static": ([tl, i32, opts, _P, ctypes.POINTER(_P)], i32),
            "optim_plan_trace": ([_P, i32], i32),
            "optim_plan_trace_read": ([_P, ctypes.POINTER(optim_kernel_time), i32, ctypes.POINTER(i32),
                                       ctypes.POINTER(i64)], i32),
            "optim_plan_set_schedule": ([_P, i32, f64, f64, i32, _P], i32),
            "optim_step_adamw": ([_P, ctypes.POINTER(optim_adamw_hp), _P, _P, _P, _P, _P], i32),
            "optim_step_ademamix": ([_P, ctypes.POINTER(optim_ademamix_hp), _P, _P, _P, _P, _P], i32),
            "optim_step_adam_mini": ([_P, ctypes.POINTER(optim_adamw_hp), _P, _P, _P, _P, _P], i32),
            "optim_step_8bit_blockwise": ([_P, ctypes.POINTER(optim_adamw_hp), i32, i32, _P, _P, _P,
                                           _P, _P], i32),
            "optim_check_finite": ([_P, _P, _P], i32),
            "optim_remainder_split": ([_P, _P, _P, i64, _P], i32),
            "optim_remainder_reconstruct": ([_P, _P, _P, i64, _P], i32),
            "optim_quant_codebook": ([i32, i32, _P, _P], i32),
            "optim_quantize_blockwise": ([_P, i32, _P, i64, _P, _P, _P], i32),
            "optim_dequantize_blockwise": ([_P, i32, _P, _P, i64, _P, _P], i32),
            "optim_grad_norm": ([_P, _P, f64, _P, _P, _P, _P], i32),
            "optim_scaler_update": ([_P, _P, _P, _P, f64, f64, i32, _P], i32),
            "optim_step_8bit_blockwise_ademamix": ([_P, ctypes.POINTER(optim_ademamix_hp), i32, i32, _P, _P,
                                                    _P, _P, _P], i32),
            "optim_step_lion": ([_P, ctypes.POINTER(optim_lion_hp), _P, _P, _P, _P, _P], i32),
            "optim_step_lamb": ([_P, ctypes.POINTER(optim_adamw_hp), _P, _P, _P, _P, _P], i32),
        }
        for name, (args, res) in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(rc: int, fn: str) -> None:
    if rc != OPTIM_OK:
        raise OptimError(rc, fn, lib().optim_last_error().decode())


def _ptr(t) -> Optional[int]:
    """Device address of a tensor argument (None and plain integers pass
    through).  The kernels walk numel() elements from data_ptr(), so a torch
    tensor must be on the GPU and contiguous: anything else is refused here,
    before the library sees it."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if hasattr(t, "is_cuda") and not t.is_cuda:
        raise ValueError(f"expected a GPU tensor, got one on {t.device}")
    if hasattr(t, "is_contiguous") and not t.is_contiguous():
        raise ValueError(f"expected a contiguous tensor, got shape {tuple(t.shape)} with strides {t.stride()}")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# --------------------------------------------------------------------------
# tensor lists
class TensorList:
    """Host arrays of an optim_tensor_list, kept alive with the structure."""

    def __init__(self, params: Sequence, grads: Sequence, *, m=None, v=None, m2=None,
                 remainders=None, qm=None, qv=None, absmax_m=None, absmax_v=None,
                 qm2=None, absmax_m2=None, master=None, scale_m=None, scale_v=None,
                 weight_decay: Sequence[float], mini_kind=None, head_numel=None,
                 param_dtype: int = OPTIM_F32, grad_dtype: int = OPTIM_F32,
                 numel: Optional[Sequence[int]] = None):
        n = len(params)
        self.n = n
        self._keep = []

        def parr(xs):
            if xs is None:
                return None
            a = (ctypes.c_void_p * max(n, 1))(*[_ptr(x) for x in xs])
            self._keep.append(a)
            return ctypes.cast(a, _PP)

        numels = list(numel) if numel is not None else [int(p.numel()) for p in params]
        self._numel = (ctypes.c_int64 * max(n, 1))(*numels)
        self._wd = (ctypes.c_double * max(n, 1))(*[float(w) for w in weight_decay])
        s = optim_tensor_list()
        s.n = n
        s.numel = ctypes.cast(self._numel, ctypes.POINTER(ctypes.c_int64))
        s.param, s.grad = parr(params), parr(grads)
        s.m, s.v, s.m2, s.remainder = parr(m), parr(v), parr(m2), parr(remainders)
        s.qm, s.qv, s.absmax_m, s.absmax_v = parr(qm), parr(qv), parr(absmax_m), parr(absmax_v)
        s.qm2, s.absmax_m2, s.master = parr(qm2), parr(absmax_m2), parr(master)
        s.scale_m, s.scale_v = parr(scale_m), parr(scale_v)
        s.weight_decay = ctypes.cast(self._wd, ctypes.POINTER(ctypes.c_double))
        if mini_kind is not None:
            self._kind = (ctypes.c_int32 * max(n, 1))(*mini_kind)
            self._hn = (ctypes.c_int64 * max(n, 1))(*(head_numel or [0] * n))
            s.mini_kind = ctypes.cast(self._kind, ctypes.POINTER(ctypes.c_int32))
            s.head_numel = ctypes.cast(self._hn, ctypes.POINTER(ctypes.c_int64))
        s.param_dtype, s.grad_dtype = param_dtype, grad_dtype
        self.struct = s


# --------------------------------------------------------------------------
# C entry points (same names)
def optim_plan_workspace_size(tl: TensorList, algo: int, opts: Optional[optim_plan_opts] = None) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().optim_plan_workspace_size(ctypes.byref(tl.struct), algo,
                                           ctypes.byref(opts) if opts else None, ctypes.byref(out)),
           "optim_plan_workspace_size")
    return out.value


def optim_plan_create(tl: TensorList, algo: int, opts, workspace, nbytes: int, stream=None) -> int:
    h = ctypes.c_void_p(0)
    _check(lib().optim_plan_create(ctypes.byref(tl.struct), algo, ctypes.byref(opts) if opts else None,
                                   _ptr(workspace), nbytes, _stream(stream), ctypes.byref(h)),
           "optim_plan_create")
    return h.value


def optim_plan_create_static(tl: TensorList, algo: int, opts, stream=None) -> int:
    h = ctypes.c_void_p(0)
    _check(lib().optim_plan_create_static(ctypes.byref(tl.struct), algo, ctypes.byref(opts) if opts else None,
                                          _stream(stream), ctypes.byref(h)),
           "optim_plan_create_static")
    return h.value


def optim_plan_trace(plan: int, capacity: int) -> None:
    _check(lib().optim_plan_trace(plan, int(capacity)), "optim_plan_trace")


def optim_plan_trace_read(plan: int, max_records: int = 1 << 16):
    """(records, dropped): records are (kernel name, workgroups, ms) in launch
    order; waits for the traced launches to finish and empties the trace."""
    buf = (optim_kernel_time * max(1, max_records))()
    n = ctypes.c_int32(0)
    dropped = ctypes.c_int64(0)
    _check(lib().optim_plan_trace_read(plan, buf, max_records, ctypes.byref(n), ctypes.byref(dropped)),
           "optim_plan_trace_read")
    recs = [(buf[i].kernel.decode(), int(buf[i].workgroups), float(buf[i].ms)) for i in range(min(n.value, max_records))]
    return recs, int(dropped.value)


def optim_plan_destroy(plan: int) -> None:
    _check(lib().optim_plan_destroy(plan), "optim_plan_destroy")


def optim_plan_set_schedule(plan: int, kind: int, lr_max: float, lr_min: float, K: int, iter_dev) -> None:
    _check(lib().optim_plan_set_schedule(plan, kind, lr_max, lr_min, K, _ptr(iter_dev)),
           "optim_plan_set_schedule")


def optim_step_adamw(plan, hp: optim_adamw_hp, lr_dev, inv_scale_dev, found_inf_dev, step_dev,
                     stream=None) -> None:
    _check(lib().optim_step_adamw(plan, ctypes.byref(hp), _ptr(lr_dev), _ptr(inv_scale_dev),
                                  _ptr(found_inf_dev), _ptr(step_dev), _stream(stream)),
           "optim_step_adamw")


def optim_step_ademamix(plan, hp: optim_ademamix_hp, lr_dev, inv_scale_dev, found_inf_dev, step_dev,
                        stream=None) -> None:
    _check(lib().optim_step_ademamix(plan, ctypes.byref(hp), _ptr(lr_dev), _ptr(inv_scale_dev),
                                     _ptr(found_inf_dev), _ptr(step_dev), _stream(stream)),
           "optim_step_ademamix")


def optim_step_adam_mini(plan, hp: optim_adamw_hp, lr_dev, inv_scale_dev, found_inf_dev, step_dev,
                         stream=None) -> None:
    _check(lib().optim_step_adam_mini(plan, ctypes.byref(hp), _ptr(lr_dev), _ptr(inv_scale_dev),
                                      _ptr(found_inf_dev), _ptr(step_dev), _stream(stream)),
           "optim_step_adam_mini")


def optim_step_8bit_blockwise(plan, hp: optim_adamw_hp, bits: int, block: int, lr_dev, inv_scale_dev,
                              found_inf_dev, step_dev, stream=None) -> None:
    _check(lib().optim_step_8bit_blockwise(plan, ctypes.byref(hp), bits, block, _ptr(lr_dev),
                                           _ptr(inv_scale_dev), _ptr(found_inf_dev), _ptr(step_dev),
                                           _stream(stream)),
           "optim_step_8bit_blockwise")


def optim_step_lion(plan, hp: optim_lion_hp, lr_dev, inv_scale_dev, found_inf_dev, step_dev,
                    stream=None) -> None:
    _check(lib().optim_step_lion(plan, ctypes.byref(hp), _ptr(lr_dev), _ptr(inv_scale_dev), _ptr(found_inf_dev),
                                 _ptr(step_dev), _stream(stream)), "optim_step_lion")


def optim_step_lamb(plan, hp: optim_adamw_hp, lr_dev, inv_scale_dev, found_inf_dev, step_dev,
                    stream=None) -> None:
    _check(lib().optim_step_lamb(plan, ctypes.byref(hp), _ptr(lr_dev), _ptr(inv_scale_dev), _ptr(found_inf_dev),
                                 _ptr(step_dev), _stream(stream)), "optim_step_lamb")


def optim_step_8bit_blockwise_ademamix(plan, hp: optim_ademamix_hp, bits: int, block: int, lr_dev,
                                       inv_scale_dev, found_inf_dev, step_dev, stream=None) -> None:
    _check(lib().optim_step_8bit_blockwise_ademamix(plan, ctypes.byref(hp), bits, block, _ptr(lr_dev),
                                                    _ptr(inv_scale_dev), _ptr(found_inf_dev), _ptr(step_dev),
                                                    _stream(stream)),
           "optim_step_8bit_blockwise_ademamix")


def optim_check_finite(plan, found_inf_dev, stream=None) -> None:
    _check(lib().optim_check_finite(plan, _ptr(found_inf_dev), _stream(stream)), "optim_check_finite")


def optim_grad_norm(plan, inv_scale_dev, max_norm: float, found_inf_dev, norm_dev, clip_inv_scale_dev,
                    stream=None) -> None:
    _check(lib().optim_grad_norm(plan, _ptr(inv_scale_dev), float(max_norm), _ptr(found_inf_dev),
                                 _ptr(norm_dev), _ptr(clip_inv_scale_dev), _stream(stream)), "optim_grad_norm")


def optim_scaler_update(scale_dev, inv_scale_dev, growth_tracker_dev, found_inf_dev, growth_factor: float,
                        backoff_factor: float, growth_interval: int, stream=None) -> None:
    _check(lib().optim_scaler_update(_ptr(scale_dev), _ptr(inv_scale_dev), _ptr(growth_tracker_dev),
                                     _ptr(found_inf_dev), float(growth_factor), float(backoff_factor),
                                     int(growth_interval), _stream(stream)), "optim_scaler_update")


def optim_remainder_split(master, bf16, rem, n: int, stream=None) -> None:
    _check(lib().optim_remainder_split(_ptr(master), _ptr(bf16), _ptr(rem), n, _stream(stream)),
           "optim_remainder_split")


def optim_remainder_reconstruct(bf16, rem, master, n: int, stream=None) -> None:
    _check(lib().optim_remainder_reconstruct(_ptr(bf16), _ptr(rem), _ptr(master), n, _stream(stream)),
           "optim_remainder_reconstruct")


def optim_quantize_blockwise(plan, is_signed: bool, x, n: int, codes, absmax, stream=None) -> None:
    _check(lib().optim_quantize_blockwise(plan, int(is_signed), _ptr(x), n, _ptr(codes), _ptr(absmax),
                                          _stream(stream)), "optim_quantize_blockwise")


def optim_dequantize_blockwise(plan, is_signed: bool, codes, absmax, n: int, x, stream=None) -> None:
    _check(lib().optim_dequantize_blockwise(plan, int(is_signed), _ptr(codes), _ptr(absmax), n, _ptr(x),
                                            _stream(stream)), "optim_dequantize_blockwise")


def optim_quant_codebook(bits: int, is_signed: bool):
    import numpy as np
    mb = bits - 1 if is_signed else bits
    vals = np.zeros(1 << mb, np.float32)
    thr = np.zeros(1 << mb, np.float32)
    _check(lib().optim_quant_codebook(bits, int(is_signed), vals.ctypes.data, thr.ctypes.data),
           "optim_quant_codebook")
    return vals, thr


# --------------------------------------------------------------------------
# convenience: a plan that owns its workspace tensor
class Plan:
    """Plan + workspace.  ``tl`` must hold device tensors that outlive it."""

    def __init__(self, tl: TensorList, algo: int, *, bits: int = 0, block: int = 0, grid: int = 0,
                 tile: int = 0, state_dtype: int = OPTIM_F32, segment_bytes: int = 0,
                 state_layout: int = 0, device=None, stream=None):
        import torch
        self.algo = algo
        self.tl = tl
        self.opts = optim_plan_opts(bits, block, grid, tile, state_dtype, segment_bytes, state_layout)
        nbytes = optim_plan_workspace_size(tl, algo, self.opts)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device or "cuda")
        self.handle = optim_plan_create(tl, algo, self.opts, self.workspace, nbytes, stream)

    def close(self) -> None:
        if getattr(self, "handle", None):
            optim_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# --------------------------------------------------------------------------
# Adam-mini partition by parameter name ("Adam-mini <> DTensor", AdamWMini)
_EMBED_KEYS = ("embed", "embd", "wte", "lm_head.weight", "output.weight")
_QK_KEYS = ("q_proj.weight", "k_proj.weight", "wq.weight", "wk.weight")


def adam_mini_partition(names: Sequence[str], numels: Sequence[int], dim: int, n_heads: int,
                        weight_decay: float):
    """Per tensor: (mini_kind, head_numel, weight_decay).  Embedding/output
    tensors keep a full v; q/k tensors share v per block of dim*dim/n_heads
    elements; all others share one v; names with 'norm' or 'ln_f' get no
    decay."""
    if (dim * dim) % n_heads:
        raise ValueError(f"dim*dim ({dim * dim}) not divisible by n_heads ({n_heads})")
    kinds: List[int] = []
    heads: List[int] = []
    wds: List[float] = []
    for name, n in zip(names, numels):
        wds.append(0.0 if ("norm" in name or "ln_f" in name) else weight_decay)
        if any(k in name for k in _EMBED_KEYS):
            kinds.append(OPTIM_MINI_FULL_V)
            heads.append(0)
        elif any(k in name for k in _QK_KEYS):
            kinds.append(OPTIM_MINI_HEAD)
            heads.append(dim * dim // n_heads)
        else:
            kinds.append(OPTIM_MINI_SCALAR)
            heads.append(int(n))
    return kinds, heads, wds
