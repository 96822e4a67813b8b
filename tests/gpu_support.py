"""Shared helpers for the GPU parity tests: device state for each algorithm,
device scalars, and the relative-error metric.  Calls go through the C-ABI
binding; nothing here computes an optimizer step."""
from __future__ import annotations

import sys

import numpy as np
import torch

import optimizer_step_adamw_amd as osa

DEV = "cuda"

# parity bounds: relerr_tau after 1 step / at the end of <= 100 steps
TOL_STEP1 = 2e-6
TOL_RUN = 5e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def relerr_tau(x, ref, tau):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(x - ref) / np.maximum(np.abs(ref), tau))) if x.size else 0.0


def err_report(x, ref, tau):
    """relerr_tau, the largest plain relative error (over ref != 0) and the
    share of elements where the floor tau engaged (|ref| < tau)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    nz = ref != 0
    plain = float(np.max(np.abs(x[nz] - ref[nz]) / np.abs(ref[nz]))) if nz.any() else 0.0
    share = float(np.mean(np.abs(ref) < tau)) if ref.size else 0.0
    return f"relerr_tau {relerr_tau(x, ref, tau):.3e}, max plain rel {plain:.3e}, tau engaged on {100 * share:.2f}%"


class DevScalars:
    """lr / step / found_inf / iter / inv_scale device scalars of one run."""

    def __init__(self, lr: float, inv_scale=None):
        self.lr = torch.tensor([lr], dtype=torch.float32, device=DEV)
        self.step = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.found_inf = torch.zeros(1, dtype=torch.float32, device=DEV)
        self.iter = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.inv_scale = (None if inv_scale is None else
                          torch.tensor([inv_scale], dtype=torch.float32, device=DEV))


def bf16_bits(t: torch.Tensor) -> torch.Tensor:
    """fp32 -> bf16 (RNE, torch's cast), returned as int16 bit patterns."""
    return t.to(torch.bfloat16).view(torch.int16)


def to_np_u16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class AdamState:
    """Device buffers for AdamW / AdEMAMix / Adam-mini over a tensor list."""

    def __init__(self, p0: list, *, grad_bf16=False, param_bf16=False, ademamix=False,
                 v_len=None, moments_interleaved=False):
        n = len(p0)
        self.param_bf16 = param_bf16
        self.grad_bf16 = grad_bf16
        if param_bf16:
            self.p = [torch.empty(x.numel(), dtype=torch.int16, device=DEV) for x in p0]
            self.r = [torch.empty(x.numel(), dtype=torch.int16, device=DEV) for x in p0]
            for x, b, r in zip(p0, self.p, self.r):
                osa.optim_remainder_split(x, b, r, x.numel())
        else:
            self.p = [x.clone() for x in p0]
            self.r = None
        gdt = torch.int16 if grad_bf16 else torch.float32
        self.g = [torch.zeros(x.numel(), dtype=gdt, device=DEV) for x in p0]
        if moments_interleaved:
            # the plan's interleaved moment layout: m, v (, m2) of each block of
            # 1024 elements side by side in one array per tensor
            k = 3 if ademamix else 2
            self.m = [torch.zeros(k * ((x.numel() + 1023) // 1024 * 1024), dtype=torch.float32, device=DEV)
                      for x in p0]
            self.v = self.m2 = None
        else:
            self.m = [torch.zeros(x.numel(), dtype=torch.float32, device=DEV) for x in p0]
            vl = v_len or [x.numel() for x in p0]
            self.v = [torch.zeros(k, dtype=torch.float32, device=DEV) for k in vl]
            self.m2 = [torch.zeros(x.numel(), dtype=torch.float32, device=DEV) for x in p0] if ademamix else None
        self.n = n

    def tensor_list(self, wd, mini_kind=None, head_numel=None):
        return osa.TensorList(
            self.p, self.g, m=self.m, v=self.v, m2=self.m2, remainders=self.r, weight_decay=wd,
            mini_kind=mini_kind, head_numel=head_numel,
            param_dtype=osa.OPTIM_BF16 if self.param_bf16 else osa.OPTIM_F32,
            grad_dtype=osa.OPTIM_BF16 if self.grad_bf16 else osa.OPTIM_F32)

    def master(self, i) -> torch.Tensor:
        """fp32 master of tensor i (reconstructed on the GPU for bf16 params)."""
        if not self.param_bf16:
            return self.p[i]
        out = torch.empty(self.p[i].numel(), dtype=torch.float32, device=DEV)
        osa.optim_remainder_reconstruct(self.p[i], self.r[i], out, out.numel())
        return out

    def buffers(self):
        out = list(self.p) + list(self.m) + list(self.v or [])
        if self.r:
            out += list(self.r)
        if self.m2:
            out += list(self.m2)
        return out


class QuantState:
    """Device buffers for the blockwise 8-bit / 4-bit step."""

    def __init__(self, p0: list, bits: int, block: int, ademamix: bool = False):
        self.bits, self.block = bits, block
        self.p = [x.clone() for x in p0]
        self.g = [torch.zeros_like(x) for x in p0]
        nbytes = [(x.numel() * bits + 7) // 8 for x in p0]
        nblk = [(x.numel() + block - 1) // block for x in p0]
        self.qm = [torch.zeros(k, dtype=torch.uint8, device=DEV) for k in nbytes]
        self.qv = [torch.zeros(k, dtype=torch.uint8, device=DEV) for k in nbytes]
        self.am = [torch.zeros(k, dtype=torch.float32, device=DEV) for k in nblk]
        self.av = [torch.zeros(k, dtype=torch.float32, device=DEV) for k in nblk]
        self.qm2 = [torch.zeros(k, dtype=torch.uint8, device=DEV) for k in nbytes] if ademamix else None
        self.am2 = [torch.zeros(k, dtype=torch.float32, device=DEV) for k in nblk] if ademamix else None

    def tensor_list(self, wd):
        return osa.TensorList(self.p, self.g, qm=self.qm, qv=self.qv, absmax_m=self.am,
                              absmax_v=self.av, qm2=self.qm2, absmax_m2=self.am2, weight_decay=wd)

    def buffers(self):
        out = list(self.p) + list(self.qm) + list(self.qv) + list(self.am) + list(self.av)
        if self.qm2:
            out += list(self.qm2) + list(self.am2)
        return out


def snapshot(bufs):
    return [b.clone() for b in bufs]


def all_equal(a, b) -> bool:
    """Bit for bit (NaN patterns compare equal to themselves, -0.0 differs
    from +0.0)."""
    return len(a) == len(b) and all(
        x.shape == y.shape and torch.equal(x.reshape(-1).view(torch.uint8), y.reshape(-1).view(torch.uint8))
        for x, y in zip(a, b))
