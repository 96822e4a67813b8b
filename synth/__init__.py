"""Seeded synthetic inputs for the optimizer-step workloads.

This module holds workload shapes, value distributions, hyperparameters and
seeds, and nothing of the optimizer's arithmetic.  Both the HIP path's tests
and the oracle draw their inputs from here.

Seeds: every draw is keyed by (2040, workload, tensor index, step, stream);
stream 0 = initial parameters, 1 = gradients, 2 = inf-injection site.
"N(0, s)" means a normal with standard deviation s: float64 normals are scaled
by s and rounded once to float32.

Host draws use numpy PCG64 keyed by a SeedSequence (float64 normal * std,
rounded to float32).  Device draws (for the billion-element lists, where host
RNG is too slow) use torch's float32 generator on the device seeded from the
same key; which one a test used is stated there.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

ROOT_SEED = 2040
P0, GRAD, INF = 0, 1, 2


def key_seed(*key: int) -> int:
    ss = np.random.SeedSequence([ROOT_SEED, *[int(k) for k in key]])
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))


def host_rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT_SEED, *key])))


def host_normal(n: int, std: float, *key: int) -> np.ndarray:
    """float32 array of n draws from N(0, std) (float64 normal * std, RNE)."""
    return (host_rng(*key).standard_normal(n) * std).astype(np.float32)


def device_normal(n: int, std: float, device, *key: int):
    """N(0, std) drawn on a torch device: float32 normals from torch's
    generator seeded with the key, times std in float32 (used for the
    billion-element lists, where host generation is too slow)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(key_seed(*key))
    out = torch.randn(n, dtype=torch.float32, device=device, generator=gen)
    out.mul_(std)
    return out


def device_randint(high: int, device, *key: int) -> int:
    import torch
    gen = torch.Generator(device="cpu")
    gen.manual_seed(key_seed(*key))
    return int(torch.randint(0, high, (1,), generator=gen).item())


# --------------------------------------------------------------------------
# Llama-shaped parameter lists
@dataclass
class TensorSpec:
    name: str
    shape: Tuple[int, ...]

    @property
    def numel(self) -> int:
        n = 1
        for s in self.shape:
            n *= s
        return n

    @property
    def is_norm(self) -> bool:
        return "norm" in self.name


def llama_list(n_layers: int, dim: int, ffn: int, vocab: int, tied: bool) -> List[TensorSpec]:
    out = [TensorSpec("tok_embeddings.weight", (vocab, dim))]
    for i in range(n_layers):
        pre = f"layers.{i}."
        out += [
            TensorSpec(pre + "attention.wq.weight", (dim, dim)),
            TensorSpec(pre + "attention.wk.weight", (dim, dim)),
            TensorSpec(pre + "attention.wv.weight", (dim, dim)),
            TensorSpec(pre + "attention.wo.weight", (dim, dim)),
            TensorSpec(pre + "feed_forward.w1.weight", (ffn, dim)),
            TensorSpec(pre + "feed_forward.w2.weight", (dim, ffn)),
            TensorSpec(pre + "feed_forward.w3.weight", (ffn, dim)),
            TensorSpec(pre + "attention_norm.weight", (dim,)),
            TensorSpec(pre + "ffn_norm.weight", (dim,)),
        ]
    out.append(TensorSpec("norm.weight", (dim,)))
    if not tied:
        out.append(TensorSpec("output.weight", (vocab, dim)))
    return out


# --------------------------------------------------------------------------
# workloads
@dataclass
class AdamWHP:
    lr: float
    beta1: float
    beta2: float
    eps: float
    wd: float


@dataclass
class Workload:
    name: str
    index: int
    tensors: List[TensorSpec]
    p_std: float
    g_std: float
    steps: int
    hp: AdamWHP
    extra: dict = field(default_factory=dict)

    @property
    def numel(self) -> int:
        return sum(t.numel for t in self.tensors)


def c1_single_tensor() -> Workload:
    """One fp32 tensor of 1,048,576 elements, AdamW, 10 steps."""
    return Workload("adamw_fp32_1M", 0, [TensorSpec("w", (1 << 20,))], 0.02, 1e-3, 10,
                    AdamWHP(1e-3, 0.9, 0.999, 1e-8, 0.01))


def c2_decay_stress() -> Workload:
    """fp32 4096x4096, AdamW lr=0.1 wd=0.1, 100 steps, plus AdEMAMix on it."""
    return Workload("adamw_ademamix_fp32_4096x4096", 1, [TensorSpec("w", (4096, 4096))],
                    0.02, 1e-2, 100, AdamWHP(0.1, 0.9, 0.999, 1e-8, 0.1),
                    extra=dict(beta3=0.9999, alpha=5.0))


def c3_llama_1b() -> Workload:
    """Llama-shaped ~1.1B list (16 layers, d=2048, ffn=8192, vocab=32000, tied
    embedding): bf16 params + int16 remainders, bf16 grads x65536, inf every 50
    steps, cosine lr on the device (lr_max 3e-4, 100 iterations)."""
    return Workload("adamw_bf16_remainder_amp_llama1b", 2,
                    llama_list(16, 2048, 8192, 32000, tied=True), 0.02, 1e-3, 100,
                    AdamWHP(3e-4, 0.9, 0.95, 1e-8, 0.1),
                    extra=dict(loss_scale=65536.0, inf_every=50, lr_min=0.0))


def c4_blockwise() -> Workload:
    """268,435,456 fp32 params, blockwise 8-bit (block 256) and 4-bit (block 128)."""
    return Workload("adamw_blockwise_8bit_4bit_268M", 3, [TensorSpec("w", (1 << 28,))],
                    0.02, 1e-3, 10, AdamWHP(1e-3, 0.9, 0.999, 1e-8, 0.01),
                    extra=dict(block8=256, block4=128))


def c5_adam_mini_7b() -> Workload:
    """Adam-mini over a 7B Llama-shaped list (32 layers, d=4096, 32 heads,
    ffn=11008, vocab=32000, untied output)."""
    return Workload("adam_mini_llama7b", 4, llama_list(32, 4096, 11008, 32000, tied=False),
                    0.02, 1e-3, 10, AdamWHP(3e-4, 0.9, 0.95, 1e-8, 0.1),
                    extra=dict(dim=4096, n_heads=32))


def initial_param_host(spec: TensorSpec, std: float, wl_index: int, t_idx: int) -> np.ndarray:
    if spec.is_norm:
        return np.ones(spec.numel, np.float32)
    return host_normal(spec.numel, std, wl_index, t_idx, 0, P0)


def initial_param_device(spec: TensorSpec, std: float, wl_index: int, t_idx: int, device):
    import torch
    if spec.is_norm:
        return torch.ones(spec.numel, dtype=torch.float32, device=device)
    return device_normal(spec.numel, std, device, wl_index, t_idx, 0, P0)
