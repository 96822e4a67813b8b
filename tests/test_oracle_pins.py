"""Pins of the CPU oracle to facts fixed outside the oracle itself.

Each test names the passage it rests on: a closed form, an invariant, a value
the pages print, a library routine (torch.optim.AdamW in float64, torch's
bf16 rounding, numpy's searchsorted) or brute force.  No GPU.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from synth import host_normal

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rel_tau(x, ref, tau):
    return np.max(np.abs(np.asarray(x, np.float64) - ref) / np.maximum(np.abs(ref), tau))


def fresh(n, seed, std_p=0.02):
    p = host_normal(n, std_p, 900, seed, 0, 0).astype(np.float64)
    return p, np.zeros(n), np.zeros(n)


def grads(n, std, seed, step):
    return host_normal(n, std, 900, seed, step, 1).astype(np.float64)


# ------------------------------------------------------------------ AdamW
@pytest.mark.parametrize("lr,wd", [(1e-3, 0.01), (0.1, 0.1), (3e-4, 0.0)])
def test_adamw_fresh_step_closed_form(orc, lr, wd):
    """bitsandbytes PR #2040, PR body: one step from zero state has the closed
    form p1 = p0*(1-lr*wd) - lr*g/(|g|+eps)."""
    n = 4096
    p, m, v = fresh(n, 1)
    p0 = p.copy()
    g = grads(n, 1e-3, 1, 0)
    orc.adamw_step(p, m, v, g, lr, 0.9, 0.999, 1e-8, wd, 1)
    expect = p0 * (1 - lr * wd) - lr * g / (np.abs(g) + 1e-8)
    assert rel_tau(p, expect, lr) < 1e-13


@pytest.mark.parametrize("lr,wd,betas", [(1e-3, 0.01, (0.9, 0.999)), (0.1, 0.1, (0.9, 0.999)),
                                         (3e-4, 0.1, (0.9, 0.95))])
def test_adamw_matches_torch_float64(orc, lr, wd, betas):
    """bitsandbytes PR #2040, second review: torch.optim.AdamW in float64 is
    the referee; the decay-first ordering agrees with it (to rounding)."""
    n, steps = 2048, 25
    p, m, v = fresh(n, 2)
    tp = torch.nn.Parameter(torch.from_numpy(p.copy()))
    opt = torch.optim.AdamW([tp], lr=lr, betas=betas, eps=1e-8, weight_decay=wd,
                            foreach=False, fused=False)
    for t in range(1, steps + 1):
        g = grads(n, 1e-2, 2, t)
        orc.adamw_step(p, m, v, g, lr, betas[0], betas[1], 1e-8, wd, t)
        tp.grad = torch.from_numpy(g.copy())
        opt.step()
    assert rel_tau(p, tp.detach().numpy(), lr) < 1e-12


def test_mutant_fails_torch_referee(orc):
    """Same referee: the decay-after ordering is a different algorithm (gap
    1.126e-7 at lr=1e-3, wd=0.01, 20 steps on the page), so it must fail a
    check the correct ordering passes."""
    ref = golden("decay_ordering_bnb2040.json")["referee"]
    n, lr, wd = 4096, ref["lr"], ref["wd"]
    p, m, v = fresh(n, 3)
    pm, mm, vm = p.copy(), m.copy(), v.copy()
    tp = torch.nn.Parameter(torch.from_numpy(p.copy()))
    opt = torch.optim.AdamW([tp], lr=lr, eps=1e-8, weight_decay=wd, foreach=False)
    for t in range(1, ref["steps"] + 1):
        g = grads(n, 1e-3, 3, t)
        orc.adamw_step(p, m, v, g, lr, 0.9, 0.999, 1e-8, wd, t)
        orc.mutant_adamw_decay_after_step(pm, mm, vm, g, lr, 0.9, 0.999, 1e-8, wd, t)
        tp.grad = torch.from_numpy(g.copy())
        opt.step()
    t_ref = tp.detach().numpy()
    gap_correct = np.max(np.abs(p - t_ref))
    gap_mutant = np.max(np.abs(pm - t_ref))
    assert gap_correct < 1e-15
    # same order of magnitude as the page's 1.126e-07 (harness differs)
    assert ref["decay_after_vs_torch"] / 4 < gap_mutant < ref["decay_after_vs_torch"] * 4


def test_orderings_coincide_at_zero_wd(orc):
    """PR body 'This changes results': runs with weight_decay = 0 are unaffected."""
    n = 1024
    p, m, v = fresh(n, 4)
    pm, mm, vm = p.copy(), m.copy(), v.copy()
    for t in range(1, 11):
        g = grads(n, 1e-2, 4, t)
        orc.adamw_step(p, m, v, g, 0.1, 0.9, 0.999, 1e-8, 0.0, t)
        orc.mutant_adamw_decay_after_step(pm, mm, vm, g, 0.1, 0.9, 0.999, 1e-8, 0.0, t)
    assert np.array_equal(p, pm)


def test_one_step_gap_identity(orc):
    """Second review, one-step algebra: from a common state the orderings
    differ by exactly step_size*update*lr*wd."""
    n, lr, wd = 2048, 0.05, 0.1
    p, m, v = fresh(n, 5)
    for t in range(1, 6):
        orc.adamw_step(p, m, v, grads(n, 1e-2, 5, t), lr, 0.9, 0.999, 1e-8, wd, t)
    g = grads(n, 1e-2, 5, 6)
    a = (p.copy(), m.copy(), v.copy())
    b = (p.copy(), m.copy(), v.copy())
    orc.adamw_step(*a, g, lr, 0.9, 0.999, 1e-8, wd, 6)
    orc.mutant_adamw_decay_after_step(*b, g, lr, 0.9, 0.999, 1e-8, wd, 6)
    # update u = m_hat/denom from the new moments (same in both)
    bc1, bc2 = 1 - 0.9 ** 6, 1 - 0.999 ** 6
    u = (a[1] / bc1) / (np.sqrt(a[2] / bc2) + 1e-8)
    assert np.allclose(b[0] - a[0], lr * u * lr * wd, rtol=1e-9, atol=1e-18)


def test_gap_scales_as_lr_squared(orc):
    """Second review, gap-vs-lr table: a hundredfold per tenfold in lr."""
    gold = golden("decay_ordering_bnb2040.json")["gap_vs_lr"]
    n, wd = 4096, gold["wd"]
    gaps = []
    for lr in gold["lr"]:
        p, m, v = fresh(n, 6)
        pm, mm, vm = p.copy(), m.copy(), v.copy()
        for t in range(1, gold["steps"] + 1):
            g = grads(n, 1e-3, 6, t)
            orc.adamw_step(p, m, v, g, lr, 0.9, 0.999, 1e-8, wd, t)
            orc.mutant_adamw_decay_after_step(pm, mm, vm, g, lr, 0.9, 0.999, 1e-8, wd, t)
        gaps.append(np.max(np.abs(p - pm)))
    ours = np.array(gaps[1:]) / np.array(gaps[:-1])
    page = np.array(gold["gap"][1:]) / np.array(gold["gap"][:-1])
    assert np.all(np.abs(ours - page) / page < 0.05), (ours, page)


def test_fresh_step_gap_lr01_wd01(orc):
    """PR body: at lr=0.1, wd=0.1 a fresh step leaves the orderings 1.0e-3 apart."""
    gold = golden("decay_ordering_bnb2040.json")["fresh_step"]
    n = 4096
    p, m, v = fresh(n, 7)
    pm, mm, vm = p.copy(), m.copy(), v.copy()
    g = grads(n, 1e-2, 7, 1)
    orc.adamw_step(p, m, v, g, gold["lr"], 0.9, 0.999, 1e-8, gold["wd"], 1)
    orc.mutant_adamw_decay_after_step(pm, mm, vm, g, gold["lr"], 0.9, 0.999, 1e-8, gold["wd"], 1)
    gap = np.max(np.abs(p - pm))
    assert abs(gap - gold["ordering_gap"]) / gold["ordering_gap"] < 0.01


def test_adamw_constant_gradient_closed_form(orc):
    """Bias correction at t > 1: with a constant gradient c, m_hat = c and
    v_hat = c^2 exactly, so u = c/(|c|+eps) every step and
    p_T = (1-a)^T p0 - lr*u*(1-(1-a)^T)/a with a = lr*wd (geometric series)."""
    n, lr, wd, T = 1024, 0.01, 0.1, 40
    p, m, v = fresh(n, 8)
    p0 = p.copy()
    c = grads(n, 1e-2, 8, 0)
    for t in range(1, T + 1):
        orc.adamw_step(p, m, v, c, lr, 0.9, 0.99, 1e-8, wd, t)
    a = lr * wd
    u = c / (np.abs(c) + 1e-8)
    expect = (1 - a) ** T * p0 - lr * u * (1 - (1 - a) ** T) / a
    assert rel_tau(p, expect, lr) < 1e-12


# ------------------------------------------------------------------ AdEMAMix
def test_ademamix_fresh_step_closed_form(orc):
    """PR body: on a fresh step AdEMAMix adds alpha*(1-beta3)*g to AdamW's
    update: p1 = p0(1-lr*wd) - lr*(1+alpha*(1-beta3))*g/(|g|+eps)."""
    n, lr, wd, a, b3 = 4096, 0.1, 0.1, 5.0, 0.9999
    p, m1, nu = fresh(n, 9)
    m2 = np.zeros(n)
    p0 = p.copy()
    g = grads(n, 1e-2, 9, 1)
    orc.ademamix_step(p, m1, m2, nu, g, lr, 0.9, 0.999, b3, a, 1e-8, wd, 1)
    expect = p0 * (1 - lr * wd) - lr * (1 + a * (1 - b3)) * g / (np.abs(g) + 1e-8)
    assert rel_tau(p, expect, lr) < 1e-13


def test_ademamix_alpha_zero_is_adamw(orc):
    n, lr, wd = 2048, 0.1, 0.1
    p, m, v = fresh(n, 10)
    q, m1, nu = p.copy(), m.copy(), v.copy()
    m2 = np.zeros(n)
    for t in range(1, 21):
        g = grads(n, 1e-2, 10, t)
        orc.adamw_step(p, m, v, g, lr, 0.9, 0.999, 1e-8, wd, t)
        orc.ademamix_step(q, m1, m2, nu, g, lr, 0.9, 0.999, 0.9999, 0.0, 1e-8, wd, t)
    assert rel_tau(q, p, lr) < 1e-13


def test_ademamix_constant_gradient_slow_ema(orc):
    """With a constant gradient c: m1_hat = c, sqrt(nu_hat) = |c| and the slow
    EMA, not bias-corrected, is m2_t = (1-beta3^t) c, so
    u_t = (1 + alpha*(1-beta3^t)) c/(|c|+eps)."""
    n, lr, wd, a, b3, T = 512, 0.01, 0.1, 5.0, 0.99, 30
    p, m1, nu = fresh(n, 11)
    m2 = np.zeros(n)
    expect = p.copy()
    c = grads(n, 1e-2, 11, 0)
    for t in range(1, T + 1):
        orc.ademamix_step(p, m1, m2, nu, c, lr, 0.9, 0.999, b3, a, 1e-8, wd, t)
        u = (1 + a * (1 - b3 ** t)) * c / (np.abs(c) + 1e-8)
        expect = expect * (1 - lr * wd) - lr * u
    assert rel_tau(p, expect, lr) < 1e-12
    assert np.allclose(m2, (1 - b3 ** T) * c, rtol=1e-12)


# ------------------------------------------------------------------ Adam-mini
def test_adam_mini_fresh_step_closed_form(orc):
    """Adam-mini <> DTensor, AdamWMini: at t=1 h = sqrt(mean_block(g^2)) + eps,
    m_hat = g, so p1 = p0(1-lr*wd) - lr*g/(RMS_block(g)+eps)."""
    rows, H, lr, wd = 8, 256, 3e-4, 0.1
    n = rows * H
    p, m, _ = fresh(n, 12)
    V = np.zeros(rows)
    p0 = p.copy()
    g = grads(n, 1e-3, 12, 1) * np.repeat(np.arange(1, rows + 1), H)  # distinct row scales
    orc.adam_mini_step(p, m, V, g, H, lr, 0.9, 0.95, 1e-8, wd, 1)
    rms = np.sqrt(np.mean(g.reshape(rows, H) ** 2, axis=1))
    expect = p0 * (1 - lr * wd) - lr * g / (np.repeat(rms, H) + 1e-8)
    assert rel_tau(p, expect, lr) < 1e-13


def test_adam_mini_block_one_is_adamw(orc):
    """head_numel = 1 gives every element its own v: plain AdamW."""
    n, lr, wd = 1024, 3e-4, 0.1
    p, m, v = fresh(n, 13)
    q, mq = p.copy(), m.copy()
    V = np.zeros(n)
    for t in range(1, 21):
        g = grads(n, 1e-3, 13, t)
        orc.adamw_step(p, m, v, g, lr, 0.9, 0.95, 1e-8, wd, t)
        orc.adam_mini_step(q, mq, V, g, 1, lr, 0.9, 0.95, 1e-8, wd, t)
    assert rel_tau(q, p, lr) < 1e-12


def test_adam_mini_constant_magnitude_rows_is_adamw(orc):
    """If every element of a block has the same |g| at every step, the block
    mean of g^2 equals each g^2, so Adam-mini equals AdamW.  Rows (blocks) get
    different magnitudes, columns do not, so a transposed block view fails."""
    rows, H, lr, wd = 16, 128, 3e-4, 0.1
    n = rows * H
    p, m, v = fresh(n, 14)
    q, mq = p.copy(), m.copy()
    V = np.zeros(rows)
    rng = np.random.default_rng(14)
    for t in range(1, 31):
        mag = np.repeat(rng.uniform(1e-4, 1e-2, rows), H)
        g = mag * rng.choice([-1.0, 1.0], n)
        orc.adamw_step(p, m, v, g, lr, 0.9, 0.95, 1e-8, wd, t)
        orc.adam_mini_step(q, mq, V, g, H, lr, 0.9, 0.95, 1e-8, wd, t)
    assert rel_tau(q, p, lr) < 1e-12


def test_adam_mini_partition_by_name(orc):
    """AdamWMini: embed/wte/embd/lm_head/output -> full v; q/k -> per-head
    blocks; everything else -> one block; norms and ln_f take wd = 0."""
    assert orc.adam_mini_kind("tok_embeddings.weight") == orc.MINI_FULL_V
    assert orc.adam_mini_kind("output.weight") == orc.MINI_FULL_V
    assert orc.adam_mini_kind("lm_head.weight") == orc.MINI_FULL_V
    assert orc.adam_mini_kind("layers.3.attention.wq.weight") == orc.MINI_HEAD
    assert orc.adam_mini_kind("model.layers.0.self_attn.k_proj.weight") == orc.MINI_HEAD
    assert orc.adam_mini_kind("layers.3.attention.wv.weight") == orc.MINI_SCALAR
    assert orc.adam_mini_kind("layers.3.feed_forward.w1.weight") == orc.MINI_SCALAR
    assert orc.adam_mini_weight_decay("layers.0.attention_norm.weight", 0.1) == 0.0
    assert orc.adam_mini_weight_decay("transformer.ln_f.weight", 0.1) == 0.0
    assert orc.adam_mini_weight_decay("layers.0.attention.wq.weight", 0.1) == 0.1


# ------------------------------------------------------------------ AMP
def test_nonfinite_detection(orc):
    """FusedAdam & PyTorch Lightning AMP, analysis: the fused step skips when
    found_inf is set; found_inf marks any NaN or +-Inf gradient."""
    x = np.linspace(-1e30, 1e30, 1001)
    assert not orc.any_nonfinite(x)
    for bad in (np.inf, -np.inf, np.nan):
        y = x.copy()
        y[517] = bad
        assert orc.any_nonfinite(y)
    assert not orc.any_nonfinite(np.array([np.finfo(np.float64).max]))


# ------------------------------------------------------------------ cosine lr
def test_cosine_lr_closed_values(orc):
    """4 bit Adam should support non constant lr: lr comes from a cosine
    schedule every step.  Plain cosine: exact at k=0, K/4, K/3, K/2, K."""
    K, hi, lo = 120, 3e-4, 1e-5
    assert orc.cosine_lr(0, K, hi, lo) == np.float32(hi)
    assert orc.cosine_lr(K, K, hi, lo) == np.float32(lo)
    assert orc.cosine_lr(K + 7, K, hi, lo) == np.float32(lo)
    assert orc.cosine_lr(K // 2, K, hi, lo) == np.float32((hi + lo) / 2)
    assert orc.cosine_lr(K // 3, K, hi, lo) == np.float32(lo + (hi - lo) * 0.75)
    assert orc.cosine_lr(K // 4, K, hi, 0.0) == np.float32(hi * (2 + math.sqrt(2)) / 4)
    vals = [orc.cosine_lr(k, K, hi, lo) for k in range(K + 1)]
    assert all(a >= b for a, b in zip(vals, vals[1:]))


# ------------------------------------------------------------------ remainders
def test_remainder_exhaustive_identity(orc):
    """TransformerEngine PR #1408, description: the fp32 master is rebuilt
    from (bf16 param, int16 remainder).  Identity on all 2^32 patterns."""
    assert orc.remainder_exhaustive_failures() == 0


def test_remainder_bf16_is_nearest_rounding(orc):
    """The stored bf16 is the master rounded to nearest (torch's bf16 cast is
    the library referee) except at exact ties, which go away from zero; the
    remainder's sign is the carry."""
    rng = np.random.default_rng(15)
    u = rng.integers(0, 2 ** 32, 1 << 20, dtype=np.uint64).astype(np.uint32)
    specials = np.array([0x00000000, 0x80000000, 0x00000001, 0x80008000, 0x00008000,
                         0x3F808000, 0xBF808000, 0x7F7F7FFF, 0x3F800000], np.uint32)
    u = np.concatenate([u, specials])
    x = u.view(np.float32)
    fin = np.isfinite(x) & (np.abs(x) < 3.38e38)
    b, r = orc.remainder_split(x)
    lo = u & 0xFFFF
    tie = lo == 0x8000
    rne = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    sel = fin & ~tie
    assert np.array_equal(b[sel], rne[sel])
    away = ((u[tie] >> 16) + 1) & 0xFFFF
    assert np.array_equal(b[tie], away.astype(np.uint16))
    assert np.array_equal(r < 0, lo >= 0x8000)
    assert np.array_equal(orc.remainder_reconstruct(b, r).view(np.uint32), u)


# ------------------------------------------------------------------ quantization
def test_dynamic_map_structure(orc):
    for b in (3, 4, 7, 8):
        M = orc.dynamic_map(b)
        assert M.size == 2 ** b and M[0] == 0.0 and M[-1] == 1.0
        assert np.all(np.diff(M) > 0)
        assert M[1] == np.float32(10.0 ** -(b - 1))
        # decade e holds 2^(b-1-e) equally spaced values in (10^-(e+1), 10^-e]
        for e in range(b):
            sel = M[(M > np.float32(10.0 ** -(e + 1))) & (M <= np.float32(10.0 ** -e))]
            assert sel.size == 2 ** (b - 1 - e)
            if sel.size > 2:
                d = np.diff(sel.astype(np.float64))
                assert np.allclose(d, d[0], rtol=1e-5)


def test_dynamic_map_hand_values(orc):
    gold = golden("dynamic_map_4bit.json")
    assert np.array_equal(orc.dynamic_map(3), np.float32(gold["signed_magnitudes_b3"]))
    M4 = orc.dynamic_map(4)
    assert np.array_equal(M4[:8], np.float32(gold["unsigned_b4_first"]))
    assert np.array_equal(M4[8:], np.float32(gold["unsigned_b4_last"]))


def _threshold_index_np(T, a):
    # largest j >= 1 with T[j] <= a, else 0 (numpy searchsorted as referee)
    return np.searchsorted(T[1:], a, side="right")


@pytest.mark.parametrize("b", [3, 4, 7, 8])
def test_quantizer_threshold_rule_near_every_threshold(orc, b):
    """Every fp32 within 64 ulps of every threshold, plus a stride over [0,1]:
    the oracle's index equals numpy.searchsorted on the same thresholds, and
    away from midpoints it is the nearest code (brute force)."""
    M = orc.dynamic_map(b)
    T = orc.thresholds(M)
    tb = T[1:].view(np.int32).astype(np.int64)
    near = (tb[:, None] + np.arange(-64, 65)[None, :]).ravel()
    stride = np.arange(0, 0x3F800001, 4099, dtype=np.int64)
    bits = np.unique(np.concatenate([near, stride, [0x3F800000]])).astype(np.int32)
    a = bits.view(np.float32)
    a = a[(a >= 0) & (a <= 1)]
    # blocks whose absmax is exactly 1.0 make the normalisation exact (r = 1)
    blk = 128
    pad = (-a.size) % (blk - 1)
    a = np.concatenate([a, np.zeros(pad, np.float32)]).reshape(-1, blk - 1)
    x = np.concatenate([a, np.ones((a.shape[0], 1), np.float32)], axis=1).ravel()
    codes, absmax = orc.quantize(x, blk, b, signed=False)
    assert np.all(absmax == 1.0)
    assert np.array_equal(codes.astype(np.int64), _threshold_index_np(T, x))
    # brute-force nearest magnitude, ties to the larger; skip points within an
    # fp32 ulp of a midpoint (where the fp32 threshold decides)
    d = np.abs(M.astype(np.float64)[None, :] - x.astype(np.float64)[:, None])
    nearest = M.size - 1 - np.argmin(d[:, ::-1], axis=1)
    mids = (M[1:].astype(np.float64) + M[:-1]) / 2
    dist = np.min(np.abs(x.astype(np.float64)[:, None] - mids[None, :]), axis=1)
    ok = dist > 2 * np.spacing(np.float32(1.0))
    assert np.array_equal(codes[ok], nearest[ok])


def test_zero_state_quantizes_exactly(orc):
    """bitsandbytes PR #2040, PR body: a fresh optimizer's zero state
    quantizes exactly."""
    for bits, blk in ((8, 256), (4, 128)):
        for signed in (True, False):
            mb = bits - 1 if signed else bits
            codes, am = orc.quantize(np.zeros(1000, np.float32), blk, mb, signed)
            assert not codes.any() and not am.any()
            assert not orc.dequantize(codes, am, blk, mb, signed).any()


def test_absmax_element_roundtrips(orc):
    x = host_normal(256 * 64, 1e-3, 901, 0, 0, 0)
    for mb, signed in ((7, True), (8, False), (3, True), (4, False)):
        xx = x if signed else np.abs(x)
        codes, am = orc.quantize(xx, 256, mb, signed)
        back = orc.dequantize(codes, am, 256, mb, signed).reshape(-1, 256)
        blocks = xx.reshape(-1, 256)
        j = np.argmax(np.abs(blocks), axis=1)
        rows = np.arange(blocks.shape[0])
        assert np.array_equal(back[rows, j], blocks[rows, j])


def test_nibble_packing_layout(orc):
    codes = np.array([1, 2, 3, 15, 0], np.uint8)
    packed = orc.pack_nibbles(codes)
    assert packed.tolist() == [0x21, 0xF3, 0x00]
    assert orc.unpack_nibbles(packed, 5).tolist() == codes.tolist()


@pytest.mark.parametrize("bits,block", [(8, 256), (4, 128)])
def test_blockwise_fresh_step(orc, bits, block):
    """PR body: one step from a fresh optimizer; the zero state dequantizes to
    zero, m = fl32(c1*g) and the update is within fp32 rounding of the closed
    form -lr*g/(|g|+eps).  At lr=0.1, wd=0.1 the decay-after ordering sits
    1.0e-3 away, far outside that agreement."""
    n, lr, wd = block * 40, 0.1, 0.1
    p = host_normal(n, 0.02, 902, bits, 0, 0).astype(np.float64)
    p0 = p.copy()
    g = host_normal(n, 1e-3, 902, bits, 1, 1)
    qm = np.zeros(n, np.uint8)
    qv = np.zeros(n, np.uint8)
    am = np.zeros(n // block, np.float32)
    av = np.zeros(n // block, np.float32)
    sm, sv = orc.blockwise_step(p, g, qm, qv, am, av, bits, block, lr, 0.9, 0.999, 1e-8, wd, 1)
    gd = g.astype(np.float64)
    assert np.array_equal(sm, np.float32(np.float32(0.1) * g))  # c1 = fl32(0.1)
    expect = p0 * (1 - lr * wd) - lr * gd / (np.abs(gd) + 1e-8)
    assert rel_tau(p, expect, lr) < 2e-6
    mutant = (p0 - lr * gd / (np.abs(gd) + 1e-8)) * (1 - lr * wd)
    assert np.max(np.abs(p - mutant)) > 0.9e-3
    # the codes are those of the fresh fp32 states
    c_m, a_m = orc.quantize(sm, block, bits - 1, True)
    assert np.array_equal(c_m, qm) and np.array_equal(a_m, am)
    assert np.array_equal(am, np.max(np.abs(sm).reshape(-1, block), axis=1))


# ------------------------------------------------------------------ clipping and loss scale
def test_grad_norm_library_and_closed_form(orc):
    """FusedAdam & PyTorch Lightning AMP: clipping is folded into the fused
    step, so the norm is that of the unscaled gradients G*s over the whole
    list.  Referee: torch.linalg.vector_norm in float64; closed form: a
    constant list of N entries c has norm |c| sqrt(N)."""
    gs = [host_normal(n, 1.0, 903, 0, i, 1).astype(np.float64) * 65536.0 for i, n in enumerate((5, 4097, 300))]
    s = 2.0 ** -16
    ref = torch.linalg.vector_norm(torch.cat([torch.from_numpy(g * s) for g in gs])).item()
    assert abs(orc.grad_norm(gs, s) - ref) <= 1e-14 * ref
    assert orc.grad_norm([np.full(7, -3.0), np.full(9, -3.0)], 0.25) == 0.75 * 4.0
    assert orc.grad_norm([np.zeros(5)], 1.0) == 0.0


@pytest.mark.parametrize("max_norm", [0.05, 1.0, 1e6])
def test_clip_matches_torch_clip_grad_norm(orc, max_norm):
    """Referee: torch.nn.utils.clip_grad_norm_ (float64) on the unscaled
    gradients; the oracle's coefficient times G*s gives the same gradients,
    and its returned total norm is the oracle's norm."""
    gs = [host_normal(n, 1e-2, 904, 1, i, 1).astype(np.float64) * 1024.0 for i, n in enumerate((100, 33, 2048))]
    s = 1.0 / 1024.0
    params = [torch.nn.Parameter(torch.zeros(g.size, dtype=torch.float64)) for g in gs]
    for p, g in zip(params, gs):
        p.grad = torch.from_numpy(g * s)
    total = torch.nn.utils.clip_grad_norm_(params, max_norm).item()
    norm = orc.grad_norm(gs, s)
    assert abs(norm - total) <= 1e-14 * total
    c = orc.clip_coef(norm, max_norm)
    assert (c == 1.0) == (max_norm >= norm)
    for p, g in zip(params, gs):
        assert np.allclose(g * s * c, p.grad.numpy(), rtol=1e-14, atol=0)  # torch: norm of per-tensor norms


def test_clip_coef_special_cases(orc):
    assert orc.clip_coef(5.0, 0.0) == 1.0          # no clipping requested
    assert orc.clip_coef(5.0, float("inf")) == 1.0
    assert orc.clip_coef(float("inf"), 1.0) == 1.0  # step skipped anyway
    assert orc.clip_coef(float("nan"), 1.0) == 1.0
    assert orc.clip_coef(0.0, 1.0) == 1.0
    assert orc.clip_coef(4.0, 2.0) == 2.0 / (4.0 + 1e-6)


def test_scaler_update_matches_torch(orc):
    """Referee: torch._amp_update_scale_ on CPU float32 (GradScaler's update)
    over a fixed pattern of clean and overflowing steps, including growth to
    +inf (not applied) and backoff from a large scale: scale and count equal
    after every iteration, bit for bit."""
    pattern = [0, 0, 0, 1, 0, 0, 0, 0, 0, 0, 1, 1, 0, 0, 0, 0, 0, 0, 0, 0]
    for scale0, growth, backoff, interval in ((65536.0, 2.0, 0.5, 3), (2.0 ** 126, 2.0, 0.5, 2),
                                               (3.0, 1.7, 0.3, 1)):
        st = orc.ScalerState(scale0)
        ts = torch.tensor([scale0], dtype=torch.float32)
        tg = torch.tensor([0], dtype=torch.int32)
        for f in pattern:
            st.update(bool(f), growth, backoff, interval)
            torch._amp_update_scale_(ts, tg, torch.tensor([float(f)]), growth, backoff, interval)
            assert st.scale.view(np.uint32)[0] == ts.numpy().view(np.uint32)[0], (scale0, f)
            assert st.tracker[0] == tg.item()


def test_scaler_update_closed_form(orc):
    """k clean steps from scale S0 with interval N and growth 2 give
    S0 * 2^floor(k/N) and count k mod N; one overflow halves the scale and
    resets the count."""
    st = orc.ScalerState(1024.0)
    for k in range(1, 26):
        st.update(False, 2.0, 0.5, 4)
        assert st.scale[0] == 1024.0 * 2 ** (k // 4) and st.tracker[0] == k % 4
    st.update(True, 2.0, 0.5, 4)
    assert st.scale[0] == 1024.0 * 2 ** 6 / 2 and st.tracker[0] == 0


# ------------------------------------------------------------------ blockwise AdEMAMix
@pytest.mark.parametrize("bits,block", [(8, 256), (4, 128)])
def test_blockwise_ademamix_fresh_step(orc, bits, block):
    """bitsandbytes PR #2040 body: a fresh 8-bit AdEMAMix step has AdamW's
    closed form plus alpha*(1-beta3)*g; zero states quantize exactly; the
    three fresh states are the fp32 products of g; the decay-after ordering
    sits 1e-3 away at lr = 0.1, wd = 0.1."""
    n, lr, wd, a, b3 = block * 40, 0.1, 0.1, 5.0, 0.9999
    p = host_normal(n, 0.02, 905, bits, 0, 0).astype(np.float64)
    p0 = p.copy()
    g = host_normal(n, 1e-3, 905, bits, 1, 1)
    q = [np.zeros(n, np.uint8) for _ in range(3)]
    ab = [np.zeros(n // block, np.float32) for _ in range(3)]
    sm, sm2, sv = orc.blockwise_ademamix_step(p, g, q[0], q[1], q[2], ab[0], ab[1], ab[2], bits, block,
                                              lr, 0.9, 0.999, b3, a, 1e-8, wd, 1)
    assert np.array_equal(sm, np.float32(np.float32(0.1) * g))
    assert np.array_equal(sm2, np.float32(np.float32(1.0 - b3) * g))
    assert np.array_equal(sv, np.float32(np.float32(1.0 - 0.999) * np.float32(g * g)))
    gd = g.astype(np.float64)
    k = 1 + a * (1 - b3)
    expect = p0 * (1 - lr * wd) - lr * k * gd / (np.abs(gd) + 1e-8)
    assert rel_tau(p, expect, lr) < 2e-6
    mutant = (p0 - lr * k * gd / (np.abs(gd) + 1e-8)) * (1 - lr * wd)
    assert np.max(np.abs(p - mutant)) > 0.9e-3
    for st, code, am, signed in ((sm, q[0], ab[0], True), (sm2, q[1], ab[1], True), (sv, q[2], ab[2], False)):
        c, A = orc.quantize(st, block, bits - 1 if signed else bits, signed)
        assert np.array_equal(c, code) and np.array_equal(A, am)


def _constant_magnitude_grads(nblk, block, steps, seed):
    """g[t] = mag[t, block] * sign: each element keeps its sign over time and
    every element of a block has the same magnitude at every step."""
    rng = np.random.default_rng(seed)
    sign = rng.choice([-1.0, 1.0], nblk * block)
    for _ in range(steps):
        yield (np.repeat(rng.uniform(1e-4, 1e-2, nblk), block) * sign).astype(np.float32)


@pytest.mark.parametrize("bits,block", [(8, 256), (4, 128)])
def test_blockwise_constant_magnitude_blocks_track_adamw(orc, bits, block):
    """With the gradients above every element of a block has the same |m|
    and the same v at every step, so each normalised magnitude is the map's
    largest value, 1, held exactly: the quantized states carry no error and
    the blockwise step follows AdamW (pinned to torch in float64 above) over
    30 steps, up to the fp32 state recipe.  A block boundary off by one
    element, a wrong bias correction after step 1 or a dropped state update
    breaks it."""
    nblk, lr, wd, steps = 12, 1e-3, 0.1, 30
    n = nblk * block
    p = host_normal(n, 0.02, 907, bits, 0, 0).astype(np.float64)
    q, m, v = p.copy(), np.zeros(n), np.zeros(n)
    qm, qv = np.zeros(n, np.uint8), np.zeros(n, np.uint8)
    am, av = np.zeros(nblk, np.float32), np.zeros(nblk, np.float32)
    for t, g in enumerate(_constant_magnitude_grads(nblk, block, steps, 907 + bits), start=1):
        orc.adamw_step(p, m, v, g.astype(np.float64), lr, 0.9, 0.999, 1e-8, wd, t)
        orc.blockwise_step(q, g, qm, qv, am, av, bits, block, lr, 0.9, 0.999, 1e-8, wd, t)
        assert rel_tau(q, p, lr) < 1e-5, t
    top = (1 << (bits - 1)) - 1  # the signed map's largest magnitude code
    assert set(np.unique(qm & top).tolist()) == {top} and set(np.unique(qv).tolist()) == {(1 << bits) - 1}


@pytest.mark.parametrize("bits,block", [(8, 256), (4, 128)])
def test_blockwise_ademamix_constant_magnitude_blocks_track_ademamix(orc, bits, block):
    """The same construction for the three AdEMAMix states (m1, m2, nu all
    exact): the blockwise AdEMAMix step follows the fp64 AdEMAMix step
    (pinned by its fresh-step and constant-gradient closed forms and by
    alpha = 0 being AdamW) over 30 steps."""
    nblk, lr, wd, b3, a, steps = 12, 1e-3, 0.1, 0.9999, 5.0, 30
    n = nblk * block
    p = host_normal(n, 0.02, 908, bits, 0, 0).astype(np.float64)
    r, m1, m2, nu = p.copy(), np.zeros(n), np.zeros(n), np.zeros(n)
    q = [np.zeros(n, np.uint8) for _ in range(3)]
    ab = [np.zeros(nblk, np.float32) for _ in range(3)]
    for t, g in enumerate(_constant_magnitude_grads(nblk, block, steps, 909 + bits), start=1):
        orc.ademamix_step(p, m1, m2, nu, g.astype(np.float64), lr, 0.9, 0.999, b3, a, 1e-8, wd, t)
        orc.blockwise_ademamix_step(r, g, q[0], q[1], q[2], ab[0], ab[1], ab[2], bits, block, lr, 0.9, 0.999,
                                    b3, a, 1e-8, wd, t)
        assert rel_tau(r, p, lr) < 1e-5, t


def test_blockwise_ademamix_alpha_zero_is_blockwise_adamw(orc):
    """alpha = 0 takes m2 out of the update: the m and nu codes and absmax
    equal the 2-state blockwise AdamW step's bit for bit over several steps,
    and p agrees to fp64 rounding (lr (m/bc1)/h against (lr/bc1) m/h)."""
    n, block, bits = 256 * 12 + 77, 256, 8
    p = host_normal(n, 0.02, 906, 0, 0, 0).astype(np.float64)
    pa = p.copy()
    q = [np.zeros(n, np.uint8) for _ in range(3)]
    ab = [np.zeros((n + block - 1) // block, np.float32) for _ in range(3)]
    qa = [np.zeros(n, np.uint8) for _ in range(2)]
    aa = [np.zeros((n + block - 1) // block, np.float32) for _ in range(2)]
    for t in range(1, 8):
        g = host_normal(n, 1e-3, 906, 0, t, 1)
        orc.blockwise_ademamix_step(p, g, q[0], q[1], q[2], ab[0], ab[1], ab[2], bits, block,
                                    1e-3, 0.9, 0.999, 0.9999, 0.0, 1e-8, 0.01, t)
        orc.blockwise_step(pa, g, qa[0], qa[1], aa[0], aa[1], bits, block, 1e-3, 0.9, 0.999, 1e-8, 0.01, t)
        assert rel_tau(p, pa, 1e-3) < 1e-13
        assert np.array_equal(q[0], qa[0]) and np.array_equal(q[2], qa[1])
        assert np.array_equal(ab[0], aa[0]) and np.array_equal(ab[2], aa[1])


# ------------------------------------------------------------------ Lion
def test_lion_constant_gradient_closed_form(orc):
    """With a constant gradient the interpolation c keeps the gradient's sign,
    so each step moves p by exactly lr against it after the decay:
    p_T = (1-a)^T p0 - lr sign(g) (1-(1-a)^T)/a, a = lr wd (decay first, as
    the bitsandbytes PR review describes Lion); sign(0) = 0 leaves pure decay."""
    n, lr, wd, T = 1000, 1e-3, 0.1, 25
    p = host_normal(n, 0.02, 907, 0, 0, 0).astype(np.float64)
    p0 = p.copy()
    g = host_normal(n, 1e-3, 907, 0, 0, 1)
    g[::10] = 0.0
    m = np.zeros(n, np.float32)
    for _ in range(T):
        orc.lion_step(p, m, g, lr, 0.9, 0.99, wd)
    a = lr * wd
    s = np.sign(g).astype(np.float64)  # not float32: lr would round to fp32
    expect = (1 - a) ** T * p0 - lr * s * (1 - (1 - a) ** T) / a
    assert rel_tau(p, expect, lr) < 1e-11
    assert np.all(m[::10] == 0.0)


def test_lion_reversal_follows_the_interpolation(orc):
    """Hand-worked two steps (lr 0.1, wd 0, beta1 0.9, beta2 0.99): g = +1
    moves p to -0.1 and leaves m = fl32(0.01); then g = -0.085 gives
    c = 0.9 m + 0.1 g = +0.0005 > 0, so p moves on to -0.2 although the
    gradient turned (updating m first, or using beta2 for c, or the sign of
    g, would move it back to 0); m = 0.99 m + 0.01 g = 0.00905."""
    p = np.zeros(1)
    m = np.zeros(1, np.float32)
    orc.lion_step(p, m, np.array([1.0], np.float32), 0.1, 0.9, 0.99, 0.0)
    assert p[0] == -0.1 and m[0] == np.float32(0.01)
    orc.lion_step(p, m, np.array([-0.085], np.float32), 0.1, 0.9, 0.99, 0.0)
    assert p[0] == -0.2
    assert abs(m[0] - 0.00905) < 1e-9
    # a larger reversal, g = -0.2: c = 0.009 - 0.02 < 0 turns p back to 0
    # (beta2 in the interpolation, 0.0099 - 0.002 > 0, would not)
    p, m = np.zeros(1), np.zeros(1, np.float32)
    for g in (1.0, -0.2):
        orc.lion_step(p, m, np.array([g], np.float32), 0.1, 0.9, 0.99, 0.0)
    assert abs(p[0]) < 1e-17 and abs(m[0] - 0.0079) < 1e-9


# ------------------------------------------------------------------ LAMB
@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_lamb_step_norm_is_lr_times_param_norm(orc, wd):
    """LAMB's layer-wise normalisation: ||p_new - p|| = lr ||p|| on every step
    (trust ratio ||p||/||u|| times the update u), here over 6 steps."""
    n, lr = 3000, 1e-2
    p = host_normal(n, 0.02, 908, 0, 0, 0).astype(np.float64)
    m, v = np.zeros(n), np.zeros(n)
    for t in range(1, 7):
        prev = p.copy()
        orc.lamb_step(p, m, v, grads(n, 1e-3, 8, t), lr, 0.9, 0.999, 1e-6, wd, t)
        assert abs(np.linalg.norm(p - prev) - lr * np.linalg.norm(prev)) <= 1e-12 * lr * np.linalg.norm(prev)


def test_lamb_fresh_step_direction(orc):
    """From zero moments the bias-corrected direction is g/(|g|+eps), so the
    first step is parallel to g/(|g|+eps) + wd p0 (cosine 1); a zero
    parameter has trust ratio 1 and takes Adam's fresh step -lr g/(|g|+eps)."""
    n, lr, wd, eps = 2048, 1e-2, 0.1, 1e-6
    p = host_normal(n, 0.02, 909, 0, 0, 0).astype(np.float64)
    p0 = p.copy()
    g = grads(n, 1e-3, 9, 1)
    orc.lamb_step(p, np.zeros(n), np.zeros(n), g, lr, 0.9, 0.999, eps, wd, 1)
    u = g / (np.abs(g) + eps) + wd * p0
    d = p0 - p
    assert abs(d @ u / (np.linalg.norm(d) * np.linalg.norm(u)) - 1.0) < 1e-12
    z = np.zeros(n)
    orc.lamb_step(z, np.zeros(n), np.zeros(n), g, lr, 0.9, 0.999, eps, wd, 1)
    assert np.allclose(z, -lr * g / (np.abs(g) + eps), rtol=1e-13, atol=0)


def test_lamb_scale_equivariance(orc):
    """Without decay the update scales with the parameter: stepping c*p0
    gives c times the step of p0 (the trust ratio carries ||p||)."""
    n, lr = 1500, 1e-2
    p = host_normal(n, 0.02, 910, 0, 0, 0).astype(np.float64)
    q = 8.0 * p
    ma, va, mb, vb = np.zeros(n), np.zeros(n), np.zeros(n), np.zeros(n)
    for t in range(1, 5):
        g = grads(n, 1e-3, 10, t)
        orc.lamb_step(p, ma, va, g, lr, 0.9, 0.999, 1e-6, 0.0, t)
        orc.lamb_step(q, mb, vb, g, lr, 0.9, 0.999, 1e-6, 0.0, t)
    assert rel_tau(q, 8.0 * p, 1e-3) < 1e-13


# ------------------------------------------------------------------ low-precision model copy
def _patterns():
    """Every high half of the fp32 pattern with the low halves that decide
    rounding (exact, below / at / above the bf16 and the fp16 halfway
    points, odd and even kept bits), plus random patterns."""
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0x0000, 0x0001, 0x0FFF, 0x1000, 0x1001, 0x2000, 0x3000, 0x7FFF, 0x8000, 0x8001,
                     0xA000, 0xFFFF], np.uint32)
    grid = (hi[:, None] | lows[None, :]).ravel()
    rnd = np.random.default_rng(911).integers(0, 1 << 32, 1 << 20, dtype=np.uint64).astype(np.uint32)
    return np.concatenate([grid, rnd])


def test_model_copy_bf16_is_torch_rne(orc):
    """Transformer Engine remainder page, review thread: with master weights
    the model copy is the fp32 master rounded to the model dtype.  Referee:
    torch's float32 -> bfloat16 cast (round to nearest even); NaNs stay NaN."""
    u = _patterns()
    x = u.view(np.float32)
    got = orc.round_model_copy(x, half=False)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all(got[nan] & 0x007F)


def test_model_copy_f16_is_numpy_rne(orc):
    """Referee: numpy's float32 -> float16 cast (IEEE round to nearest even,
    overflow to inf, gradual underflow), on the same patterns."""
    u = _patterns()
    x = u.view(np.float32)
    got = orc.round_model_copy(x, half=True)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all(np.isnan(got[nan].view(np.float16)))
    # hand-worked: 65520 is the halfway point to 2^16 (rounds to inf), the
    # smallest subnormal 2^-24 and half of it (a tie to even: zero)
    assert orc.round_model_copy(np.float32([65504.0, 65519.0, 65520.0]), True).tolist() == [0x7BFF, 0x7BFF, 0x7C00]
    assert orc.round_model_copy(np.float32([2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -25]), True).tolist() == [1, 0, 1]


# ------------------------------------------------------------------ scaled 16-bit moments
def _scaled_run(orc, half, steps, n=3000, key=0):
    p = host_normal(n, 0.02, 912, key, 0, 0).astype(np.float64)
    q = p.copy()
    qm, qv = np.zeros(n, np.uint16), np.zeros(n, np.uint16)
    sm, sv = np.ones(1, np.float32), np.ones(1, np.float32)
    m, v = np.zeros(n), np.zeros(n)
    out = []
    for t in range(1, steps + 1):
        g = host_normal(n, 1e-3, 912, key, t, 1)
        m32, v32 = orc.adamw_scaled_step(p, qm, qv, sm, sv, g, half, 1e-3, 0.9, 0.999, 1e-8, 0.1, t)
        orc.adamw_step(q, m, v, g.astype(np.float64), 1e-3, 0.9, 0.999, 1e-8, 0.1, t)
        out.append((m32, v32))
    return p, q, qm, qv, sm, sv, out


def _h(bits, half):
    return bits.view(np.float16).astype(np.float64) if half else orc_bf16(bits)


def orc_bf16(bits):
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("half", [True, False])
def test_scaled_states_fresh_step(orc, half):
    """Transformer Engine page, review thread (state scaling: stored * scale
    is the fp32 state; the new state is value * rscale copied into the
    low-precision tensor).  From zero states the fp32 moments are the fresh
    products of g and the update is AdamW's (the states used are fp32); fp16
    states put the tensor's largest |m| on 65504 with scale = amax/65504,
    bf16 states keep scale 1 and are the moments rounded to nearest even."""
    p, q, qm, qv, sm, sv, out = _scaled_run(orc, half, 1)
    m32, v32 = out[0]
    assert rel_tau(p, q, 1e-3) < 2e-6
    for bits, s, st in ((qm, sm, m32), (qv, sv, v32)):
        if half:
            assert np.max(np.abs(bits.view(np.float16).astype(np.float64))) == 65504.0
            assert s[0] == np.float32(np.float64(np.max(np.abs(st))) / 65504.0)
        else:
            assert s[0] == 1.0 and np.array_equal(bits, orc.round_model_copy(st, False))


@pytest.mark.parametrize("half", [True, False])
def test_scaled_states_round_trip_precision(orc, half):
    """stored * scale reproduces every moment that is not tiny against the
    tensor's largest to the 16-bit format's half-ulp (2^-11 fp16, 2^-8 bf16)."""
    _, _, qm, qv, sm, sv, out = _scaled_run(orc, half, 3)
    m32, v32 = out[-1]
    tol = 2.0 ** -11 if half else 2.0 ** -8
    for bits, s, st in ((qm, sm, m32), (qv, sv, v32)):
        back = np.float32(_h(bits, half) * np.float64(s[0]))
        big = np.abs(st) >= np.max(np.abs(st)) * 2.0 ** -12
        rel = np.abs(back[big].astype(np.float64) - st[big]) / np.abs(st[big])
        assert np.max(rel) <= tol * (1 + 1e-6)


def test_scaled_fp16_states_track_fp32_adamw(orc):
    """Over 20 steps the fp16-state trajectory stays close to fp32-state
    AdamW (relerr_tau 5.3e-3: the smallest second moments sit in fp16's
    subnormal range after scaling); bf16 states, with 8 significant bits,
    drift several times further."""
    p16, q, *_ = _scaled_run(orc, True, 20)
    pb, qb, *_ = _scaled_run(orc, False, 20)
    e16, eb = rel_tau(p16, q, 1e-3), rel_tau(pb, qb, 1e-3)
    assert e16 < 1e-2 and e16 < eb / 4
