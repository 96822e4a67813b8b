"""GPU parity at sizes the oracle finishes in seconds: every entry point
compared element by element with the CPU oracle, on seeded inputs spanning
several work units, ragged tails, unaligned tensors and the degenerate cases
(empty lists, zero-size tensors, lr = 0, skipped steps)."""
import numpy as np
import pytest
import torch

import oracle as orc
import optimizer_step_adamw_amd as osa
from gpu_support import (DEV, TOL_RUN, TOL_STEP1, AdamState, DevScalars, QuantState, all_equal,
                         relerr_tau, say, snapshot, to_np_u16)
from synth import host_normal

pytestmark = pytest.mark.gpu

RAGGED = [1, 7, 8, 9, 4095, 4096, 4097, 10007, 65539]


def _p0(sizes, key, std=0.02):
    return [host_normal(n, std, 910, key, i, 0) for i, n in enumerate(sizes)]


def _to_dev(xs, unaligned=()):
    out = []
    for i, x in enumerate(xs):
        t = torch.from_numpy(x).to(DEV)
        if i in unaligned:  # a view 4 bytes past a 16-byte boundary
            buf = torch.empty(x.size + 1, dtype=torch.float32, device=DEV)
            buf[1:].copy_(t)
            t = buf[1:]
        out.append(t)
    return out


def _grads(sizes, key, t, std):
    return [host_normal(n, std, 911, key, i, t) for i, n in enumerate(sizes)]


def _load_grads(state, gs, scale=1.0):
    """Copy host fp32 grads to the device (bf16 grads: round x scale to bf16);
    returns the float64 values the oracle sees (after unscaling)."""
    seen = []
    for dst, g in zip(state.g, gs):
        if state.grad_bf16:
            b = torch.from_numpy(g).to(DEV).mul_(scale).to(torch.bfloat16)
            dst.copy_(b.view(torch.int16))
            seen.append(orc.bf16_bits_to_f64(to_np_u16(dst)) / scale)
        else:
            dst.copy_(torch.from_numpy(g).to(DEV))
            seen.append(g.astype(np.float64))
    return seen


def _run_adam(algo, sizes, steps, *, lr, betas=(0.9, 0.999), eps=1e-8, wd_of=None, grad_bf16=False,
              param_bf16=False, unaligned=(), beta3=0.9999, alpha=5.0, g_std=1e-2, key=0, tile=0,
              grid=0):
    wd = [wd_of(i) if wd_of else 0.01 * (i % 3) for i in range(len(sizes))]
    p0 = _p0(sizes, key)
    st = AdamState(_to_dev(p0, unaligned), grad_bf16=grad_bf16, param_bf16=param_bf16,
                   ademamix=algo == osa.OPTIM_ALGO_ADEMAMIX)
    if unaligned:  # give the unaligned tensor unaligned moments as well
        for i in unaligned:
            for lst in (st.m, st.v):
                buf = torch.zeros(sizes[i] + 1, dtype=torch.float32, device=DEV)
                lst[i] = buf[1:]
    plan = osa.Plan(st.tensor_list(wd), algo, tile=tile, grid=grid)
    sc = DevScalars(lr)
    op = [x.astype(np.float64) for x in p0]
    om = [np.zeros(n) for n in sizes]
    ov = [np.zeros(n) for n in sizes]
    om2 = [np.zeros(n) for n in sizes]
    lr32 = float(np.float32(lr))
    worst = 0.0
    for t in range(1, steps + 1):
        g = _load_grads(st, _grads(sizes, key, t, g_std))
        if algo == osa.OPTIM_ALGO_ADAMW:
            osa.optim_step_adamw(plan.handle, osa.optim_adamw_hp(*betas, eps), sc.lr, None, None, sc.step)
        else:
            osa.optim_step_ademamix(plan.handle, osa.optim_ademamix_hp(betas[0], betas[1], beta3, alpha, eps),
                                    sc.lr, None, None, sc.step)
        for i in range(len(sizes)):
            if algo == osa.OPTIM_ALGO_ADAMW:
                orc.adamw_step(op[i], om[i], ov[i], g[i], lr32, betas[0], betas[1], eps, wd[i], t)
            else:
                orc.ademamix_step(op[i], om[i], om2[i], ov[i], g[i], lr32, betas[0], betas[1], beta3,
                                  alpha, eps, wd[i], t)
        err = max(relerr_tau(st.master(i).cpu().numpy(), op[i], lr32) for i in range(len(sizes)))
        worst = max(worst, err)
        assert err <= (TOL_STEP1 if t == 1 else TOL_RUN), (t, err)
    assert int(sc.step.item()) == steps
    say(f"algo={algo} sizes={len(sizes)} steps={steps} worst relerr_tau={worst:.3e}")
    return st, plan


def test_adamw_fp32_ragged_unaligned():
    _run_adam(osa.OPTIM_ALGO_ADAMW, RAGGED, 12, lr=0.1, wd_of=lambda i: 0.1 * (i % 2),
              unaligned=(5,))


def test_adamw_bf16_grads():
    _run_adam(osa.OPTIM_ALGO_ADAMW, RAGGED, 8, lr=1e-3, grad_bf16=True, key=1)


def test_adamw_bf16_params_with_remainders():
    st, _ = _run_adam(osa.OPTIM_ALGO_ADAMW, RAGGED, 10, lr=3e-4, betas=(0.9, 0.95), grad_bf16=True,
                      param_bf16=True, key=2, g_std=1e-3)
    # the stored bf16 param is split(master) of the stored master, bit for bit
    for i in range(st.n):
        master = st.master(i).cpu().numpy()
        b, r = orc.remainder_split(master)
        assert np.array_equal(b, to_np_u16(st.p[i]))
        assert np.array_equal(r, st.r[i].cpu().numpy())


@pytest.mark.parametrize("algo,tile,grid", [(osa.OPTIM_ALGO_ADAMW, 1024, 0), (osa.OPTIM_ALGO_ADAMW, 8192, 0),
                                            (osa.OPTIM_ALGO_ADAMW, 2048, 7), (osa.OPTIM_ALGO_ADEMAMIX, 1024, 0)])
def test_launch_shapes(algo, tile, grid):
    """Smallest and larger work units and a persistent grid of 7 workgroups
    cover the same elements (full groups, single groups, ragged ends): bf16
    params with remainders and bf16 grads exercise the 16-bit accesses."""
    bf16 = algo == osa.OPTIM_ALGO_ADAMW
    _run_adam(algo, RAGGED, 4, lr=3e-4, betas=(0.9, 0.95), grad_bf16=bf16, param_bf16=bf16, g_std=1e-3,
              key=5, tile=tile, grid=grid)


# More than 2^20 elements: the default plan takes 4096-element units and the
# step its early-load form with 4 groups per lane; ragged tensors mix whole
# units (early form) and partial ones.
MID = [1 << 20, 4096 * 100 + 37, 3000]


@pytest.mark.parametrize("algo,bf16", [(osa.OPTIM_ALGO_ADAMW, True), (osa.OPTIM_ALGO_ADEMAMIX, False)])
def test_mid_size_list_early_units(algo, bf16):
    _run_adam(algo, MID, 3, lr=3e-4, betas=(0.9, 0.95), grad_bf16=bf16, param_bf16=bf16, g_std=1e-3, key=21)


@pytest.mark.parametrize("algo", [osa.OPTIM_ALGO_ADAMW, osa.OPTIM_ALGO_ADEMAMIX])
def test_launch_forms_give_the_same_bits(algo):
    """4096-element units (early form, 4 groups), 2048-element units (early
    form, 2 groups), 8192-element units and a persistent grid (no early
    loads) compute the same elementwise step: identical bits."""
    runs = [_run_adam(algo, MID, 2, lr=1e-3, key=22, tile=t, grid=g)[0]
            for t, g in ((0, 0), (2048, 0), (8192, 0), (4096, 11))]
    for st in runs[1:]:
        assert all_equal(runs[0].buffers(), st.buffers())


def test_ademamix_fp32_ragged():
    _run_adam(osa.OPTIM_ALGO_ADEMAMIX, RAGGED, 12, lr=0.1, wd_of=lambda i: 0.1, key=3)


def test_ademamix_fresh_step_closed_form():
    """bitsandbytes PR #2040 body: fresh AdEMAMix step = AdamW's closed form
    with the extra alpha*(1-beta3)*g term."""
    n, lr, wd, a, b3 = 40000, 0.1, 0.1, 5.0, 0.9999
    p0 = _p0([n], 4)
    st = AdamState(_to_dev(p0), ademamix=True)
    plan = osa.Plan(st.tensor_list([wd]), osa.OPTIM_ALGO_ADEMAMIX)
    sc = DevScalars(lr)
    g = _load_grads(st, _grads([n], 4, 1, 1e-2))[0]
    osa.optim_step_ademamix(plan.handle, osa.optim_ademamix_hp(0.9, 0.999, b3, a, 1e-8), sc.lr, None,
                            None, sc.step)
    lr32 = float(np.float32(lr))
    expect = p0[0] * (1 - lr32 * wd) - lr32 * (1 + a * (1 - b3)) * g / (np.abs(g) + 1e-8)
    assert relerr_tau(st.p[0].cpu().numpy(), expect, lr32) <= TOL_STEP1


# ------------------------------------------------------------------ Adam-mini
MINI_LIST = [("tok_embeddings.weight", 37 * 64), ("layers.0.attention.wq.weight", 64 * 64),
             ("layers.0.attention.wk.weight", 64 * 64), ("layers.0.attention.wv.weight", 64 * 64),
             ("layers.0.feed_forward.w1.weight", 172 * 64), ("layers.0.attention_norm.weight", 64),
             ("layers.1.attention.wq.weight", 64 * 64), ("big.w2.weight", 3 * 4096 + 5),
             ("norm.weight", 64), ("output.weight", 37 * 64)]


def _mini_run(steps, key, grad_bf16=False, lr=3e-4, wd=0.1, dim=64, heads=4, items=MINI_LIST, tile=0,
              segment_bytes=0, grid=0, param_bf16=False):
    names = [n for n, _ in items]
    sizes = [s for _, s in items]
    kinds, hn, wds = osa.adam_mini_partition(names, sizes, dim=dim, n_heads=heads, weight_decay=wd)
    vlen = [s if k == osa.OPTIM_MINI_FULL_V else s // h for k, s, h in zip(kinds, sizes, hn)]
    p0 = _p0(sizes, key)
    st = AdamState(_to_dev(p0), grad_bf16=grad_bf16, param_bf16=param_bf16, v_len=vlen)
    plan = osa.Plan(st.tensor_list(wds, mini_kind=kinds, head_numel=hn), osa.OPTIM_ALGO_ADAM_MINI, tile=tile,
                    segment_bytes=segment_bytes, grid=grid)
    sc = DevScalars(lr)
    lr32 = float(np.float32(lr))
    # oracle side: its own partition by name
    okind = [orc.adam_mini_kind(n) for n in names]
    owd = [orc.adam_mini_weight_decay(n, wd) for n in names]
    oblock = [dim * dim // heads if k == orc.MINI_HEAD else s for k, s in zip(okind, sizes)]
    op = [x.astype(np.float64) for x in p0]
    om = [np.zeros(s) for s in sizes]
    ov = [np.zeros(s) if k == orc.MINI_FULL_V else np.zeros(s // b) for k, s, b in zip(okind, sizes, oblock)]
    for t in range(1, steps + 1):
        g = _load_grads(st, _grads(sizes, key, t, 1e-3))
        osa.optim_step_adam_mini(plan.handle, osa.optim_adamw_hp(0.9, 0.95, 1e-8), sc.lr, None, None, sc.step)
        for i in range(len(sizes)):
            if okind[i] == orc.MINI_FULL_V:
                orc.adamw_step(op[i], om[i], ov[i], g[i], lr32, 0.9, 0.95, 1e-8, owd[i], t)
            else:
                orc.adam_mini_step(op[i], om[i], ov[i], g[i], oblock[i], lr32, 0.9, 0.95, 1e-8, owd[i], t)
        err = max(relerr_tau((st.master(i) if param_bf16 else st.p[i]).cpu().numpy(), op[i], lr32)
                  for i in range(len(sizes)))
        assert err <= (TOL_STEP1 if t == 1 else TOL_RUN), (t, err)
    return st


def test_adam_mini_small_list():
    _mini_run(10, 5)


@pytest.mark.parametrize("grad_bf16,grid,segment_bytes", [(True, 0, 0), (False, 7, 20000)])
def test_adam_mini_bf16_params_with_remainders(grad_bf16, grid, segment_bytes):
    """bf16 params + int16 remainders ([TE]: the fp32 master rebuilt
    bit-exactly) under Adam-mini's shared-v update, against the oracle on
    the reconstructed master."""
    _mini_run(6, 8, grad_bf16=grad_bf16, param_bf16=True, grid=grid, segment_bytes=segment_bytes)


def test_adam_mini_bf16_grads_and_unaligned_blocks():
    """head_numel = 25 (dim 10, 4 heads): blocks start off 16-byte boundaries."""
    items = [("layers.0.attention.wq.weight", 100), ("layers.0.attention.wk.weight", 100),
             ("layers.0.attention.wo.weight", 100), ("embed.weight", 30)]
    _mini_run(6, 6, grad_bf16=True, dim=10, heads=4, items=items)


def test_adam_mini_small_units():
    """1024-element units: a head block of 8192 (dim 128, 2 heads) spans 8
    units whose partial sums the finalize adds; ragged other tensors."""
    items = [("layers.0.attention.wq.weight", 128 * 128), ("layers.0.attention.wk.weight", 128 * 128),
             ("layers.0.feed_forward.w1.weight", 128 * 300 + 7), ("layers.0.attention_norm.weight", 128),
             ("output.weight", 5003)]
    _mini_run(5, 9, dim=128, heads=2, items=items, tile=1024)


def test_adam_mini_100_steps_two_layer_slice():
    """100 steps on a two-layer Llama-shaped slice with all three kinds: the
    embedding and output with full v, q/k with one v per head block, every
    other tensor (v/o projections, MLP, norms) with one v."""
    dim, heads, ffn, vocab = 256, 4, 688, 1000
    items = [("tok_embeddings.weight", vocab * dim)]
    for layer in range(2):
        items += [(f"layers.{layer}.attention.{w}.weight", dim * dim) for w in ("wq", "wk", "wv", "wo")]
        items += [(f"layers.{layer}.feed_forward.{w}.weight", ffn * dim) for w in ("w1", "w2", "w3")]
        items += [(f"layers.{layer}.attention_norm.weight", dim), (f"layers.{layer}.ffn_norm.weight", dim)]
    items += [("norm.weight", dim), ("output.weight", vocab * dim)]
    _mini_run(100, 11, dim=dim, heads=heads, items=items)


def test_adam_mini_deterministic():
    a = _mini_run(4, 7)
    b = _mini_run(4, 7)
    assert all_equal(a.buffers(), b.buffers())


@pytest.mark.parametrize("segment_bytes,grid", [(1, 0), (20000, 0), (20000, 5)])
def test_adam_mini_segments_match_one_segment(segment_bytes, grid):
    """The step runs its block-sum, finalize and update kernels per segment
    (consecutive shared-v tensors up to segment_bytes of gradient, a larger
    tensor alone; full-v tensors apart).  Every tensor alone (1 byte) and
    1-2 tensors per segment (20000 bytes: the norm joins the next q block)
    give the bits of a single segment over the list, and the oracle's
    values within the bounds; also with a persistent grid of 5 workgroups
    walking each segment's units."""
    a = _mini_run(4, 7, segment_bytes=segment_bytes, grid=grid)
    b = _mini_run(4, 7, segment_bytes=1 << 40)
    assert all_equal(a.buffers(), b.buffers())


# ------------------------------------------------------------------ blockwise
@pytest.mark.parametrize("bits,block", [(8, 256), (4, 128), (8, 64), (4, 512)])
def test_blockwise_codes_bit_exact(bits, block):
    """Codes and absmax equal the oracle's bit for bit at every step (the
    state recipe is a fixed sequence of fp32 operations); p within bounds."""
    sizes = [77, 1000, 4096, 5000, 3 * 4096 + 2 * 256 + 13]
    lr, wd = 1e-3, 0.01
    p0 = _p0(sizes, 8 + bits)
    qs = QuantState(_to_dev(p0), bits, block)
    plan = osa.Plan(qs.tensor_list([wd] * len(sizes)), osa.OPTIM_ALGO_BLOCKWISE, bits=bits, block=block)
    sc = DevScalars(lr)
    lr32 = float(np.float32(lr))
    op = [x.astype(np.float64) for x in p0]
    oqm = [np.zeros(n, np.uint8) for n in sizes]
    oqv = [np.zeros(n, np.uint8) for n in sizes]
    oam = [np.zeros((n + block - 1) // block, np.float32) for n in sizes]
    oav = [np.zeros((n + block - 1) // block, np.float32) for n in sizes]
    for t in range(1, 11):
        gs = _grads(sizes, 12, t, 1e-3)
        for dst, g in zip(qs.g, gs):
            dst.copy_(torch.from_numpy(g).to(DEV))
        osa.optim_step_8bit_blockwise(plan.handle, osa.optim_adamw_hp(0.9, 0.999, 1e-8), bits, block, sc.lr,
                                      None, None, sc.step)
        for i, n in enumerate(sizes):
            orc.blockwise_step(op[i], gs[i], oqm[i], oqv[i], oam[i], oav[i], bits, block, lr32, 0.9, 0.999,
                               1e-8, wd, t)
            gm, gv = qs.qm[i].cpu().numpy(), qs.qv[i].cpu().numpy()
            if bits == 4:
                em, ev = orc.pack_nibbles(oqm[i]), orc.pack_nibbles(oqv[i])
            else:
                em, ev = oqm[i], oqv[i]
            assert np.array_equal(gm, em), (t, i, np.flatnonzero(gm != em)[:10])
            assert np.array_equal(gv, ev), (t, i, np.flatnonzero(gv != ev)[:10])
            assert np.array_equal(qs.am[i].cpu().numpy().view(np.uint32), oam[i].view(np.uint32))
            assert np.array_equal(qs.av[i].cpu().numpy().view(np.uint32), oav[i].view(np.uint32))
            err = relerr_tau(qs.p[i].cpu().numpy(), op[i], lr32)
            assert err <= (TOL_STEP1 if t == 1 else TOL_RUN), (t, i, err)


@pytest.mark.parametrize("bits,block,tile", [(8, 256, 16384), (4, 128, 0)])
def test_blockwise_arrays_across_a_2gib_address_boundary(bits, block, tile):
    """Every array of the tensor sits in one 4 GiB allocation, placed so that
    the low 32 bits of its addresses run through 0x80000000 (the step keeps
    per-unit pointers in scalar registers; each half of a pointer must be
    moved without sign extension)."""
    n = 3 * 16384 + 2 * 256 + 13
    nb, nblk = (n * bits + 7) // 8, (n + block - 1) // block
    sizes = [4 * n, 4 * n, nb, nb, 4 * nblk, 4 * nblk]
    span = sum((x + 255) // 256 * 256 for x in sizes)
    buf = torch.zeros((1 << 32) + span, dtype=torch.uint8, device=DEV)
    off = (0x7FFFC000 - buf.data_ptr()) % (1 << 32)
    views, o = [], off
    for x in sizes:
        views.append(buf[o:o + x])
        o += (x + 255) // 256 * 256
    assert views[0].data_ptr() % (1 << 32) < 0x80000000 < (views[0].data_ptr() + 4 * n) % (1 << 32)
    p, g = views[0].view(torch.float32), views[1].view(torch.float32)
    qm, qv, am, av = views[2], views[3], views[4].view(torch.float32), views[5].view(torch.float32)
    p0 = _p0([n], 30 + bits)[0]
    p.copy_(torch.from_numpy(p0).to(DEV))
    tl = osa.TensorList([p], [g], qm=[qm], qv=[qv], absmax_m=[am], absmax_v=[av], weight_decay=[0.01])
    plan = osa.Plan(tl, osa.OPTIM_ALGO_BLOCKWISE, bits=bits, block=block, tile=tile)
    sc = DevScalars(1e-3)
    lr32 = float(np.float32(1e-3))
    op = p0.astype(np.float64)
    oqm, oqv = np.zeros(n, np.uint8), np.zeros(n, np.uint8)
    oam, oav = np.zeros(nblk, np.float32), np.zeros(nblk, np.float32)
    for t in range(1, 4):
        gh = _grads([n], 31, t, 1e-3)[0]
        g.copy_(torch.from_numpy(gh).to(DEV))
        osa.optim_step_8bit_blockwise(plan.handle, osa.optim_adamw_hp(0.9, 0.999, 1e-8), bits, block, sc.lr,
                                      None, None, sc.step)
        orc.blockwise_step(op, gh, oqm, oqv, oam, oav, bits, block, lr32, 0.9, 0.999, 1e-8, 0.01, t)
        em = orc.pack_nibbles(oqm) if bits == 4 else oqm
        ev = orc.pack_nibbles(oqv) if bits == 4 else oqv
        assert np.array_equal(qm.cpu().numpy(), em), t
        assert np.array_equal(qv.cpu().numpy(), ev), t
        assert np.array_equal(am.cpu().numpy().view(np.uint32), oam.view(np.uint32)), t
        assert np.array_equal(av.cpu().numpy().view(np.uint32), oav.view(np.uint32)), t
        assert relerr_tau(p.cpu().numpy(), op, lr32) <= (TOL_STEP1 if t == 1 else TOL_RUN), t
    del buf, views, p, g, qm, qv, am, av, tl, plan
    torch.cuda.empty_cache()


@pytest.mark.parametrize("bits,block", [(8, 256), (4, 128), (8, 64), (4, 512)])
def test_blockwise_ademamix_codes_bit_exact(bits, block):
    """Blockwise AdEMAMix: the three code arrays and absmax equal the
    oracle's bit for bit at every step of ten; p within the step bounds;
    ragged tensors, several units, a persistent-grid-free default launch."""
    sizes = [77, 1000, 4096, 5000, 3 * 4096 + 2 * 256 + 13, 16384 + 512]
    lr, wd, b3, alpha = 1e-3, 0.01, 0.999, 5.0
    p0 = _p0(sizes, 40 + bits)
    qs = QuantState(_to_dev(p0), bits, block, ademamix=True)
    plan = osa.Plan(qs.tensor_list([wd] * len(sizes)), osa.OPTIM_ALGO_BLOCKWISE_ADEMAMIX, bits=bits, block=block,
                    tile=4096)
    hp = osa.optim_ademamix_hp(0.9, 0.999, b3, alpha, 1e-8)
    sc = DevScalars(lr)
    lr32 = float(np.float32(lr))
    op = [x.astype(np.float64) for x in p0]
    oq = [[np.zeros(n, np.uint8) for n in sizes] for _ in range(3)]
    oa = [[np.zeros((n + block - 1) // block, np.float32) for n in sizes] for _ in range(3)]
    pack = (lambda c: orc.pack_nibbles(c)) if bits == 4 else (lambda c: c)
    for t in range(1, 11):
        gs = _grads(sizes, 41, t, 1e-3)
        for dst, g in zip(qs.g, gs):
            dst.copy_(torch.from_numpy(g).to(DEV))
        osa.optim_step_8bit_blockwise_ademamix(plan.handle, hp, bits, block, sc.lr, None, None, sc.step)
        for i, n in enumerate(sizes):
            orc.blockwise_ademamix_step(op[i], gs[i], oq[0][i], oq[1][i], oq[2][i], oa[0][i], oa[1][i], oa[2][i],
                                        bits, block, lr32, 0.9, 0.999, b3, alpha, 1e-8, wd, t)
            for dev, want in ((qs.qm[i], oq[0][i]), (qs.qm2[i], oq[1][i]), (qs.qv[i], oq[2][i])):
                got = dev.cpu().numpy()
                assert np.array_equal(got, pack(want)), (t, i, np.flatnonzero(got != pack(want))[:10])
            for dev, want in ((qs.am[i], oa[0][i]), (qs.am2[i], oa[1][i]), (qs.av[i], oa[2][i])):
                assert np.array_equal(dev.cpu().numpy().view(np.uint32), want.view(np.uint32)), (t, i)
            err = relerr_tau(qs.p[i].cpu().numpy(), op[i], lr32)
            assert err <= (TOL_STEP1 if t == 1 else TOL_RUN), (t, i, err)
    assert int(sc.step.item()) == 10


def test_blockwise_ademamix_fresh_step_closed_form():
    """bitsandbytes PR #2040 body: one fresh 8-bit AdEMAMix step at lr = 0.1,
    wd = 0.1 is the AdamW closed form with the extra alpha*(1-beta3)*g;
    decay-after sits 1e-3 away."""
    n, lr, wd, a, b3 = 256 * 300, 0.1, 0.1, 5.0, 0.9999
    p0 = _p0([n], 42)
    qs = QuantState(_to_dev(p0), 8, 256, ademamix=True)
    plan = osa.Plan(qs.tensor_list([wd]), osa.OPTIM_ALGO_BLOCKWISE_ADEMAMIX, bits=8, block=256)
    sc = DevScalars(lr)
    g = _grads([n], 42, 1, 1e-3)[0]
    qs.g[0].copy_(torch.from_numpy(g).to(DEV))
    osa.optim_step_8bit_blockwise_ademamix(plan.handle, osa.optim_ademamix_hp(0.9, 0.999, b3, a, 1e-8), 8, 256,
                                           sc.lr, None, None, sc.step)
    lr32 = float(np.float32(lr))
    gd = g.astype(np.float64)
    k = 1 + a * (1 - b3)
    got = qs.p[0].cpu().numpy()
    assert relerr_tau(got, p0[0] * (1 - lr32 * wd) - lr32 * k * gd / (np.abs(gd) + 1e-8), lr32) <= TOL_STEP1
    mutant = (p0[0] - lr32 * k * gd / (np.abs(gd) + 1e-8)) * (1 - lr32 * wd)
    assert np.max(np.abs(got - mutant)) > 0.9e-3


def test_blockwise_fresh_step_discriminates_ordering():
    """bitsandbytes PR #2040 body: one fresh 8-bit step at lr=0.1, wd=0.1 has
    the closed form -lr*g/(|g|+eps) after decay; decay-after is 1e-3 away."""
    n, lr, wd = 256 * 300, 0.1, 0.1
    p0 = _p0([n], 13)
    qs = QuantState(_to_dev(p0), 8, 256)
    plan = osa.Plan(qs.tensor_list([wd]), osa.OPTIM_ALGO_BLOCKWISE, bits=8, block=256)
    sc = DevScalars(lr)
    g = _grads([n], 13, 1, 1e-3)[0]
    qs.g[0].copy_(torch.from_numpy(g).to(DEV))
    osa.optim_step_8bit_blockwise(plan.handle, osa.optim_adamw_hp(0.9, 0.999, 1e-8), 8, 256, sc.lr, None,
                                  None, sc.step)
    lr32 = float(np.float32(lr))
    gd = g.astype(np.float64)
    p = qs.p[0].cpu().numpy()
    closed = p0[0] * (1 - lr32 * wd) - lr32 * gd / (np.abs(gd) + 1e-8)
    mutant = (p0[0] - lr32 * gd / (np.abs(gd) + 1e-8)) * (1 - lr32 * wd)
    assert relerr_tau(p, closed, lr32) <= TOL_STEP1
    assert np.max(np.abs(p - mutant)) > 0.9e-3


# ------------------------------------------------------------------ AMP
def test_check_finite_finds_every_position():
    for grad_bf16 in (False, True):
        sizes = [9, 4097, 10007]
        st = AdamState(_to_dev(_p0(sizes, 14), unaligned=(1,)), grad_bf16=grad_bf16)
        plan = osa.Plan(st.tensor_list([0.0] * 3), osa.OPTIM_ALGO_ADAMW)
        _load_grads(st, _grads(sizes, 14, 1, 1e-3))
        fi = torch.zeros(1, dtype=torch.float32, device=DEV)
        osa.optim_check_finite(plan.handle, fi)
        assert fi.item() == 0.0
        bad_vals = [float("inf"), float("-inf"), float("nan")]
        for ti, idx in [(0, 0), (0, 8), (1, 4096), (1, 17), (2, 10006), (2, 5000)]:
            for bv in bad_vals:
                saved = st.g[ti][idx].clone()
                st.g[ti][idx] = torch.tensor(bv).to(torch.bfloat16).view(torch.int16) if grad_bf16 else bv
                fi.zero_()
                osa.optim_check_finite(plan.handle, fi)
                assert fi.item() == 1.0, (grad_bf16, ti, idx, bv)
                st.g[ti][idx] = saved
        fi.zero_()
        osa.optim_check_finite(plan.handle, fi)
        assert fi.item() == 0.0


def test_skipped_step_writes_nothing():
    """FusedAdam & PyTorch Lightning AMP: with found_inf set the fused step is
    a no-op: every param, remainder and state byte and the step count stay
    unchanged; the schedule's iteration counter still advances."""
    sizes = RAGGED
    st = AdamState(_to_dev(_p0(sizes, 15)), grad_bf16=True, param_bf16=True)
    plan = osa.Plan(st.tensor_list([0.1] * len(sizes)), osa.OPTIM_ALGO_ADAMW)
    sc = DevScalars(0.0, inv_scale=2.0 ** -16)
    osa.optim_plan_set_schedule(plan.handle, osa.OPTIM_SCHED_COSINE, 3e-4, 0.0, 100, sc.iter)
    hp = osa.optim_adamw_hp(0.9, 0.95, 1e-8)
    for t in range(3):
        _load_grads(st, _grads(sizes, 15, t, 1e-3), scale=65536.0)
        osa.optim_step_adamw(plan.handle, hp, sc.lr, sc.inv_scale, sc.found_inf, sc.step)
    before = snapshot(st.buffers())
    step_before = int(sc.step.item())
    _load_grads(st, _grads(sizes, 15, 9, 1e-3), scale=65536.0)
    st.g[6][4000] = torch.tensor(float("inf")).to(torch.bfloat16).view(torch.int16)
    sc.found_inf.zero_()
    osa.optim_check_finite(plan.handle, sc.found_inf)
    osa.optim_step_adamw(plan.handle, hp, sc.lr, sc.inv_scale, sc.found_inf, sc.step)
    torch.cuda.synchronize()
    assert sc.found_inf.item() == 1.0
    assert all_equal(before, st.buffers())
    assert int(sc.step.item()) == step_before
    assert int(sc.iter.item()) == 4
    assert sc.lr.item() == float(orc.cosine_lr(3, 100, 3e-4, 0.0))


def test_power_of_two_scale_is_bitwise_equivalent():
    """AMP with grads scaled by 2^16 and inv_scale 2^-16 equals the unscaled
    run bit for bit (the unscale is exact and applied once)."""
    sizes = [5000, 4096, 3]
    p0 = _p0(sizes, 16)
    a = AdamState(_to_dev(p0), grad_bf16=True, param_bf16=True)
    b = AdamState(_to_dev(p0), grad_bf16=True, param_bf16=True)
    pa = osa.Plan(a.tensor_list([0.1, 0.0, 0.1]), osa.OPTIM_ALGO_ADAMW)
    pb = osa.Plan(b.tensor_list([0.1, 0.0, 0.1]), osa.OPTIM_ALGO_ADAMW)
    sa, sb = DevScalars(1e-3), DevScalars(1e-3, inv_scale=2.0 ** -16)
    hp = osa.optim_adamw_hp(0.9, 0.95, 1e-8)
    for t in range(1, 6):
        gs = _grads(sizes, 16, t, 1e-3)
        _load_grads(a, gs)
        _load_grads(b, gs, scale=65536.0)
        osa.optim_step_adamw(pa.handle, hp, sa.lr, None, None, sa.step)
        osa.optim_step_adamw(pb.handle, hp, sb.lr, sb.inv_scale, sb.found_inf, sb.step)
    assert all_equal(a.p + a.r + a.m + a.v, b.p + b.r + b.m + b.v)


def test_zero_lr_leaves_params_unchanged():
    sizes = [4096, 77]
    st = AdamState(_to_dev(_p0(sizes, 17)))
    plan = osa.Plan(st.tensor_list([0.1, 0.1]), osa.OPTIM_ALGO_ADAMW)
    sc = DevScalars(0.0)
    before = snapshot(st.p)
    _load_grads(st, _grads(sizes, 17, 1, 1e-3))
    osa.optim_step_adamw(plan.handle, osa.optim_adamw_hp(0.9, 0.999, 1e-8), sc.lr, None, None, sc.step)
    assert all_equal(before, st.p)
    assert int(sc.step.item()) == 1 and st.m[0].abs().max().item() > 0


def test_cosine_lr_values_on_device():
    """4 bit Adam should support non constant lr: the lr lives on the device
    and is rewritten in place each step; every value equals the oracle's."""
    st = AdamState(_to_dev(_p0([64], 18)))
    plan = osa.Plan(st.tensor_list([0.0]), osa.OPTIM_ALGO_ADAMW)
    sc = DevScalars(0.0)
    osa.optim_plan_set_schedule(plan.handle, osa.OPTIM_SCHED_COSINE, 3e-4, 1e-5, 100, sc.iter)
    lrs = torch.zeros(105, dtype=torch.float32, device=DEV)
    for k in range(105):
        osa.optim_step_adamw(plan.handle, osa.optim_adamw_hp(0.9, 0.95, 1e-8), sc.lr, None, None, sc.step)
        lrs[k] = sc.lr[0]
    got = lrs.cpu().numpy()
    want = np.array([orc.cosine_lr(k, 100, 3e-4, 1e-5) for k in range(105)], np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert int(sc.iter.item()) == 105


def test_empty_and_zero_size_lists():
    st = AdamState([])
    plan = osa.Plan(st.tensor_list([]), osa.OPTIM_ALGO_ADAMW)
    sc = DevScalars(1e-3)
    osa.optim_step_adamw(plan.handle, osa.optim_adamw_hp(0.9, 0.999, 1e-8), sc.lr, None, None, sc.step)
    assert int(sc.step.item()) == 1
    _run_adam(osa.OPTIM_ALGO_ADAMW, [0, 5, 0], 3, lr=1e-3, key=19)


def test_empty_plans_of_every_step_commit():
    """A plan with no tensors still launches one workgroup per kernel, which
    has no unit to walk: every step form publishes its step counter and
    nothing else."""
    hp = osa.optim_adamw_hp(0.9, 0.999, 1e-8)
    hpe = osa.optim_ademamix_hp(0.9, 0.999, 0.9999, 5.0, 1e-8)
    e = lambda **kw: osa.TensorList([], [], weight_decay=[], numel=[], **kw)
    cases = [
        (osa.OPTIM_ALGO_ADEMAMIX, {}, lambda pl, sc: osa.optim_step_ademamix(pl.handle, hpe, sc.lr, None, None, sc.step)),
        (osa.OPTIM_ALGO_ADAM_MINI, {}, lambda pl, sc: osa.optim_step_adam_mini(pl.handle, hp, sc.lr, None, None, sc.step)),
        (osa.OPTIM_ALGO_LION, {}, lambda pl, sc: osa.optim_step_lion(pl.handle, osa.optim_lion_hp(0.9, 0.99), sc.lr,
                                                                    None, None, sc.step)),
        (osa.OPTIM_ALGO_LAMB, {}, lambda pl, sc: osa.optim_step_lamb(pl.handle, hp, sc.lr, None, None, sc.step)),
        (osa.OPTIM_ALGO_BLOCKWISE, dict(bits=8, block=256),
         lambda pl, sc: osa.optim_step_8bit_blockwise(pl.handle, hp, 8, 256, sc.lr, None, None, sc.step)),
        (osa.OPTIM_ALGO_BLOCKWISE_ADEMAMIX, dict(bits=4, block=128),
         lambda pl, sc: osa.optim_step_8bit_blockwise_ademamix(pl.handle, hpe, 4, 128, sc.lr, None, None, sc.step)),
        (osa.OPTIM_ALGO_ADAMW, dict(state_dtype=osa.OPTIM_F16),
         lambda pl, sc: osa.optim_step_adamw(pl.handle, hp, sc.lr, None, None, sc.step)),
        (osa.OPTIM_ALGO_ADAMW, dict(state_dtype=osa.OPTIM_BF16),
         lambda pl, sc: osa.optim_step_adamw(pl.handle, hp, sc.lr, None, None, sc.step)),
    ]
    for algo, opts, step in cases:
        plan = osa.Plan(e(), algo, **opts)
        sc = DevScalars(1e-3)
        step(plan, sc)
        step(plan, sc)
        assert int(sc.step.item()) == 2, (algo, opts)
        plan.close()


def test_checkpoint_resume_is_bitwise():
    """State is raw caller-owned buffers plus the step counter: restoring them
    into fresh buffers under a new plan continues bit for bit."""
    sizes = [10007, 4096]
    p0 = _p0(sizes, 20)
    a = AdamState(_to_dev(p0))
    pa = osa.Plan(a.tensor_list([0.1, 0.0]), osa.OPTIM_ALGO_ADAMW)
    sa = DevScalars(1e-2)
    hp = osa.optim_adamw_hp(0.9, 0.999, 1e-8)
    for t in range(1, 4):
        _load_grads(a, _grads(sizes, 20, t, 1e-2))
        osa.optim_step_adamw(pa.handle, hp, sa.lr, None, None, sa.step)
    b = AdamState(_to_dev(p0))
    for dst, src in zip(b.p + b.m + b.v, a.p + a.m + a.v):
        dst.copy_(src)
    pb = osa.Plan(b.tensor_list([0.1, 0.0]), osa.OPTIM_ALGO_ADAMW)
    sb = DevScalars(1e-2)
    sb.step.copy_(sa.step)
    for t in range(4, 7):
        gs = _grads(sizes, 20, t, 1e-2)
        _load_grads(a, gs)
        _load_grads(b, gs)
        osa.optim_step_adamw(pa.handle, hp, sa.lr, None, None, sa.step)
        osa.optim_step_adamw(pb.handle, hp, sb.lr, None, None, sb.step)
    assert all_equal(a.p + a.m + a.v, b.p + b.m + b.v)


def test_device_side_validation():
    st = AdamState(_to_dev(_p0([100], 21)))
    tl = st.tensor_list([0.0])
    need = osa.optim_plan_workspace_size(tl, osa.OPTIM_ALGO_ADAMW)
    small = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(osa.OptimError) as e:
        osa.optim_plan_create(tl, osa.OPTIM_ALGO_ADAMW, None, small, need - 256)
    assert e.value.code == osa.OPTIM_EWORKSPACE
    big = torch.empty(need + 512, dtype=torch.uint8, device=DEV)
    with pytest.raises(osa.OptimError) as e:
        osa.optim_plan_create(tl, osa.OPTIM_ALGO_ADAMW, None, big.data_ptr() + 8, need)
    assert e.value.code == osa.OPTIM_EWORKSPACE
    plan = osa.Plan(tl, osa.OPTIM_ALGO_ADAMW)
    sc = DevScalars(1e-3)
    with pytest.raises(osa.OptimError) as e:
        osa.optim_step_adamw(plan.handle, osa.optim_adamw_hp(1.0, 0.999, 1e-8), sc.lr, None, None, sc.step)
    assert e.value.code == osa.OPTIM_EINVAL
    with pytest.raises(osa.OptimError) as e:
        osa.optim_step_adam_mini(plan.handle, osa.optim_adamw_hp(0.9, 0.999, 1e-8), sc.lr, None, None, sc.step)
    assert e.value.code == osa.OPTIM_EINVAL
    assert int(sc.step.item()) == 0


def test_remainder_exhaustive_against_oracle():
    """TransformerEngine PR #1408: split on the GPU equals the oracle's split
    on all 2^32 patterns, and reconstruct(split(x)) == x bit for bit."""
    CH = 1 << 28
    b = torch.empty(CH, dtype=torch.int16, device=DEV)
    r = torch.empty(CH, dtype=torch.int16, device=DEV)
    back = torch.empty(CH, dtype=torch.float32, device=DEV)
    for c in range(16):
        base = c * CH
        x = torch.arange(base, base + CH, dtype=torch.int64, device=DEV).to(torch.int32).view(torch.float32)
        osa.optim_remainder_split(x, b, r, CH)
        osa.optim_remainder_reconstruct(b, r, back, CH)
        assert torch.equal(back.view(torch.int32), x.view(torch.int32)), c
        ob, orr = orc.remainder_split(np.arange(base, base + CH, dtype=np.uint32).view(np.float32))
        assert np.array_equal(to_np_u16(b), ob), c
        assert np.array_equal(r.cpu().numpy(), orr), c
        say(f"remainder chunk {c} ok")


def test_step_replays_in_a_hip_graph():
    """Every step-varying value lives on the device and no memset is
    recorded, so a whole AMP step (finite check + bf16/remainder AdamW +
    cosine lr) can be captured once and replayed; each replay, with eager
    work in between, equals the same step run eagerly, bit for bit."""
    sizes = [5000, 4097, 33]
    p0 = _p0(sizes, 22)
    eager = AdamState(_to_dev(p0), grad_bf16=True, param_bf16=True)
    graph = AdamState(_to_dev(p0), grad_bf16=True, param_bf16=True)
    pe = osa.Plan(eager.tensor_list([0.1, 0.0, 0.1]), osa.OPTIM_ALGO_ADAMW)
    pg = osa.Plan(graph.tensor_list([0.1, 0.0, 0.1]), osa.OPTIM_ALGO_ADAMW)
    se, sg = DevScalars(0.0, inv_scale=2.0 ** -16), DevScalars(0.0, inv_scale=2.0 ** -16)
    for plan, sc in ((pe, se), (pg, sg)):
        osa.optim_plan_set_schedule(plan.handle, osa.OPTIM_SCHED_COSINE, 3e-4, 0.0, 10, sc.iter)
    hp = osa.optim_adamw_hp(0.9, 0.95, 1e-8)

    def step(plan, sc):
        sc.found_inf.zero_()
        osa.optim_check_finite(plan.handle, sc.found_inf)
        osa.optim_step_adamw(plan.handle, hp, sc.lr, sc.inv_scale, sc.found_inf, sc.step)

    torch.cuda.synchronize()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            step(pg, sg)
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    # capture recorded the work without running it: nothing has moved yet
    assert int(sg.step.item()) == 0 and int(sg.iter.item()) == 0
    for t in range(6):
        gs = _grads(sizes, 22, t, 1e-3)
        _load_grads(eager, gs, scale=65536.0)
        _load_grads(graph, gs, scale=65536.0)
        if t == 3:  # one skipped step: the replay must skip too
            for st in (eager, graph):
                st.g[1][17] = torch.tensor(float("inf")).to(torch.bfloat16).view(torch.int16)
        step(pe, se)
        g.replay()
        torch.cuda.synchronize()
        assert all_equal(eager.buffers(), graph.buffers()), t
        for a, b in ((se.step, sg.step), (se.iter, sg.iter), (se.lr, sg.lr), (se.found_inf, sg.found_inf)):
            assert torch.equal(a, b), t
    assert int(sg.step.item()) == 5 and int(sg.iter.item()) == 6
