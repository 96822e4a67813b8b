"""GPU parity of the Lion and LAMB steps against the CPU oracle, at sizes the
oracle finishes in seconds: ragged tensors over several work units, fp32 and
bf16 (+ remainder) params, fp32 and bf16 grads with a power-of-two loss
scale, other launch shapes, and skipped steps."""
import numpy as np
import pytest
import torch

import oracle as orc
import optimizer_step_adamw_amd as osa
from gpu_support import (DEV, TOL_RUN, TOL_STEP1, AdamState, DevScalars, all_equal, relerr_tau, say, snapshot,
                         to_np_u16)
from synth import host_normal

pytestmark = pytest.mark.gpu

RAGGED = [1, 7, 8, 9, 4095, 4096, 4097, 10007, 65539]


def _p0(sizes, key):
    return [host_normal(n, 0.02, 930, key, i, 0) for i, n in enumerate(sizes)]


def _load(state, sizes, key, t, scale):
    """Stores G = g*scale (fp32, or bf16 rounded) and returns the float32
    gradient the kernel sees, G * (1/scale) (exact: scale is a power of two)."""
    out = []
    for i, (dst, n) in enumerate(zip(state.g, sizes)):
        g = torch.from_numpy(host_normal(n, 1e-3, 931, key, i, t)).to(DEV) * scale
        if state.grad_bf16:
            dst.copy_(g.to(torch.bfloat16).view(torch.int16))
            G = orc.bf16_bits_to_f64(to_np_u16(dst))
        else:
            dst.copy_(g)
            G = dst.cpu().numpy().astype(np.float64)
        out.append((G / scale).astype(np.float32))
    return out


# more than 2^20 elements: 4096-element units, early-load form with 4 groups
MID = [1 << 20, 4096 * 100 + 37, 3000]


@pytest.mark.parametrize("bf16,tile,grid,sizes", [(False, 0, 0, RAGGED), (True, 0, 0, RAGGED), (False, 1024, 0, RAGGED),
                                                  (True, 2048, 7, RAGGED), (False, 0, 0, MID), (True, 0, 0, MID)])
def test_lion_matches_oracle(bf16, tile, grid, sizes):
    """m bit for bit (the fp32 recipe is fixed, so every sign decision is the
    oracle's); p within the step bounds over 12 steps.  The default plans take
    the early-load form (2048-element units for the ragged list, 4096 for the
    list above 2^20 elements)."""
    lr, wd = 1e-3, 0.1
    wds = [wd * (i % 2) for i in range(len(sizes))]
    p0 = _p0(sizes, 1 + bf16)
    st = AdamState([torch.from_numpy(x).to(DEV) for x in p0], grad_bf16=bf16, param_bf16=bf16)
    plan = osa.Plan(st.tensor_list(wds), osa.OPTIM_ALGO_LION, tile=tile, grid=grid)
    scale = 65536.0 if bf16 else 1.0
    sc = DevScalars(lr, inv_scale=1.0 / scale if bf16 else None)
    hp = osa.optim_lion_hp(0.9, 0.99)
    lr32 = float(np.float32(lr))
    op = [x.astype(np.float64) for x in p0]
    om = [np.zeros(n, np.float32) for n in sizes]
    for t in range(1, 13):
        g = _load(st, sizes, 2 + bf16, t, scale)
        osa.optim_step_lion(plan.handle, hp, sc.lr, sc.inv_scale, None, sc.step)
        for i in range(len(sizes)):
            orc.lion_step(op[i], om[i], g[i], lr32, 0.9, 0.99, wds[i])
            assert np.array_equal(st.m[i].cpu().numpy().view(np.uint32), om[i].view(np.uint32)), (t, i)
            err = relerr_tau(st.master(i).cpu().numpy(), op[i], lr32)
            assert err <= (TOL_STEP1 if t == 1 else TOL_RUN), (t, i, err)
    assert int(sc.step.item()) == 12
    say(f"lion bf16={bf16} tile={tile} grid={grid} n={sum(sizes)}: m bit-exact, p within bounds")


@pytest.mark.parametrize("bf16,tile,grid", [(False, 0, 0), (True, 0, 0), (False, 1024, 0), (False, 2048, 5)])
def test_lamb_matches_oracle(bf16, tile, grid):
    """p within the step bounds over 10 steps; each tensor's step norm is
    lr times its parameter norm (the trust ratio), as in the oracle."""
    sizes = RAGGED
    lr, wd, eps = 1e-2, 0.1, 1e-6
    wds = [wd * (i % 2) for i in range(len(sizes))]
    p0 = _p0(sizes, 3 + bf16)
    st = AdamState([torch.from_numpy(x).to(DEV) for x in p0], grad_bf16=bf16, param_bf16=bf16)
    plan = osa.Plan(st.tensor_list(wds), osa.OPTIM_ALGO_LAMB, tile=tile, grid=grid)
    scale = 65536.0 if bf16 else 1.0
    sc = DevScalars(lr, inv_scale=1.0 / scale if bf16 else None)
    hp = osa.optim_adamw_hp(0.9, 0.999, eps)
    lr32 = float(np.float32(lr))
    op = [x.astype(np.float64) for x in p0]
    om = [np.zeros(n) for n in sizes]
    ov = [np.zeros(n) for n in sizes]
    worst = 0.0
    for t in range(1, 11):
        g = _load(st, sizes, 4 + bf16, t, scale)
        before = [st.master(i).cpu().numpy().astype(np.float64) for i in range(len(sizes))]
        osa.optim_step_lamb(plan.handle, hp, sc.lr, sc.inv_scale, None, sc.step)
        for i in range(len(sizes)):
            orc.lamb_step(op[i], om[i], ov[i], g[i], lr32, 0.9, 0.999, eps, wds[i], t)
            got = st.master(i).cpu().numpy()
            err = relerr_tau(got, op[i], lr32)
            worst = max(worst, err)
            assert err <= (TOL_STEP1 if t == 1 else TOL_RUN), (t, i, err)
            if sizes[i] > 1 and not bf16:
                step = np.linalg.norm(got - before[i])
                assert abs(step - lr32 * np.linalg.norm(before[i])) <= 1e-4 * step, (t, i)
    assert int(sc.step.item()) == 10
    say(f"lamb bf16={bf16} tile={tile} grid={grid}: worst relerr_tau {worst:.3e}")


@pytest.mark.parametrize("algo", [osa.OPTIM_ALGO_LION, osa.OPTIM_ALGO_LAMB])
def test_skipped_step_writes_nothing(algo):
    sizes = [4097, 33]
    st = AdamState([torch.from_numpy(x).to(DEV) for x in _p0(sizes, 5)])
    plan = osa.Plan(st.tensor_list([0.1, 0.0]), algo)
    sc = DevScalars(1e-3)
    _load(st, sizes, 6, 1, 1.0)
    step = (lambda: osa.optim_step_lion(plan.handle, osa.optim_lion_hp(0.9, 0.99), sc.lr, None, sc.found_inf,
                                        sc.step)) if algo == osa.OPTIM_ALGO_LION else \
        (lambda: osa.optim_step_lamb(plan.handle, osa.optim_adamw_hp(0.9, 0.999, 1e-6), sc.lr, None,
                                     sc.found_inf, sc.step))
    step()
    before = snapshot(st.buffers())
    sc.found_inf.fill_(1.0)
    step()
    assert all_equal(before, st.buffers()) and int(sc.step.item()) == 1
    sc.found_inf.zero_()
    step()
    assert not all_equal(before, st.buffers()) and int(sc.step.item()) == 2
