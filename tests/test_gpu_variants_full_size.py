"""Full-size parity of the Lion, LAMB and master-weight steps: the 4096 x 4096
tensor with the benchmark's inputs (its synthetic parameters and gradients,
hyperparameters and default launch configuration), every element against
the oracle over three steps."""
import numpy as np
import pytest
import torch

import oracle as orc
import optimizer_step_adamw_amd as osa
import synth
from gpu_support import DEV, TOL_RUN, TOL_STEP1, DevScalars, relerr_tau, say

pytestmark = pytest.mark.gpu

STEPS = 3


def _inputs():
    wl = synth.c2_decay_stress()
    p0 = synth.initial_param_device(wl.tensors[0], wl.p_std, wl.index, 0, DEV)
    g = synth.device_normal(wl.numel, wl.g_std, DEV, wl.index, 0, 1, synth.GRAD)
    return wl, p0, g


def _tol(t):
    return TOL_STEP1 if t == 1 else TOL_RUN


def test_lion_full_size():
    wl, p0, g = _inputs()
    p, m = p0.clone(), torch.zeros_like(p0)
    plan = osa.Plan(osa.TensorList([p], [g], m=[m], weight_decay=[wl.hp.wd]), osa.OPTIM_ALGO_LION)
    sc = DevScalars(1e-4)
    lr32 = float(np.float32(1e-4))
    op = p0.cpu().numpy().astype(np.float64)
    om = np.zeros(wl.numel, np.float32)
    g32 = g.cpu().numpy()
    for t in range(1, STEPS + 1):
        osa.optim_step_lion(plan.handle, osa.optim_lion_hp(0.9, 0.99), sc.lr, None, None, sc.step)
        orc.lion_step(op, om, g32, lr32, 0.9, 0.99, wl.hp.wd)
        assert np.array_equal(m.cpu().numpy().view(np.uint32), om.view(np.uint32)), t
        err = relerr_tau(p.cpu().numpy(), op, lr32)
        assert err <= _tol(t), (t, err)
    say(f"lion 4096x4096: m bit-exact, p relerr_tau {err:.2e}")


def test_lamb_full_size():
    wl, p0, g = _inputs()
    p, m, v = p0.clone(), torch.zeros_like(p0), torch.zeros_like(p0)
    plan = osa.Plan(osa.TensorList([p], [g], m=[m], v=[v], weight_decay=[wl.hp.wd]), osa.OPTIM_ALGO_LAMB)
    sc = DevScalars(1e-3)
    lr32 = float(np.float32(1e-3))
    op = p0.cpu().numpy().astype(np.float64)
    om, ov = np.zeros(wl.numel), np.zeros(wl.numel)
    g64 = g.cpu().numpy().astype(np.float64)
    for t in range(1, STEPS + 1):
        osa.optim_step_lamb(plan.handle, osa.optim_adamw_hp(wl.hp.beta1, wl.hp.beta2, 1e-6), sc.lr, None, None,
                            sc.step)
        orc.lamb_step(op, om, ov, g64, lr32, wl.hp.beta1, wl.hp.beta2, 1e-6, wl.hp.wd, t)
        err = relerr_tau(p.cpu().numpy(), op, lr32)
        assert err <= _tol(t), (t, err)
    say(f"lamb 4096x4096: p relerr_tau {err:.2e}")


@pytest.mark.parametrize("half", [False, True])
def test_master_copy_full_size(half):
    wl, p0, g = _inputs()
    hp = wl.hp
    master = p0.clone()
    model = torch.zeros(wl.numel, dtype=torch.int16, device=DEV)
    m, v = torch.zeros_like(p0), torch.zeros_like(p0)
    plan = osa.Plan(osa.TensorList([model], [g], m=[m], v=[v], master=[master], weight_decay=[hp.wd],
                                   param_dtype=osa.OPTIM_F16 if half else osa.OPTIM_BF16), osa.OPTIM_ALGO_ADAMW)
    sc = DevScalars(hp.lr)
    lr32 = float(np.float32(hp.lr))
    op = p0.cpu().numpy().astype(np.float64)
    om, ov = np.zeros(wl.numel), np.zeros(wl.numel)
    g64 = g.cpu().numpy().astype(np.float64)
    for t in range(1, STEPS + 1):
        osa.optim_step_adamw(plan.handle, osa.optim_adamw_hp(hp.beta1, hp.beta2, hp.eps), sc.lr, None, None, sc.step)
        orc.adamw_step(op, om, ov, g64, lr32, hp.beta1, hp.beta2, hp.eps, hp.wd, t)
        got = master.cpu().numpy()
        err = relerr_tau(got, op, lr32)
        assert err <= _tol(t), (t, err)
        copy = model.cpu().numpy().view(np.uint16)
        assert np.array_equal(copy, orc.round_model_copy(got, half)), t
    say(f"master half={half} 4096x4096: copy bit-exact, master relerr_tau {err:.2e}")
