"""End-to-end AMP loop on a tiny model, after the deterministic repro on the
"FusedAdam & PyTorch Lightning AMP" page (Lightning issue #15501): a 10x10
linear layer with bias, mean-squared-error loss, Adam at lr 1, 10 steps, loss
tables compared across precision settings.

The model's forward and backward run in fp32 on the CPU (torch autograd is
plumbing here; CPU matmuls are deterministic); every optimizer step is the
library's fused step on the GPU.  With a power-of-two loss scale the scaled
backward is exact, so the fused step that unscales once must reproduce the
unscaled run bit for bit: every loss and every parameter.  Unscaling in the
caller as well (the hazard the page analyses: unscale_ before a fused step
that unscales again) must change the trajectory.  A non-finite gradient
injected at one step must skip that step: the run then repeats, one step
late, exactly what a run that never saw it does."""
import numpy as np
import pytest
import torch

import optimizer_step_adamw_amd as osa
from gpu_support import DEV, DevScalars
from synth import host_normal

pytestmark = pytest.mark.gpu

STEPS = 10
SCALE = 65536.0


def _data():
    x = torch.from_numpy(host_normal(16 * 10, 1.0, 2809, 0)).view(16, 10)
    y = torch.from_numpy(host_normal(16 * 10, 1.0, 2809, 1)).view(16, 10)
    w0 = host_normal(100, 0.3, 2809, 2)
    b0 = host_normal(10, 0.3, 2809, 3)
    return x, y, w0, b0


def _run(mode, inf_at=None, steps=STEPS):
    """mode: 'fp32' (no scale), 'amp' (loss x 2^16, fused unscale), or
    'double' (loss x 2^16, grads unscaled by the caller and again by the
    step).  inf_at: step index whose scaled gradient gets a +inf."""
    x, y, w0, b0 = _data()
    W = torch.from_numpy(w0).to(DEV)
    b = torch.from_numpy(b0).to(DEV)
    gW, gb = torch.zeros_like(W), torch.zeros_like(b)
    M = [torch.zeros_like(W), torch.zeros_like(b)]
    V = [torch.zeros_like(W), torch.zeros_like(b)]
    plan = osa.Plan(osa.TensorList([W, b], [gW, gb], m=M, v=V, weight_decay=[0.0, 0.0]), osa.OPTIM_ALGO_ADAMW)
    sc = DevScalars(1.0, inv_scale=None if mode == "fp32" else 1.0 / SCALE)
    hp = osa.optim_adamw_hp(0.9, 0.999, 1e-8)
    scale = 1.0 if mode == "fp32" else SCALE
    losses = []
    for k in range(steps):
        Wc = W.cpu().view(10, 10).clone().requires_grad_(True)
        bc = b.cpu().clone().requires_grad_(True)
        loss = ((x @ Wc.T + bc - y) ** 2).mean()
        losses.append(float(loss.detach()))
        (loss * scale).backward()
        g_w, g_b = Wc.grad.reshape(-1), bc.grad
        if mode == "double":
            g_w, g_b = g_w / scale, g_b / scale
        if k == inf_at:
            g_w = g_w.clone()
            g_w[37] = float("inf")
        gW.copy_(g_w)
        gb.copy_(g_b)
        sc.found_inf.zero_()
        osa.optim_check_finite(plan.handle, sc.found_inf)
        osa.optim_step_adamw(plan.handle, hp, sc.lr, sc.inv_scale, sc.found_inf, sc.step)
    torch.cuda.synchronize()
    out = dict(losses=np.array(losses, np.float32), W=W.cpu().numpy(), b=b.cpu().numpy(),
               step=int(sc.step.item()))
    plan.close()
    return out


def test_amp_loop_matches_fp32_bit_for_bit():
    a, s = _run("fp32"), _run("amp")
    assert a["step"] == s["step"] == STEPS
    assert np.array_equal(a["losses"].view(np.uint32), s["losses"].view(np.uint32)), (a["losses"], s["losses"])
    assert np.array_equal(a["W"].view(np.uint32), s["W"].view(np.uint32))
    assert np.array_equal(a["b"].view(np.uint32), s["b"].view(np.uint32))
    # the run trains: lr 1 moves every weight, and the loss changes
    assert a["losses"][-1] != a["losses"][0]


def test_double_unscale_changes_the_trajectory():
    a, d = _run("fp32"), _run("double")
    assert d["step"] == STEPS
    assert not np.array_equal(a["losses"], d["losses"])
    assert not np.array_equal(a["W"], d["W"])


def test_inf_step_is_skipped_in_the_loop():
    """The step with the +inf gradient writes nothing (params, m, v) and does
    not count, so the next step sees the same model, the same gradient and
    the same t as the skipped one: from there the run repeats the clean run
    one step late, bit for bit, and ends where 9 clean steps end."""
    s = _run("amp", inf_at=4)
    a = _run("amp", steps=STEPS - 1)
    assert s["step"] == a["step"] == STEPS - 1
    u = lambda x: x.view(np.uint32)
    assert np.array_equal(u(s["losses"][:5]), u(a["losses"][:5]))
    assert s["losses"][5] == s["losses"][4]
    assert np.array_equal(u(s["losses"][5:]), u(a["losses"][4:]))
    assert np.array_equal(u(s["W"]), u(a["W"])) and np.array_equal(u(s["b"]), u(a["b"]))
