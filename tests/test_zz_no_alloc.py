"""The plan on the library's static workspace (optim_plan_create_static,
for callers that cannot allocate device memory) against the plan on a
caller workspace (optim_plan_create): the same steps on copies of the same
state give the same bits, on two static plans in a row, the second over a
smaller list; the first is refused once the second exists."""
import numpy as np
import pytest
import torch

import optimizer_step_adamw_amd as osa
from gpu_support import DEV, AdamState, DevScalars, all_equal, say, snapshot
from synth import host_normal

pytestmark = pytest.mark.gpu


def _grads(st, sizes, key, t, scale=1.0):
    for i, (dst, n) in enumerate(zip(st.g, sizes)):
        g = torch.from_numpy(host_normal(n, 1e-3, 960, key, i, t)).to(DEV) * scale
        dst.copy_(g.to(torch.bfloat16).view(torch.int16) if st.grad_bf16 else g)


def _twin(p0, v_len=None, **kw):
    a = AdamState([torch.from_numpy(x).to(DEV) for x in p0], v_len=v_len, **kw)
    b = AdamState([torch.from_numpy(x).to(DEV) for x in p0], v_len=v_len, **kw)
    return a, b


def test_static_plans_match_workspace_plans_twice():
    print("case: Adam-mini list on the static workspace, then a smaller LAMB list", flush=True)
    # ---- first call: Adam-mini (partials and block factors in the workspace)
    head = 65536
    sizes = [8 * head, 100003, 50001, 4096, 777]
    kinds = [osa.OPTIM_MINI_HEAD, osa.OPTIM_MINI_SCALAR, osa.OPTIM_MINI_FULL_V, osa.OPTIM_MINI_SCALAR,
             osa.OPTIM_MINI_SCALAR]
    heads = [head, sizes[1], 0, sizes[3], sizes[4]]
    wd = [0.1, 0.1, 0.1, 0.0, 0.1]
    vlen = [n if k == osa.OPTIM_MINI_FULL_V else n // h for n, k, h in zip(sizes, kinds, heads)]
    p0 = [host_normal(n, 0.02, 961, 0, i, 0) for i, n in enumerate(sizes)]
    A, B = _twin(p0, v_len=vlen)
    ref = osa.Plan(A.tensor_list(wd, kinds, heads), osa.OPTIM_ALGO_ADAM_MINI)
    tlb = B.tensor_list(wd, kinds, heads)
    h1 = osa.optim_plan_create_static(tlb, osa.OPTIM_ALGO_ADAM_MINI, None)
    sa, sb = DevScalars(3e-4), DevScalars(3e-4)
    hp = osa.optim_adamw_hp(0.9, 0.95, 1e-8)
    for t in (1, 2, 3):
        _grads(A, sizes, 1, t)
        for x, y in zip(B.g, A.g):
            x.copy_(y)
        osa.optim_step_adam_mini(ref.handle, hp, sa.lr, None, None, sa.step)
        osa.optim_step_adam_mini(h1, hp, sb.lr, None, None, sb.step)
    torch.cuda.synchronize()
    assert all_equal(A.buffers(), B.buffers()) and torch.equal(sa.step, sb.step)
    assert int(sb.step.item()) == 3
    say("Adam-mini: static plan equals the workspace plan bit for bit over 3 steps")

    # ---- second call, smaller list: LAMB (two partials per unit), bf16
    # grads with a loss scale, the fused check + norm, an overflow step
    sizes2 = [5000, 333, 4096]
    p02 = [host_normal(n, 0.02, 962, 0, i, 0) for i, n in enumerate(sizes2)]
    C, D = _twin(p02, grad_bf16=True)
    ref2 = osa.Plan(C.tensor_list([0.1, 0.0, 0.1]), osa.OPTIM_ALGO_LAMB)
    h2 = osa.optim_plan_create_static(D.tensor_list([0.1, 0.0, 0.1]), osa.OPTIM_ALGO_LAMB, None)
    # the first static plan is now refused by every entry point, launching nothing
    before = snapshot(B.buffers())
    with pytest.raises(osa.OptimError) as ei:
        osa.optim_step_adam_mini(h1, hp, sb.lr, None, None, sb.step)
    assert ei.value.code == osa.OPTIM_EINVAL and "superseded" in str(ei.value)
    with pytest.raises(osa.OptimError):
        osa.optim_check_finite(h1, sb.found_inf)
    torch.cuda.synchronize()
    assert all_equal(before, B.buffers()) and int(sb.step.item()) == 3
    osa.optim_plan_destroy(h1)
    scale = 1024.0
    sc, sd = DevScalars(1e-3, 1.0 / scale), DevScalars(1e-3, 1.0 / scale)
    fc, fd = torch.zeros(1, device=DEV), torch.zeros(1, device=DEV)  # clip factors
    nc, nd = torch.zeros(1, device=DEV), torch.zeros(1, device=DEV)
    hl = osa.optim_adamw_hp(0.9, 0.999, 1e-6)
    for t in (1, 2, 3, 4):
        _grads(C, sizes2, 2, t, scale)
        if t == 3:
            C.g[1][17] = torch.tensor(float("inf")).to(torch.bfloat16).view(torch.int16)
        for x, y in zip(D.g, C.g):
            x.copy_(y)
        for plan, s, f, nrm in ((ref2.handle, sc, fc, nc), (h2, sd, fd, nd)):
            s.found_inf.zero_()
            osa.optim_grad_norm(plan, s.inv_scale, 0.05, s.found_inf, nrm, f)
            osa.optim_step_lamb(plan, hl, s.lr, f, s.found_inf, s.step)
    torch.cuda.synchronize()
    assert all_equal(C.buffers(), D.buffers())
    assert torch.equal(fc, fd) and torch.equal(nc, nd) and torch.equal(sc.step, sd.step)
    assert int(sd.step.item()) == 3  # the overflow step was skipped
    say("LAMB (smaller list, AMP norm + clip, one skipped step): static plan equals the workspace plan")
    osa.optim_plan_destroy(h2)
    ref.close()
    ref2.close()


@pytest.mark.parametrize("ademamix,interleaved", [(False, False), (True, False), (False, True), (True, True)])
def test_static_plan_with_packs_matches_workspace_plan(ademamix, interleaved):
    """A list of small tensors, laid end to end in packs (their member
    records in the static workspace), then a larger tensor: the static plan
    steps bit for bit as the workspace plan, with bf16 params + remainders,
    moments in separate arrays or interleaved in one array per tensor."""
    print(f"case: static plan with packs, ademamix={ademamix} interleaved={interleaved}", flush=True)
    sizes = [300, 7, 1000, 4, 65, 513, 9000, 1, 2047, 12]
    p0 = [host_normal(n, 0.02, 963, 0, i, 0) for i, n in enumerate(sizes)]
    A, B = _twin(p0, param_bf16=True, ademamix=ademamix, moments_interleaved=interleaved)
    wd = [0.1 if i % 3 else 0.0 for i in range(len(sizes))]
    algo = osa.OPTIM_ALGO_ADEMAMIX if ademamix else osa.OPTIM_ALGO_ADAMW
    layout = osa.OPTIM_LAYOUT_INTERLEAVED if interleaved else osa.OPTIM_LAYOUT_SEPARATE
    ref = osa.Plan(A.tensor_list(wd), algo, state_layout=layout)
    h = osa.optim_plan_create_static(B.tensor_list(wd), algo, osa.optim_plan_opts(0, 0, 0, 0, 0, 0, layout))
    sa, sb = DevScalars(1e-3), DevScalars(1e-3)
    for t in (1, 2, 3):
        _grads(A, sizes, 3, t)
        for x, y in zip(B.g, A.g):
            x.copy_(y)
        for plan, s in ((ref.handle, sa), (h, sb)):
            if ademamix:
                osa.optim_step_ademamix(plan, osa.optim_ademamix_hp(0.9, 0.999, 0.9999, 5.0, 1e-8), s.lr, None,
                                        None, s.step)
            else:
                osa.optim_step_adamw(plan, osa.optim_adamw_hp(0.9, 0.999, 1e-8), s.lr, None, None, s.step)
    torch.cuda.synchronize()
    assert all_equal(A.buffers(), B.buffers()) and int(sb.step.item()) == 3
    say(f"{'AdEMAMix' if ademamix else 'AdamW'} with packs (interleaved={interleaved}): static plan equals the "
        "workspace plan over 3 steps")
    osa.optim_plan_destroy(h)
    ref.close()
