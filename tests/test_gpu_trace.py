"""The kernel trace of a plan (optim_plan_trace / optim_plan_trace_read):
one record per launch, in launch order, with the kernels' names and grids;
traced steps give the same bits as untraced ones; launches past the
capacity run untraced and are counted."""
import numpy as np
import pytest
import torch

import optimizer_step_adamw_amd as osa
from gpu_support import DEV, AdamState, DevScalars, all_equal, say
from synth import host_normal

pytestmark = pytest.mark.gpu


def test_trace_records_every_adam_mini_launch_and_changes_nothing():
    print("case: Adam-mini, 3 segments, traced against untraced", flush=True)
    head = 65536
    sizes = [4 * head, 70001, 50001, 4 * head]
    kinds = [osa.OPTIM_MINI_HEAD, osa.OPTIM_MINI_SCALAR, osa.OPTIM_MINI_FULL_V, osa.OPTIM_MINI_HEAD]
    heads = [head, sizes[1], 0, head]
    vlen = [n if k == osa.OPTIM_MINI_FULL_V else n // h for n, k, h in zip(sizes, kinds, heads)]
    wd = [0.1] * 4
    p0 = [torch.from_numpy(host_normal(n, 0.02, 970, 0, i, 0)).to(DEV) for i, n in enumerate(sizes)]
    A = AdamState(p0, v_len=vlen)
    B = AdamState(p0, v_len=vlen)
    for i, n in enumerate(sizes):
        g = torch.from_numpy(host_normal(n, 1e-3, 970, 1, i, 1)).to(DEV)
        A.g[i].copy_(g)
        B.g[i].copy_(g)
    # segments: [head tensor, scalar tensor] (shared v), [full v], [head tensor]
    seg = (sizes[0] + sizes[1]) * 4
    pa = osa.Plan(A.tensor_list(wd, kinds, heads), osa.OPTIM_ALGO_ADAM_MINI, segment_bytes=seg)
    pb = osa.Plan(B.tensor_list(wd, kinds, heads), osa.OPTIM_ALGO_ADAM_MINI, segment_bytes=seg)
    sa, sb = DevScalars(1e-3), DevScalars(1e-3)
    hp = osa.optim_adamw_hp(0.9, 0.95, 1e-8)
    osa.optim_plan_trace(pb.handle, 64)
    for _ in range(2):
        osa.optim_step_adam_mini(pa.handle, hp, sa.lr, None, None, sa.step)
        osa.optim_step_adam_mini(pb.handle, hp, sb.lr, None, None, sb.step)
    recs, dropped = osa.optim_plan_trace_read(pb.handle)
    assert dropped == 0
    names = [r[0] for r in recs]
    one = ["mini_sumsq_kernel", "mini_finalize_kernel", "mini_update_kernel", "mini_update_kernel",
           "mini_sumsq_kernel", "mini_finalize_kernel", "mini_update_kernel"]
    assert names == one * 2, names
    # 4096-element units; a HEAD tensor's blocks of 65536 are 16 units each
    cdiv = lambda a, b: (a + b - 1) // b
    seg_units = [4 * 16 + cdiv(sizes[1], 4096), cdiv(sizes[2], 4096), 4 * 16]
    grids = [cdiv(seg_units[0], 2), 5, seg_units[0], seg_units[1], cdiv(seg_units[2], 2), 4, seg_units[2]]
    assert [r[1] for r in recs] == grids * 2, recs
    assert all(r[2] > 0.0 for r in recs)
    torch.cuda.synchronize()
    assert all_equal(A.buffers(), B.buffers()) and torch.equal(sa.step, sb.step)
    # past the capacity: untraced and counted; reading empties the trace
    osa.optim_plan_trace(pb.handle, 4)
    osa.optim_step_adam_mini(pb.handle, hp, sb.lr, None, None, sb.step)
    recs, dropped = osa.optim_plan_trace_read(pb.handle)
    assert len(recs) == 4 and dropped == 3
    recs, dropped = osa.optim_plan_trace_read(pb.handle)
    assert recs == [] and dropped == 0
    osa.optim_plan_trace(pb.handle, 0)
    with pytest.raises(osa.OptimError):
        osa.optim_plan_trace_read(pb.handle)
    say("trace: 14 launches recorded in order; traced steps equal untraced ones bit for bit")
    pa.close()
    pb.close()


def test_trace_of_single_kernel_steps_and_norm():
    """AdamW (one kernel per step) and the gradient norm (check + sums, two
    reduction stages): names and counts."""
    n = 1 << 20
    st = AdamState([torch.zeros(n, device=DEV)])
    st.g[0].normal_()
    plan = osa.Plan(st.tensor_list([0.0]), osa.OPTIM_ALGO_ADAMW)
    s = DevScalars(1e-3)
    hp = osa.optim_adamw_hp(0.9, 0.999, 1e-8)
    osa.optim_plan_trace(plan.handle, 16)
    osa.optim_step_adamw(plan.handle, hp, s.lr, None, None, s.step)
    norm, clip = torch.zeros(1, device=DEV), torch.zeros(1, device=DEV)
    osa.optim_grad_norm(plan.handle, None, 1.0, s.found_inf, norm, clip)
    osa.optim_check_finite(plan.handle, s.found_inf)
    recs, _ = osa.optim_plan_trace_read(plan.handle)
    assert [r[0] for r in recs] == ["adam_kernel", "finite_kernel", "norm_stage1_kernel", "norm_finalize_kernel",
                                     "finite_kernel"], recs
    assert recs[0][1] == n // 2048 and recs[3][1] == 1
    say(f"trace: AdamW 2^20 kernel {1e3 * recs[0][2]:.1f} us")
    plan.close()
