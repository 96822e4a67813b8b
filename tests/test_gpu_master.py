"""GPU parity of the master-weight variant (Transformer Engine page, review
thread: an FP32 master beside a BF16 or FP16 model parameter): the AdamW
and AdEMAMix steps update the fp32 master like fp32 params and rewrite the
model copy as the master rounded to nearest even -- checked bit for bit
against the oracle's rounding of the GPU's master at every step."""
import numpy as np
import pytest
import torch

import oracle as orc
import optimizer_step_adamw_amd as osa
from gpu_support import DEV, TOL_RUN, TOL_STEP1, DevScalars, relerr_tau, say
from synth import host_normal

pytestmark = pytest.mark.gpu

RAGGED = [1, 7, 8, 9, 4095, 4096, 4097, 10007, 65539]


def _edge_values():
    """Master values across the fp16 range: subnormals, ties, near the
    largest finite value and beyond it (the copy overflows to inf)."""
    v = np.float32([6e-8, 3e-8, 1e-6, -2.5e-5, 6.1e-5, 1.0, -1.0009765625, 1.00048828125, 65504.0, 65519.0,
                    65520.0, -70000.0, 1e5, 3.0e38])
    return np.tile(v, 300)[:4097]


@pytest.mark.parametrize("algo,half,grad_bf16", [(osa.OPTIM_ALGO_ADAMW, False, True), (osa.OPTIM_ALGO_ADAMW, True, False),
                                                 (osa.OPTIM_ALGO_ADEMAMIX, True, True),
                                                 (osa.OPTIM_ALGO_ADEMAMIX, False, False)])
def test_master_weights_match_oracle(algo, half, grad_bf16):
    sizes = RAGGED + [4097]
    lr, wd, b3, alpha = 1e-3, 0.1, 0.999, 5.0
    p0 = [host_normal(n, 0.02, 940, half, i, 0) for i, n in enumerate(RAGGED)] + [_edge_values()]
    master = [torch.from_numpy(x).to(DEV) for x in p0]
    model = [torch.zeros(n, dtype=torch.int16, device=DEV) for n in sizes]
    g = [torch.zeros(n, dtype=torch.int16 if grad_bf16 else torch.float32, device=DEV) for n in sizes]
    m = [torch.zeros(n, device=DEV) for n in sizes]
    v = [torch.zeros(n, device=DEV) for n in sizes]
    m2 = [torch.zeros(n, device=DEV) for n in sizes] if algo == osa.OPTIM_ALGO_ADEMAMIX else None
    wds = [wd * (i % 2) for i in range(len(sizes))]
    tl = osa.TensorList(model, g, m=m, v=v, m2=m2, master=master, weight_decay=wds,
                        param_dtype=osa.OPTIM_F16 if half else osa.OPTIM_BF16,
                        grad_dtype=osa.OPTIM_BF16 if grad_bf16 else osa.OPTIM_F32)
    plan = osa.Plan(tl, algo)
    sc = DevScalars(lr)
    lr32 = float(np.float32(lr))
    op = [x.astype(np.float64) for x in p0]
    om, ov, om2 = ([np.zeros(n) for n in sizes] for _ in range(3))
    for t in range(1, 9):
        gs = []
        for i, n in enumerate(sizes):
            gh = torch.from_numpy(host_normal(n, 1e-2, 941, half, i, t)).to(DEV)
            if grad_bf16:
                g[i].copy_(gh.to(torch.bfloat16).view(torch.int16))
                gs.append(orc.bf16_bits_to_f64(g[i].cpu().numpy().view(np.uint16)))
            else:
                g[i].copy_(gh)
                gs.append(gh.cpu().numpy().astype(np.float64))
        if algo == osa.OPTIM_ALGO_ADAMW:
            osa.optim_step_adamw(plan.handle, osa.optim_adamw_hp(0.9, 0.999, 1e-8), sc.lr, None, None, sc.step)
        else:
            osa.optim_step_ademamix(plan.handle, osa.optim_ademamix_hp(0.9, 0.999, b3, alpha, 1e-8), sc.lr, None,
                                    None, sc.step)
        for i in range(len(sizes)):
            if algo == osa.OPTIM_ALGO_ADAMW:
                orc.adamw_step(op[i], om[i], ov[i], gs[i], lr32, 0.9, 0.999, 1e-8, wds[i], t)
            else:
                orc.ademamix_step(op[i], om[i], om2[i], ov[i], gs[i], lr32, 0.9, 0.999, b3, alpha, 1e-8, wds[i], t)
            got = master[i].cpu().numpy()
            err = relerr_tau(got, op[i], lr32)
            assert err <= (TOL_STEP1 if t == 1 else TOL_RUN), (t, i, err)
            copy = model[i].cpu().numpy().view(np.uint16)
            want = orc.round_model_copy(got, half)
            assert np.array_equal(copy, want), (t, i, np.flatnonzero(copy != want)[:5])
    if half:  # the edge tensor's copy holds fp16 subnormals and infinities
        last = model[-1].cpu().numpy().view(np.float16)
        assert np.isinf(last).any() and ((last != 0) & (np.abs(last) < np.float16(6.1e-5))).any()
    say(f"algo={algo} half={half}: master within bounds, model copy bit-exact")
