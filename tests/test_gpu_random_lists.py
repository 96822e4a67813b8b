"""Seeded random tensor lists against the oracle: each case draws an
algorithm (AdamW, AdEMAMix, Lion, LAMB, blockwise 8/4-bit, AdamW with fp16 /
bf16 moments), a list of 1-6 tensors of random sizes (empty, tiny, ragged,
several units), the param and grad formats the algorithm takes, a power-of-
two loss scale, and the launch shape (default or persistent grid, tile).
Three steps each; the states that follow the fixed fp32 recipe (Lion's m,
blockwise codes and absmax, 16-bit moments and their scales) are compared
bit for bit, the parameters within the step bounds."""
import numpy as np
import pytest
import torch

import oracle as orc
import optimizer_step_adamw_amd as osa
import synth
from gpu_support import DEV, TOL_RUN, TOL_STEP1, AdamState, DevScalars, QuantState, relerr_tau, say, to_np_u16

pytestmark = pytest.mark.gpu

ALGOS = ["adamw", "ademamix", "lion", "lamb", "blockwise8", "blockwise4", "f16", "bf16"]
N_CASES = 48


def _draw(case):
    rng = synth.host_rng(980, case)
    algo = ALGOS[case % len(ALGOS)]
    nt = int(rng.integers(1, 7))
    sizes = []
    for _ in range(nt):
        kind = rng.integers(0, 4)
        sizes.append(int([0, rng.integers(1, 64), rng.integers(64, 9000), rng.integers(9000, 70000)][kind]))
    blockwise = algo.startswith("blockwise")
    param_bf16 = (not blockwise) and bool(rng.integers(0, 2))
    grad_bf16 = bool(rng.integers(0, 2))
    scale = float(2.0 ** int(rng.integers(0, 17)))
    grid = int(rng.choice([0, 0, 3, 17]))
    if blockwise:
        bits = 8 if algo == "blockwise8" else 4
        block = int(rng.choice([64, 128, 256] if bits == 8 else [128, 256, 512]))
        tile = int(rng.choice([0, 2048, 4096]))
    else:
        bits = block = 0
        tile = int(rng.choice([0, 1024, 2048, 4096]))
    wd = [float(rng.choice([0.0, 0.01, 0.1])) for _ in sizes]
    lr = float(rng.choice([1e-4, 1e-3, 1e-2]))
    return dict(algo=algo, sizes=sizes, param_bf16=param_bf16, grad_bf16=grad_bf16, scale=scale, grid=grid,
                tile=tile, bits=bits, block=block, wd=wd, lr=lr)


def _set_grads(st, sizes, case, t, scale, grad_bf16):
    """Stored G = g*scale (bf16 rounded or fp32); returns the fp32 gradient
    the step sees, G / scale (exact)."""
    out = []
    for i, n in enumerate(sizes):
        g = torch.from_numpy(synth.host_normal(n, 1e-3, 981, case, i, t)).to(DEV) * scale
        if grad_bf16:
            st.g[i].copy_(g.to(torch.bfloat16).view(torch.int16))
            G = orc.bf16_bits_to_f64(to_np_u16(st.g[i]))
        else:
            st.g[i].copy_(g)
            G = st.g[i].cpu().numpy().astype(np.float64)
        out.append((G / scale).astype(np.float32))
    return out


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_list_matches_oracle(case):
    c = _draw(case)
    algo, sizes, scale = c["algo"], c["sizes"], c["scale"]
    p0 = [synth.host_normal(n, 0.02, 982, case, i, 0) for i, n in enumerate(sizes)]
    dev_p0 = [torch.from_numpy(x).to(DEV) for x in p0]
    gdt = osa.OPTIM_BF16 if c["grad_bf16"] else osa.OPTIM_F32
    pdt = osa.OPTIM_BF16 if c["param_bf16"] else osa.OPTIM_F32
    opts = dict(grid=c["grid"], tile=c["tile"])
    if algo.startswith("blockwise"):
        st = QuantState(dev_p0, c["bits"], c["block"])
        st.grad_bf16 = c["grad_bf16"]
        if c["grad_bf16"]:
            st.g = [torch.zeros(n, dtype=torch.int16, device=DEV) for n in sizes]
        tl = osa.TensorList(st.p, st.g, qm=st.qm, qv=st.qv, absmax_m=st.am, absmax_v=st.av, weight_decay=c["wd"],
                            grad_dtype=gdt)
        plan = osa.Plan(tl, osa.OPTIM_ALGO_BLOCKWISE, bits=c["bits"], block=c["block"], **opts)
    else:
        st = AdamState(dev_p0, grad_bf16=c["grad_bf16"], param_bf16=c["param_bf16"], ademamix=algo == "ademamix")
        kw = dict(remainders=st.r, weight_decay=c["wd"], param_dtype=pdt, grad_dtype=gdt)
        if algo in ("f16", "bf16"):
            st.m = [torch.zeros(n, dtype=torch.int16, device=DEV) for n in sizes]
            st.v = [torch.zeros(n, dtype=torch.int16, device=DEV) for n in sizes]
            sm = [torch.ones(1, device=DEV) for _ in sizes]
            sv = [torch.ones(1, device=DEV) for _ in sizes]
            tl = osa.TensorList(st.p, st.g, m=st.m, v=st.v, scale_m=sm, scale_v=sv, **kw)
            plan = osa.Plan(tl, osa.OPTIM_ALGO_ADAMW, state_dtype=osa.OPTIM_F16 if algo == "f16" else osa.OPTIM_BF16,
                            **opts)
        else:
            code = dict(adamw=osa.OPTIM_ALGO_ADAMW, ademamix=osa.OPTIM_ALGO_ADEMAMIX, lion=osa.OPTIM_ALGO_LION,
                        lamb=osa.OPTIM_ALGO_LAMB)[algo]
            tl = osa.TensorList(st.p, st.g, m=st.m, v=None if algo == "lion" else st.v, m2=st.m2, **kw)
            plan = osa.Plan(tl, code, **opts)
    sc = DevScalars(c["lr"], None if scale == 1.0 else 1.0 / scale)
    lr32 = float(np.float32(c["lr"]))
    hp = osa.optim_adamw_hp(0.9, 0.999, 1e-8)
    hpe = osa.optim_ademamix_hp(0.9, 0.999, 0.9999, 5.0, 1e-8)
    # oracle state
    op = [x.astype(np.float64) for x in p0]
    om = [np.zeros(n) for n in sizes]
    ov = [np.zeros(n) for n in sizes]
    om2 = [np.zeros(n) for n in sizes]
    om32 = [np.zeros(n, np.float32) for n in sizes]
    oq = [(np.zeros(n, np.uint8), np.zeros(n, np.uint8), np.zeros((n + max(c["block"], 1) - 1) // max(c["block"], 1),
                                                                   np.float32),
           np.zeros((n + max(c["block"], 1) - 1) // max(c["block"], 1), np.float32)) for n in sizes]
    o16 = [(np.zeros(n, np.uint16), np.zeros(n, np.uint16), np.ones(1, np.float32), np.ones(1, np.float32))
           for n in sizes]
    for t in (1, 2, 3):
        g = _set_grads(st, sizes, case, t, scale, c["grad_bf16"])
        if algo == "adamw" or algo in ("f16", "bf16"):
            osa.optim_step_adamw(plan.handle, hp, sc.lr, sc.inv_scale, None, sc.step)
        elif algo == "ademamix":
            osa.optim_step_ademamix(plan.handle, hpe, sc.lr, sc.inv_scale, None, sc.step)
        elif algo == "lion":
            osa.optim_step_lion(plan.handle, osa.optim_lion_hp(0.9, 0.99), sc.lr, sc.inv_scale, None, sc.step)
        elif algo == "lamb":
            osa.optim_step_lamb(plan.handle, hp, sc.lr, sc.inv_scale, None, sc.step)
        else:
            osa.optim_step_8bit_blockwise(plan.handle, hp, c["bits"], c["block"], sc.lr, sc.inv_scale, None,
                                          sc.step)
        for i, n in enumerate(sizes):
            gi = g[i]
            if algo == "adamw":
                orc.adamw_step(op[i], om[i], ov[i], gi.astype(np.float64), lr32, 0.9, 0.999, 1e-8, c["wd"][i], t)
            elif algo == "ademamix":
                orc.ademamix_step(op[i], om[i], om2[i], ov[i], gi.astype(np.float64), lr32, 0.9, 0.999, 0.9999, 5.0,
                                  1e-8, c["wd"][i], t)
            elif algo == "lion":
                orc.lion_step(op[i], om32[i], gi, lr32, 0.9, 0.99, c["wd"][i])
                assert np.array_equal(st.m[i].cpu().numpy().view(np.uint32), om32[i].view(np.uint32)), (c, t, i)
            elif algo == "lamb":
                orc.lamb_step(op[i], om[i], ov[i], gi.astype(np.float64), lr32, 0.9, 0.999, 1e-8, c["wd"][i], t)
            elif algo in ("f16", "bf16"):
                qm, qv, sm_o, sv_o = o16[i]
                orc.adamw_scaled_step(op[i], qm, qv, sm_o, sv_o, gi, algo == "f16", lr32, 0.9, 0.999, 1e-8,
                                      c["wd"][i], t)
                assert np.array_equal(to_np_u16(st.m[i]), qm) and np.array_equal(to_np_u16(st.v[i]), qv), (c, t, i)
                assert sm[i].cpu().numpy().view(np.uint32)[0] == sm_o.view(np.uint32)[0], (c, t, i)
                assert sv[i].cpu().numpy().view(np.uint32)[0] == sv_o.view(np.uint32)[0], (c, t, i)
            else:
                qm, qv, am, av = oq[i]
                orc.blockwise_step(op[i], gi, qm, qv, am, av, c["bits"], c["block"], lr32, 0.9, 0.999, 1e-8,
                                   c["wd"][i], t)
                if n:
                    assert np.array_equal(st.am[i].cpu().numpy().view(np.uint32), am.view(np.uint32)), (c, t, i)
                    assert np.array_equal(st.av[i].cpu().numpy().view(np.uint32), av.view(np.uint32)), (c, t, i)
                    if c["bits"] == 8:
                        gm, gv = st.qm[i].cpu().numpy(), st.qv[i].cpu().numpy()
                    else:
                        gm = orc.unpack_nibbles(st.qm[i].cpu().numpy(), n)
                        gv = orc.unpack_nibbles(st.qv[i].cpu().numpy(), n)
                    assert np.array_equal(gm, qm) and np.array_equal(gv, qv), (c, t, i)
            got = st.master(i).cpu().numpy() if not algo.startswith("blockwise") else st.p[i].cpu().numpy()
            err = relerr_tau(got, op[i], lr32)
            assert err <= (TOL_STEP1 if t == 1 else TOL_RUN), (c, t, i, err)
        assert int(sc.step.item()) == t
    say(f"case {case}: {algo} sizes={sizes} pbf16={c['param_bf16']} gbf16={c['grad_bf16']} scale={scale} "
        f"grid={c['grid']} tile={c['tile']} ok")
