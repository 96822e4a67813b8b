"""Lists of very many small tensors against the oracle: 20,000 tensors of
1-300 elements (seeded sizes), about one in ten starting off a 16-byte
boundary, with three weight-decay groups.  The AdamW, AdEMAMix and Lion
plans lay such tensors end to end in shared units (packs); the tests run
three steps of each (fp32 params and grads; and AdamW with bf16 params +
int16 remainders, bf16 grads and a loss scale) and check every element
against the oracle, the non-finite check and the gradient norm over the
packed list, and Adam-mini over the same sizes as 20,000 one-block (SCALAR)
tensors.

The oracle runs on the concatenation of all tensors of one weight-decay
group (the AdamW-family updates are elementwise, so this is the same
arithmetic), and Adam-mini on the concatenation of the tensors of one size
and group with a block of that size."""
import numpy as np
import pytest
import torch

import oracle as orc
import optimizer_step_adamw_amd as osa
import synth
from gpu_support import DEV, TOL_RUN, TOL_STEP1, relerr_tau, say

pytestmark = pytest.mark.gpu

N_T = 20000
WD = (0.0, 0.01, 0.1)


def layout():
    rng = synth.host_rng(990, 0)
    sizes = rng.integers(1, 301, N_T)
    unaligned = rng.random(N_T) < 0.1
    wd = rng.choice(len(WD), N_T)
    offs = np.empty(N_T, np.int64)
    pos = 0
    for i in range(N_T):
        pos = (pos + 7) // 8 * 8 + (1 if unaligned[i] else 0)  # 16 B for fp32 and 16-bit arrays, or 1 element off
        offs[i] = pos
        pos += sizes[i]
    return sizes, offs, wd, pos


SIZES, OFFS, WDI, TOTAL = layout()
# element indices of each weight-decay group, in list order
GROUP_IDX = [np.concatenate([np.arange(OFFS[i], OFFS[i] + SIZES[i]) for i in range(N_T) if WDI[i] == w])
             for w in range(len(WD))]


def views(buf):
    return [buf[o:o + n] for o, n in zip(OFFS.tolist(), SIZES.tolist())]


def host(n, *key):
    return synth.host_normal(n, 1.0, 991, *key)


P0 = host(TOTAL, 0) * np.float32(0.02)


def grads(t):
    return host(TOTAL, t) * np.float32(1e-3)


def check_p(p_dev, ref, tol, lr32):
    p = p_dev.cpu().numpy()
    worst = max(relerr_tau(p[idx], ref[w], lr32) for w, idx in enumerate(GROUP_IDX))
    assert worst <= tol, worst
    return worst


@pytest.mark.parametrize("algo", ["adamw", "ademamix", "lion"])
def test_tiny_tensors_fp32(algo):
    print(f"case: {N_T} tiny tensors, {algo}", flush=True)
    lr = 1e-4 if algo == "lion" else 1e-3
    lr32 = float(np.float32(lr))
    P = torch.from_numpy(P0.copy()).to(DEV)
    G = torch.zeros(TOTAL, device=DEV)
    M = torch.zeros(TOTAL, device=DEV)
    V = torch.zeros(TOTAL, device=DEV)
    M2 = torch.zeros(TOTAL, device=DEV)
    kw = dict(m=views(M), weight_decay=[WD[w] for w in WDI])
    if algo != "lion":
        kw["v"] = views(V)
    if algo == "ademamix":
        kw["m2"] = views(M2)
    algo_id = dict(adamw=osa.OPTIM_ALGO_ADAMW, ademamix=osa.OPTIM_ALGO_ADEMAMIX, lion=osa.OPTIM_ALGO_LION)[algo]
    plan = osa.Plan(osa.TensorList(views(P), views(G), **kw), algo_id)
    lr_d = torch.tensor([lr], device=DEV)
    step = torch.zeros(1, dtype=torch.int32, device=DEV)
    ref = [P0[idx].astype(np.float64) for idx in GROUP_IDX]
    om = [np.zeros(idx.size) for idx in GROUP_IDX]
    ov = [np.zeros(idx.size) for idx in GROUP_IDX]
    om2 = [np.zeros(idx.size) for idx in GROUP_IDX]
    om32 = [np.zeros(idx.size, np.float32) for idx in GROUP_IDX]
    for t in (1, 2, 3):
        g = grads(t)
        G.copy_(torch.from_numpy(g))
        if algo == "adamw":
            osa.optim_step_adamw(plan.handle, osa.optim_adamw_hp(0.9, 0.999, 1e-8), lr_d, None, None, step)
        elif algo == "ademamix":
            osa.optim_step_ademamix(plan.handle, osa.optim_ademamix_hp(0.9, 0.999, 0.9999, 5.0, 1e-8), lr_d, None,
                                    None, step)
        else:
            osa.optim_step_lion(plan.handle, osa.optim_lion_hp(0.9, 0.99), lr_d, None, None, step)
        for w, idx in enumerate(GROUP_IDX):
            if algo == "adamw":
                orc.adamw_step(ref[w], om[w], ov[w], g[idx], lr32, 0.9, 0.999, 1e-8, WD[w], t)
            elif algo == "ademamix":
                orc.ademamix_step(ref[w], om[w], om2[w], ov[w], g[idx], lr32, 0.9, 0.999, 0.9999, 5.0, 1e-8, WD[w], t)
            else:
                orc.lion_step(ref[w], om32[w], g[idx], lr32, 0.9, 0.99, WD[w])
        worst = check_p(P, ref, TOL_STEP1 if t == 1 else TOL_RUN, lr32)
    if algo == "lion":  # the fp32 state recipe: m bit for bit
        m = M.cpu().numpy()
        for w, idx in enumerate(GROUP_IDX):
            assert np.array_equal(m[idx].view(np.uint32), om32[w].view(np.uint32))
    assert int(step.item()) == 3
    say(f"{algo}: {N_T} tensors of 1-300 elements, 3 steps, max relerr_tau {worst:.2e}")
    plan.close()


def test_tiny_tensors_bf16_remainder_amp_and_norm():
    print(f"case: {N_T} tiny tensors, AdamW bf16 + remainder, bf16 grads x 1024, check + norm", flush=True)
    lr, scale = 1e-3, 1024.0
    lr32 = float(np.float32(lr))
    Pb = torch.zeros(TOTAL, dtype=torch.int16, device=DEV)
    R = torch.zeros(TOTAL, dtype=torch.int16, device=DEV)
    osa.optim_remainder_split(torch.from_numpy(P0).to(DEV), Pb, R, TOTAL)
    G = torch.zeros(TOTAL, dtype=torch.int16, device=DEV)
    M = torch.zeros(TOTAL, device=DEV)
    V = torch.zeros(TOTAL, device=DEV)
    tl = osa.TensorList(views(Pb), views(G), m=views(M), v=views(V), remainders=views(R),
                        weight_decay=[WD[w] for w in WDI], param_dtype=osa.OPTIM_BF16, grad_dtype=osa.OPTIM_BF16)
    plan = osa.Plan(tl, osa.OPTIM_ALGO_ADAMW)
    lr_d = torch.tensor([lr], device=DEV)
    inv = torch.tensor([1.0 / scale], device=DEV)
    fi = torch.zeros(1, device=DEV)
    step = torch.zeros(1, dtype=torch.int32, device=DEV)
    norm, clip = torch.zeros(1, device=DEV), torch.zeros(1, device=DEV)
    ref = [P0[idx].astype(np.float64) for idx in GROUP_IDX]
    om = [np.zeros(idx.size) for idx in GROUP_IDX]
    ov = [np.zeros(idx.size) for idx in GROUP_IDX]
    master = torch.zeros(TOTAL, device=DEV)
    hp = osa.optim_adamw_hp(0.9, 0.95, 1e-8)
    for t in (1, 2, 3):
        G.copy_((torch.from_numpy(grads(t)).to(DEV) * scale).to(torch.bfloat16).view(torch.int16))
        Gh = orc.bf16_bits_to_f64(G.cpu().numpy().view(np.uint16))
        if t == 2:  # an overflow in one small, unaligned tensor: found_inf, the step is skipped
            i = int(np.flatnonzero(OFFS % 8 == 1)[123])
            G[int(OFFS[i]) + int(SIZES[i]) - 1] = torch.tensor(float("inf")).to(torch.bfloat16).view(torch.int16)
        fi.zero_()
        osa.optim_grad_norm(plan.handle, inv, float("inf"), fi, norm, clip)
        if t == 2:
            assert fi.item() == 1.0
        else:
            assert fi.item() == 0.0
            want = orc.grad_norm([Gh[idx] for idx in GROUP_IDX], 1.0 / scale)
            assert abs(norm.item() - want) <= 1e-6 * want, (norm.item(), want)
            # the plain check agrees
            fi.zero_()
            osa.optim_check_finite(plan.handle, fi)
            assert fi.item() == 0.0
        osa.optim_step_adamw(plan.handle, hp, lr_d, inv, fi, step)
        if t != 2:
            tt = 1 if t == 1 else 2
            for w, idx in enumerate(GROUP_IDX):
                orc.adamw_step(ref[w], om[w], ov[w], Gh[idx] / scale, lr32, 0.9, 0.95, 1e-8, WD[w], tt)
        osa.optim_remainder_reconstruct(Pb, R, master, TOTAL)
        worst = check_p(master, ref, TOL_STEP1 if t == 1 else TOL_RUN, lr32)
    assert int(step.item()) == 2
    say(f"bf16 + remainder: {N_T} tensors, 2 applied steps and a skipped one, max relerr_tau {worst:.2e}")
    plan.close()


def test_tiny_tensors_adam_mini_scalar():
    print(f"case: {N_T} tiny tensors, Adam-mini, one shared v per tensor", flush=True)
    lr = 1e-3
    lr32 = float(np.float32(lr))
    P = torch.from_numpy(P0.copy()).to(DEV)
    G = torch.zeros(TOTAL, device=DEV)
    M = torch.zeros(TOTAL, device=DEV)
    Vb = torch.zeros(N_T, device=DEV)
    kinds = [osa.OPTIM_MINI_SCALAR] * N_T
    tl = osa.TensorList(views(P), views(G), m=views(M), v=[Vb[i:i + 1] for i in range(N_T)],
                        weight_decay=[WD[w] for w in WDI], mini_kind=kinds, head_numel=SIZES.tolist())
    plan = osa.Plan(tl, osa.OPTIM_ALGO_ADAM_MINI)
    lr_d = torch.tensor([lr], device=DEV)
    step = torch.zeros(1, dtype=torch.int32, device=DEV)
    hp = osa.optim_adamw_hp(0.9, 0.95, 1e-8)
    # oracle groups: tensors of one size and weight-decay group, concatenated
    groups = {}
    for i in range(N_T):
        groups.setdefault((int(SIZES[i]), int(WDI[i])), []).append(i)
    gidx = {k: np.concatenate([np.arange(OFFS[i], OFFS[i] + SIZES[i]) for i in v]) for k, v in groups.items()}
    ref = {k: P0[ix].astype(np.float64) for k, ix in gidx.items()}
    om = {k: np.zeros(ix.size) for k, ix in gidx.items()}
    oV = {k: np.zeros(len(groups[k])) for k in gidx}
    for t in (1, 2, 3):
        g = grads(t)
        G.copy_(torch.from_numpy(g))
        osa.optim_step_adam_mini(plan.handle, hp, lr_d, None, None, step)
        for (n, w), ix in gidx.items():
            orc.adam_mini_step(ref[(n, w)], om[(n, w)], oV[(n, w)], g[ix], n, lr32, 0.9, 0.95, 1e-8, WD[w], t)
        p = P.cpu().numpy()
        worst = max(relerr_tau(p[ix], ref[k], lr32) for k, ix in gidx.items())
        assert worst <= (TOL_STEP1 if t == 1 else TOL_RUN), worst
    vb = Vb.cpu().numpy()
    for k, members in groups.items():
        assert np.allclose(vb[members], oV[k], rtol=1e-6, atol=0)
    say(f"Adam-mini: {N_T} one-block tensors, 3 steps, max relerr_tau {worst:.2e}")
    plan.close()


# Launch shapes of the pack kernels: the default grid (a pack per workgroup,
# loads before the prologue), smaller and larger units (pack capacity
# follows min(unit, 2048)) and persistent grids (packs walked after the
# prologue).  The step is elementwise, so every shape gives the same bits.
FORMS = ((0, 0), (1024, 0), (8192, 0), (0, 13), (4096, 5))


def _forms_layout():
    rng = synth.host_rng(992, 0)
    sizes = [int(x) for x in rng.integers(1, 701, 2000)] + [100003]
    offs, pos = [], 0
    for i, n in enumerate(sizes):
        pos = (pos + 7) // 8 * 8 + (1 if rng.random() < 0.1 else 0)
        offs.append(pos)
        pos += n
    return sizes, offs, pos


@pytest.mark.parametrize("algo", ["adamw", "ademamix", "lion"])
def test_pack_launch_forms_give_the_same_bits(algo):
    print(f"case: pack launch forms, {algo}", flush=True)
    sizes, offs, total = _forms_layout()
    vw = lambda buf: [buf[o:o + n] for o, n in zip(offs, sizes)]
    p0 = synth.host_normal(total, 0.02, 993, 0)
    gs = [synth.host_normal(total, 1e-3, 993, t) for t in (1, 2)]
    wd = [WD[i % 3] for i in range(len(sizes))]
    algo_id = dict(adamw=osa.OPTIM_ALGO_ADAMW, ademamix=osa.OPTIM_ALGO_ADEMAMIX, lion=osa.OPTIM_ALGO_LION)[algo]
    results = []
    for tile, grid in FORMS:
        P = torch.from_numpy(p0.copy()).to(DEV)
        G = torch.zeros(total, device=DEV)
        M, V, M2 = (torch.zeros(total, device=DEV) for _ in range(3))
        kw = dict(m=vw(M), weight_decay=wd)
        if algo != "lion":
            kw["v"] = vw(V)
        if algo == "ademamix":
            kw["m2"] = vw(M2)
        plan = osa.Plan(osa.TensorList(vw(P), vw(G), **kw), algo_id, tile=tile, grid=grid)
        lr_d = torch.tensor([1e-3], device=DEV)
        step = torch.zeros(1, dtype=torch.int32, device=DEV)
        for g in gs:
            G.copy_(torch.from_numpy(g))
            if algo == "adamw":
                osa.optim_step_adamw(plan.handle, osa.optim_adamw_hp(0.9, 0.999, 1e-8), lr_d, None, None, step)
            elif algo == "ademamix":
                osa.optim_step_ademamix(plan.handle, osa.optim_ademamix_hp(0.9, 0.999, 0.9999, 5.0, 1e-8), lr_d,
                                        None, None, step)
            else:
                osa.optim_step_lion(plan.handle, osa.optim_lion_hp(0.9, 0.99), lr_d, None, None, step)
        assert int(step.item()) == 2
        results.append([x.cpu().numpy().view(np.uint32) for x in (P, M, V, M2)])
        plan.close()
    for (tile, grid), r in zip(FORMS[1:], results[1:]):
        for a, b in zip(results[0], r):
            assert np.array_equal(a, b), (algo, tile, grid, np.flatnonzero(a != b)[:8])
    say(f"{algo}: {len(sizes)} tensors, {len(FORMS)} launch shapes, identical bits")
