"""GPU parity of the loop around the fused step: the fused non-finite check
and global gradient norm (optim_grad_norm), clipping folded into the step's
inv_scale, and the dynamic loss-scale update (optim_scaler_update), against
the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle as orc
import optimizer_step_adamw_amd as osa
from gpu_support import DEV, TOL_RUN, TOL_STEP1, AdamState, relerr_tau, say, to_np_u16
from synth import host_normal

pytestmark = pytest.mark.gpu

RAGGED = [1, 7, 8, 9, 4095, 4096, 4097, 10007, 65539]
NORM_RTOL = 1e-6  # fp32 sums of squares per lane, fp64 beyond: ~1e-7 relative


def _scalars():
    z = lambda: torch.zeros(1, dtype=torch.float32, device=DEV)
    return z(), z(), z()  # found_inf, norm, clip


def _scaled_grads(state, sizes, key, t, scale):
    """Stored grads G = round(g * scale) (bf16 or fp32); returns G as float64."""
    out = []
    for i, (dst, n) in enumerate(zip(state.g, sizes)):
        g = torch.from_numpy(host_normal(n, 1e-3, 920, key, i, t)).to(DEV) * scale
        if state.grad_bf16:
            dst.copy_(g.to(torch.bfloat16).view(torch.int16))
            out.append(orc.bf16_bits_to_f64(to_np_u16(dst)))
        else:
            dst.copy_(g)
            out.append(dst.cpu().numpy().astype(np.float64))
    return out


@pytest.mark.parametrize("bf16,grid", [(True, 0), (False, 0), (True, 5)])
def test_grad_norm_and_clip_match_oracle(bf16, grid):
    sizes = RAGGED
    p0 = [np.zeros(n, np.float32) for n in sizes]
    st = AdamState([torch.from_numpy(x).to(DEV) for x in p0], grad_bf16=bf16)
    plan = osa.Plan(st.tensor_list([0.0] * len(sizes)), osa.OPTIM_ALGO_ADAMW, grid=grid)
    scale = 65536.0 if bf16 else 1024.0
    inv = torch.tensor([1.0 / scale], device=DEV)
    G = _scaled_grads(st, sizes, 1, 1, scale)
    norm_o = orc.grad_norm(G, 1.0 / scale)
    fi, norm, clip = _scalars()
    for max_norm in (0.5 * norm_o, 2.0 * norm_o, float("inf"), 0.0):
        fi.zero_()
        osa.optim_grad_norm(plan.handle, inv, max_norm, fi, norm, clip)
        assert fi.item() == 0.0
        assert abs(norm.item() - norm_o) <= NORM_RTOL * norm_o, (norm.item(), norm_o)
        want = (1.0 / scale) * orc.clip_coef(norm_o, max_norm)
        assert abs(clip.item() - want) <= NORM_RTOL * want, (max_norm, clip.item(), want)
        if not (0.0 < max_norm < norm_o):  # no clipping: exactly the input scale
            assert torch.equal(clip, inv)
    # a non-finite gradient anywhere sets found_inf; the clip factor stays s
    for i, pos in ((0, 0), (6, 4096), (8, 65538)):
        saved = st.g[i][pos].clone()
        bad = torch.tensor(float("nan") if i == 6 else float("-inf"))
        st.g[i][pos] = bad.to(torch.bfloat16).view(torch.int16) if bf16 else bad
        fi.zero_()
        osa.optim_grad_norm(plan.handle, inv, 0.1, fi, norm, clip)
        assert fi.item() == 1.0 and not np.isfinite(norm.item()) and torch.equal(clip, inv)
        st.g[i][pos] = saved
    # without inv_scale the norm is that of the stored gradients
    fi.zero_()
    osa.optim_grad_norm(plan.handle, None, float("inf"), fi, norm, clip)
    assert abs(norm.item() - orc.grad_norm(G)) <= NORM_RTOL * orc.grad_norm(G)
    assert clip.item() == 1.0
    say(f"bf16={bf16} grid={grid}: norm {norm_o:.6e} matches")


@pytest.mark.parametrize("bf16", [True, False])
def test_grad_norm_large_finite_gradients_clip(bf16):
    """Loss-scaled gradients whose squares overflow fp32 (|G| ~ 1e25, every
    element finite): the norm stays finite and matches the oracle's fp64
    norm, found_inf stays 0 and the clip factor follows oracle_clip_coef, as
    unscale-then-clip would ([LTN] analysis: clipping is why unscale_ runs
    before step).  Then the clipped step runs (it is not skipped)."""
    sizes = [4097, 65539, 9]
    p0 = [host_normal(n, 0.02, 921, 0, i, 0) for i, n in enumerate(sizes)]
    st = AdamState([torch.from_numpy(x).to(DEV) for x in p0], grad_bf16=bf16)
    plan = osa.Plan(st.tensor_list([0.1] * len(sizes)), osa.OPTIM_ALGO_ADAMW)
    scale = 2.0 ** 100  # stored |G| ~ 1e-3 * 2^100 ~ 1.3e27: G^2 ~ 1e54 > fp32 max
    inv = torch.tensor([2.0 ** -100], device=DEV)
    G = _scaled_grads(st, sizes, 7, 1, scale)
    assert all(np.all(np.isfinite(g)) for g in G) and max(np.max(np.abs(g)) for g in G) > 1.9e19
    norm_o = orc.grad_norm(G, 2.0 ** -100)
    fi, norm, clip = _scalars()
    max_norm = 0.25 * norm_o
    osa.optim_grad_norm(plan.handle, inv, max_norm, fi, norm, clip)
    assert fi.item() == 0.0
    assert np.isfinite(norm.item()) and abs(norm.item() - norm_o) <= NORM_RTOL * norm_o, (norm.item(), norm_o)
    want = 2.0 ** -100 * orc.clip_coef(norm_o, max_norm)
    assert abs(clip.item() - want) <= NORM_RTOL * want, (clip.item(), want)
    # the clipped step: found_inf 0, the step counter advances, p moves as
    # the oracle's step on the clipped, unscaled gradient
    lr = torch.tensor([1e-3], device=DEV)
    step = torch.zeros(1, dtype=torch.int32, device=DEV)
    hp = osa.optim_adamw_hp(0.9, 0.999, 1e-8)
    osa.optim_step_adamw(plan.handle, hp, lr, clip, fi, step)
    torch.cuda.synchronize()
    assert int(step.item()) == 1
    c = float(clip.item())
    lr32 = float(np.float32(1e-3))
    for i, n in enumerate(sizes):
        po, mo, vo = p0[i].astype(np.float64), np.zeros(n), np.zeros(n)
        # the step multiplies G by the fp32 clip factor, rounding g to fp32
        g = (G[i].astype(np.float32) * np.float32(c)).astype(np.float64)
        orc.adamw_step(po, mo, vo, g, lr32, 0.9, 0.999, 1e-8, 0.1, 1)
        assert relerr_tau(st.p[i].cpu().numpy(), po, lr32) <= TOL_STEP1
    say(f"bf16={bf16}: norm {norm_o:.6e} of gradients up to {max(np.max(np.abs(g)) for g in G):.3e} "
        f"clipped by {orc.clip_coef(norm_o, max_norm):.3f}")


def test_grad_norm_agrees_with_finite_check():
    """The fused pass sets found_inf exactly where optim_check_finite does
    (GPU against GPU, every position of a ragged tensor in turn)."""
    n = 4097
    st = AdamState([torch.zeros(n, device=DEV)], grad_bf16=True)
    plan = osa.Plan(st.tensor_list([0.0]), osa.OPTIM_ALGO_ADAMW)
    st.g[0].copy_(torch.ones(n, device=DEV).to(torch.bfloat16).view(torch.int16))
    fa, norm, clip = _scalars()
    fb = torch.zeros(1, device=DEV)
    for pos in (0, 1, 2, 3, 4, 1023, 1024, 2047, 4095, 4096):
        st.g[0][pos] = torch.tensor(float("inf")).to(torch.bfloat16).view(torch.int16)
        fa.zero_(); fb.zero_()
        osa.optim_grad_norm(plan.handle, None, 1.0, fa, norm, clip)
        osa.optim_check_finite(plan.handle, fb)
        assert fa.item() == fb.item() == 1.0, pos
        st.g[0][pos] = torch.tensor(1.0).to(torch.bfloat16).view(torch.int16)
    fa.zero_()
    osa.optim_grad_norm(plan.handle, None, float("inf"), fa, norm, clip)
    assert fa.item() == 0.0 and norm.item() == np.float32(np.sqrt(n))


def test_clipped_amp_loop_matches_oracle():
    """Ten iterations of scale -> check + norm -> clipped AdamW step -> scale
    update, bf16 params with remainders and bf16 grads, an overflow at
    iteration 5: params within the step bounds of the oracle's loop; scale,
    clean-step count and step counter bit for bit."""
    sizes = RAGGED
    lr, wd, max_norm = 1e-3, 0.1, 0.02
    p0 = [host_normal(n, 0.02, 921, 0, i, 0) for i, n in enumerate(sizes)]
    st = AdamState([torch.from_numpy(x).to(DEV) for x in p0], grad_bf16=True, param_bf16=True)
    plan = osa.Plan(st.tensor_list([wd] * len(sizes)), osa.OPTIM_ALGO_ADAMW)
    hp = osa.optim_adamw_hp(0.9, 0.95, 1e-8)
    lr_dev = torch.tensor([lr], device=DEV)
    step = torch.zeros(1, dtype=torch.int32, device=DEV)
    scale = torch.tensor([65536.0], device=DEV)
    inv = torch.tensor([1.0 / 65536.0], device=DEV)
    tracker = torch.zeros(1, dtype=torch.int32, device=DEV)
    fi, norm, clip = _scalars()
    ost = orc.ScalerState(65536.0)
    op = [x.astype(np.float64) for x in p0]
    om = [np.zeros(n) for n in sizes]
    ov = [np.zeros(n) for n in sizes]
    lr32 = float(np.float32(lr))
    t_or = 0
    clipped = 0
    for k in range(1, 11):
        S = float(ost.scale[0])
        G = _scaled_grads(st, sizes, 2, k, S)
        if k == 5:
            st.g[4][100] = torch.tensor(float("inf")).to(torch.bfloat16).view(torch.int16)
            G[4][100] = np.inf
        fi.zero_()
        osa.optim_grad_norm(plan.handle, inv, max_norm, fi, norm, clip)
        osa.optim_step_adamw(plan.handle, hp, lr_dev, clip, fi, step)
        osa.optim_scaler_update(scale, inv, tracker, fi, 2.0, 0.5, 3)
        found = any(orc.any_nonfinite(x) for x in G)
        assert fi.item() == float(found), k
        if not found:
            t_or += 1
            s = 1.0 / S
            nrm = orc.grad_norm(G, s)
            c = orc.clip_coef(nrm, max_norm)
            clipped += c < 1.0
            for i in range(len(sizes)):
                orc.adamw_step(op[i], om[i], ov[i], G[i] * s * c, lr32, 0.9, 0.95, 1e-8, wd, t_or)
        ost.update(found, 2.0, 0.5, 3)
        assert scale.cpu().numpy().view(np.uint32)[0] == ost.scale.view(np.uint32)[0], k
        assert inv.item() == np.float32(1.0 / np.float64(ost.scale[0])), k
        assert tracker.item() == ost.tracker[0] and step.item() == t_or, k
        err = max(relerr_tau(st.master(i).cpu().numpy(), op[i], lr32) for i in range(len(sizes)))
        assert err <= (TOL_STEP1 if t_or == 1 else TOL_RUN), (k, err)
    assert clipped >= 5 and t_or == 9
    say(f"clipped AMP loop: {t_or} applied steps, {clipped} clipped, final scale {ost.scale[0]}")


def test_scaler_update_matches_oracle():
    pattern = [0, 0, 0, 1, 0, 0, 0, 0, 0, 0, 1, 1, 0, 0, 0, 0, 0, 0, 0, 0]
    for scale0, growth, backoff, interval in ((65536.0, 2.0, 0.5, 3), (2.0 ** 126, 2.0, 0.5, 2),
                                               (3.0, 1.7, 0.3, 1)):
        scale = torch.tensor([scale0], device=DEV)
        inv = torch.zeros(1, device=DEV)
        tracker = torch.zeros(1, dtype=torch.int32, device=DEV)
        fi = torch.zeros(1, device=DEV)
        ost = orc.ScalerState(scale0)
        for f in pattern:
            fi.fill_(float(f))
            osa.optim_scaler_update(scale, inv, tracker, fi, growth, backoff, interval)
            ost.update(bool(f), growth, backoff, interval)
            assert scale.cpu().numpy().view(np.uint32)[0] == ost.scale.view(np.uint32)[0], (scale0, f)
            assert tracker.item() == ost.tracker[0]
            assert inv.cpu().numpy()[0] == np.float32(1.0 / np.float64(ost.scale[0]))
