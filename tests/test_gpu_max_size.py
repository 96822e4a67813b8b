"""GPU parity past 32-bit element and byte offsets: single tensors of more
than 2^31 elements (fp32 AdamW, the non-finite check and gradient norm,
8-bit blockwise) and of more than 2^32 elements (4-bit blockwise, whose
packed codes then pass 2^31 bytes).  The oracle follows windows at the
start, around the 2^31 (and 2^32) element boundaries and at the ragged end,
plus a seeded sample; every path here is elementwise or blockwise, so a
window is computed exactly as in the full run."""
import numpy as np
import pytest
import torch

import oracle as orc
import optimizer_step_adamw_amd as osa
import synth
from gpu_support import DEV, TOL_RUN, TOL_STEP1, DevScalars, QuantState, relerr_tau, say

pytestmark = pytest.mark.gpu

N31 = (1 << 31) + 4099   # ragged: not a multiple of a unit or of 4
HP = osa.optim_adamw_hp(0.9, 0.999, 1e-8)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _windows(n, align, key, w=4096):
    """Sorted element indices: windows of w (aligned to `align`) at the start,
    across 2^31 and 2^32 when inside, and at the end, plus 64 random aligned
    windows."""
    starts = [0, (1 << 31) - w // 2, (1 << 32) - w // 2, n - w]
    rng = synth.host_rng(990, key)
    starts += list(rng.integers(0, n - w, 64))
    idx = []
    for s in starts:
        s = max(0, min(int(s), n - w)) // align * align
        idx.append(np.arange(s, min(s + w, n)))
    return np.unique(np.concatenate(idx))


def test_adamw_fp32_past_2g_elements():
    n = N31
    p = synth.device_normal(n, 0.02, DEV, 990, 1)
    g = torch.empty(n, device=DEV)
    m, v = torch.zeros(n, device=DEV), torch.zeros(n, device=DEV)
    plan = osa.Plan(osa.TensorList([p], [g], m=[m], v=[v], weight_decay=[0.1]), osa.OPTIM_ALGO_ADAMW)
    sc = DevScalars(1e-3)
    lr32 = float(np.float32(1e-3))
    idx = _windows(n, 1, 1)
    di = torch.from_numpy(idx).to(DEV)
    op = p[di].double().cpu().numpy()
    om, ov = np.zeros(idx.size), np.zeros(idx.size)
    for t in (1, 2, 3):
        g.copy_(synth.device_normal(n, 1e-3, DEV, 990, 2, t))
        osa.optim_step_adamw(plan.handle, HP, sc.lr, None, None, sc.step)
        orc.adamw_step(op, om, ov, g[di].double().cpu().numpy(), lr32, 0.9, 0.999, 1e-8, 0.1, t)
        err = relerr_tau(p[di].cpu().numpy(), op, lr32)
        assert err <= (TOL_STEP1 if t == 1 else TOL_RUN), (t, err)
    say(f"AdamW n={n}: {idx.size} sampled elements, relerr_tau {err:.2e}")
    del p, g, m, v, plan
    _free()


def test_finite_check_and_norm_past_2g_elements():
    n = N31
    # the check and the norm read only the gradients, but a plan holds
    # param and state buffers of the tensor's size (bf16 + remainder here)
    p = torch.zeros(n, dtype=torch.int16, device=DEV)
    r = torch.zeros(n, dtype=torch.int16, device=DEV)
    gb = torch.full((n,), 0x3F80, dtype=torch.int16, device=DEV)  # bf16 1.0
    mm, vv = torch.zeros(n, device=DEV), torch.zeros(n, device=DEV)
    plan = osa.Plan(osa.TensorList([p], [gb], m=[mm], v=[vv], remainders=[r], weight_decay=[0.0],
                                   param_dtype=osa.OPTIM_BF16, grad_dtype=osa.OPTIM_BF16), osa.OPTIM_ALGO_ADAMW)
    fi, nrm, clip = torch.zeros(1, device=DEV), torch.zeros(1, device=DEV), torch.zeros(1, device=DEV)
    osa.optim_grad_norm(plan.handle, None, float("inf"), fi, nrm, clip)
    assert fi.item() == 0.0
    assert abs(nrm.item() - np.sqrt(n)) <= 1e-6 * np.sqrt(n), (nrm.item(), np.sqrt(n))
    inf16 = torch.tensor(float("inf")).to(torch.bfloat16).view(torch.int16)
    one16 = torch.tensor(1.0).to(torch.bfloat16).view(torch.int16)
    for pos in ((1 << 31) - 1, 1 << 31, n - 1):
        gb[pos] = inf16
        fi.zero_()
        osa.optim_check_finite(plan.handle, fi)
        assert fi.item() == 1.0, pos
        fi.zero_()
        osa.optim_grad_norm(plan.handle, None, 1.0, fi, nrm, clip)
        assert fi.item() == 1.0, pos
        gb[pos] = one16
    say(f"finite check and norm over {n} bf16 gradients: sqrt(n) and every planted inf found")
    del p, r, gb, mm, vv, plan
    _free()


@pytest.mark.parametrize("bits,n", [(8, (1 << 31) + 512 + 100), (4, (1 << 32) + 300)])
def test_blockwise_past_2g(bits, n):
    """8-bit: element offsets past 2^31; 4-bit: packed-code byte offsets past
    2^31.  Codes and absmax bit-exact on the windows (whole blocks), p within
    the step bounds, over two steps."""
    block = 256 if bits == 8 else 128
    p0 = synth.device_normal(n, 0.02, DEV, 991, bits)
    qs = QuantState([p0], bits, block)
    del p0
    _free()
    plan = osa.Plan(qs.tensor_list([0.01]), osa.OPTIM_ALGO_BLOCKWISE, bits=bits, block=block)
    sc = DevScalars(1e-3)
    lr32 = float(np.float32(1e-3))
    idx = _windows(n, block, bits, w=2048)
    # whole blocks only (the ragged last block included)
    blocks = np.unique(idx // block)
    idx = np.concatenate([np.arange(b * block, min((b + 1) * block, n)) for b in blocks])
    di = torch.from_numpy(idx).to(DEV)
    op = qs.p[0][di].double().cpu().numpy()
    k = idx.size
    qm, qv = np.zeros(k, np.uint8), np.zeros(k, np.uint8)
    am, av = np.zeros(blocks.size, np.float32), np.zeros(blocks.size, np.float32)
    # the oracle's blocks are consecutive runs of `block` elements of its
    # arrays: pad the ragged last block so the runs line up
    pad = (-k) % block
    for t in (1, 2):
        qs.g[0].copy_(synth.device_normal(n, 1e-3, DEV, 991, 10 + bits, t))
        osa.optim_step_8bit_blockwise(plan.handle, HP, bits, block, sc.lr, None, None, sc.step)
        g = qs.g[0][di].cpu().numpy()
        pp = np.concatenate([op, np.zeros(pad)])
        gg = np.concatenate([g, np.zeros(pad, np.float32)])
        qmp, qvp = np.concatenate([qm, np.zeros(pad, np.uint8)]), np.concatenate([qv, np.zeros(pad, np.uint8)])
        orc.blockwise_step(pp, gg, qmp, qvp, am, av, bits, block, lr32, 0.9, 0.999, 1e-8, 0.01, t)
        op, qm, qv = pp[:k], qmp[:k], qvp[:k]
        bi = torch.from_numpy(blocks).to(DEV)
        assert np.array_equal(qs.am[0][bi].cpu().numpy().view(np.uint32), am.view(np.uint32)), t
        assert np.array_equal(qs.av[0][bi].cpu().numpy().view(np.uint32), av.view(np.uint32)), t
        if bits == 8:
            gm, gv = qs.qm[0][di].cpu().numpy(), qs.qv[0][di].cpu().numpy()
        else:
            byte_idx = torch.from_numpy(np.unique(idx // 2)).to(DEV)
            gm = orc.unpack_nibbles(qs.qm[0][byte_idx].cpu().numpy(), k)
            gv = orc.unpack_nibbles(qs.qv[0][byte_idx].cpu().numpy(), k)
        assert np.array_equal(gm, qm), (t, int(np.sum(gm != qm)))
        assert np.array_equal(gv, qv), (t, int(np.sum(gv != qv)))
        err = relerr_tau(qs.p[0][di].cpu().numpy(), op, lr32)
        assert err <= (TOL_STEP1 if t == 1 else TOL_RUN), (t, err)
    say(f"blockwise {bits}-bit n={n}: {blocks.size} sampled blocks bit-exact, relerr_tau {err:.2e}")
    del qs, plan
    _free()


@pytest.mark.parametrize("bits,n", [(8, (1 << 30) + 512 + 100), (4, (1 << 31) + 300)])
def test_blockwise_interleaved_past_2g(bits, n):
    """Interleaved layout (each element's m and v codes side by side, the two
    absmax values of a block side by side): 8-bit takes 2 code bytes per
    element and 4-bit 1, so both tensors put code byte offsets past 2^31.
    Codes and absmax bit-exact on the windows (whole blocks), p within the
    step bounds, over two steps."""
    block = 256 if bits == 8 else 128
    nblk = (n + block - 1) // block
    p = synth.device_normal(n, 0.02, DEV, 993, bits)
    g = torch.empty_like(p)
    q = torch.zeros(n * bits // 4, dtype=torch.uint8, device=DEV)
    a = torch.zeros(2 * nblk, dtype=torch.float32, device=DEV)
    plan = osa.Plan(osa.TensorList([p], [g], qm=[q], absmax_m=[a], weight_decay=[0.01]), osa.OPTIM_ALGO_BLOCKWISE,
                    bits=bits, block=block, state_layout=osa.OPTIM_LAYOUT_INTERLEAVED)
    sc = DevScalars(1e-3)
    lr32 = float(np.float32(1e-3))
    idx = _windows(n, block, 20 + bits, w=2048)
    blocks = np.unique(idx // block)
    idx = np.concatenate([np.arange(b * block, min((b + 1) * block, n)) for b in blocks])
    di = torch.from_numpy(idx).to(DEV)
    op = p[di].double().cpu().numpy()
    k = idx.size
    qm, qv = np.zeros(k, np.uint8), np.zeros(k, np.uint8)
    am, av = np.zeros(blocks.size, np.float32), np.zeros(blocks.size, np.float32)
    pad = (-k) % block
    if bits == 8:
        code_idx = torch.from_numpy(np.stack([2 * idx, 2 * idx + 1], axis=1).ravel()).to(DEV)
    else:
        code_idx = di
    amax_idx = torch.from_numpy(np.stack([2 * blocks, 2 * blocks + 1], axis=1).ravel()).to(DEV)
    for t in (1, 2):
        g.copy_(synth.device_normal(n, 1e-3, DEV, 993, 10 + bits, t))
        osa.optim_step_8bit_blockwise(plan.handle, HP, bits, block, sc.lr, None, None, sc.step)
        gw = g[di].cpu().numpy()
        pp = np.concatenate([op, np.zeros(pad)])
        gg = np.concatenate([gw, np.zeros(pad, np.float32)])
        qmp, qvp = np.concatenate([qm, np.zeros(pad, np.uint8)]), np.concatenate([qv, np.zeros(pad, np.uint8)])
        orc.blockwise_step(pp, gg, qmp, qvp, am, av, bits, block, lr32, 0.9, 0.999, 1e-8, 0.01, t)
        op, qm, qv = pp[:k], qmp[:k], qvp[:k]
        want_a = np.stack([am, av], axis=1).ravel().view(np.uint32)
        assert np.array_equal(a[amax_idx].cpu().numpy().view(np.uint32), want_a), t
        got = q[code_idx].cpu().numpy()
        if bits == 8:
            gm, gv = got[0::2], got[1::2]
        else:
            gm, gv = got & 0xF, got >> 4
        assert np.array_equal(gm, qm), (t, int(np.sum(gm != qm)))
        assert np.array_equal(gv, qv), (t, int(np.sum(gv != qv)))
        err = relerr_tau(p[di].cpu().numpy(), op, lr32)
        assert err <= (TOL_STEP1 if t == 1 else TOL_RUN), (t, err)
    say(f"blockwise {bits}-bit interleaved n={n}: {blocks.size} sampled blocks bit-exact, relerr_tau {err:.2e}")
    del p, g, q, a, plan
    _free()
