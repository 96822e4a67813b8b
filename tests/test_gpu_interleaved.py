"""GPU parity of the blockwise 8-bit / 4-bit step in the interleaved state
layout (each element's m and v codes side by side in one array, the two
absmax values of a block side by side in another) against the CPU oracle,
which keeps the states apart: the codes and absmax after every step equal
the oracle's, rearranged into the interleaved layout, bit for bit; p within
the step bounds.  Sizes span several rows, whole and ragged blocks."""
import numpy as np
import pytest
import torch

import oracle as orc
import optimizer_step_adamw_amd as osa
from gpu_support import DEV, TOL_RUN, TOL_STEP1, DevScalars, all_equal, relerr_tau, say
from synth import host_normal

pytestmark = pytest.mark.gpu

SIZES = [77, 1000, 4096, 5000, 3 * 4096 + 2 * 256 + 13, 2 * 16384 + 300]


def interleave(qm, qv, bits):
    """Unpacked codes (one per element) -> the interleaved bytes: 8-bit m, v
    per element; 4-bit m in the low nibble, v in the high one."""
    qm, qv = qm.astype(np.uint8), qv.astype(np.uint8)
    if bits == 8:
        return np.stack([qm, qv], axis=1).ravel()
    return qm | (qv << 4)


class ILState:
    def __init__(self, p0, bits, block, code_offset=0):
        self.p = [torch.from_numpy(x).to(DEV) for x in p0]
        self.g = [torch.zeros_like(x) for x in self.p]
        # code_offset > 0: codes start that many bytes past a 16-byte boundary,
        # so every row takes the byte-wise path
        self.q = [torch.zeros(x.size * 2 * bits // 8 + code_offset, dtype=torch.uint8, device=DEV)[code_offset:]
                  for x in p0]
        self.a = [torch.zeros(2 * ((x.size + block - 1) // block), dtype=torch.float32, device=DEV) for x in p0]

    def plan(self, bits, block, wd, grad_bf16=False, tile=0, grid=0):
        tl = osa.TensorList(self.p, self.g, qm=self.q, absmax_m=self.a, weight_decay=wd,
                            grad_dtype=osa.OPTIM_BF16 if grad_bf16 else osa.OPTIM_F32)
        return osa.Plan(tl, osa.OPTIM_ALGO_BLOCKWISE, bits=bits, block=block, tile=tile, grid=grid,
                        state_layout=osa.OPTIM_LAYOUT_INTERLEAVED)


@pytest.mark.parametrize("bits,block,tile,code_offset,grid", [(8, 256, 0, 0, 0), (4, 128, 0, 0, 0), (8, 64, 0, 0, 0),
                                                              (4, 512, 0, 0, 0), (8, 256, 2048, 0, 0),
                                                              (4, 128, 16384, 0, 0), (8, 256, 0, 3, 0),
                                                              (4, 512, 0, 5, 0), (8, 256, 2048, 0, 7)])
def test_interleaved_codes_bit_exact(bits, block, tile, code_offset, grid):
    lr, wd = 1e-3, 0.01
    p0 = [host_normal(n, 0.02, 940, bits, block, i) for i, n in enumerate(SIZES)]
    st = ILState(p0, bits, block, code_offset)
    plan = st.plan(bits, block, [wd] * len(SIZES), tile=tile, grid=grid)
    sc = DevScalars(lr)
    lr32 = float(np.float32(lr))
    op = [x.astype(np.float64) for x in p0]
    oqm = [np.zeros(n, np.uint8) for n in SIZES]
    oqv = [np.zeros(n, np.uint8) for n in SIZES]
    oam = [np.zeros((n + block - 1) // block, np.float32) for n in SIZES]
    oav = [np.zeros((n + block - 1) // block, np.float32) for n in SIZES]
    for t in range(1, 9):
        gs = [host_normal(n, 1e-3, 941, bits, block, i, t) for i, n in enumerate(SIZES)]
        for dst, g in zip(st.g, gs):
            dst.copy_(torch.from_numpy(g).to(DEV))
        osa.optim_step_8bit_blockwise(plan.handle, osa.optim_adamw_hp(0.9, 0.999, 1e-8), bits, block, sc.lr,
                                      None, None, sc.step)
        for i, n in enumerate(SIZES):
            orc.blockwise_step(op[i], gs[i], oqm[i], oqv[i], oam[i], oav[i], bits, block, lr32, 0.9, 0.999,
                               1e-8, wd, t)
            got = st.q[i].cpu().numpy()
            want = interleave(oqm[i], oqv[i], bits)
            assert np.array_equal(got, want), (t, i, np.flatnonzero(got != want)[:10])
            ga = st.a[i].cpu().numpy().view(np.uint32)
            wa = np.stack([oam[i], oav[i]], axis=1).ravel().view(np.uint32)
            assert np.array_equal(ga, wa), (t, i, np.flatnonzero(ga != wa)[:10])
            err = relerr_tau(st.p[i].cpu().numpy(), op[i], lr32)
            assert err <= (TOL_STEP1 if t == 1 else TOL_RUN), (t, i, err)
    assert int(sc.step.item()) == 8
    say(f"interleaved bits={bits} block={block} tile={tile} code_offset={code_offset}: codes and absmax "
        "bit-exact over 8 steps")


@pytest.mark.parametrize("bits,block", [(8, 256), (4, 128)])
def test_interleaved_matches_separate_layout(bits, block):
    """Same inputs, bf16 grads with a power-of-two loss scale, a skipped
    step: the interleaved plan's params equal the separate plan's bit for
    bit, and its states are the separate ones rearranged."""
    sizes = SIZES
    wd = [0.1 * (i % 2) for i in range(len(sizes))]
    p0 = [host_normal(n, 0.02, 942, bits, i) for i, n in enumerate(sizes)]
    il = ILState(p0, bits, block)
    sp = [torch.from_numpy(x).to(DEV) for x in p0]
    sg = [torch.zeros(n, dtype=torch.int16, device=DEV) for n in sizes]
    nb = [(n * bits + 7) // 8 for n in sizes]
    nk = [(n + block - 1) // block for n in sizes]
    sqm = [torch.zeros(k, dtype=torch.uint8, device=DEV) for k in nb]
    sqv = [torch.zeros(k, dtype=torch.uint8, device=DEV) for k in nb]
    sam = [torch.zeros(k, dtype=torch.float32, device=DEV) for k in nk]
    sav = [torch.zeros(k, dtype=torch.float32, device=DEV) for k in nk]
    il.g = [torch.zeros(n, dtype=torch.int16, device=DEV) for n in sizes]
    pl_il = il.plan(bits, block, wd, grad_bf16=True)
    pl_sep = osa.Plan(osa.TensorList(sp, sg, qm=sqm, qv=sqv, absmax_m=sam, absmax_v=sav, weight_decay=wd,
                                     grad_dtype=osa.OPTIM_BF16), osa.OPTIM_ALGO_BLOCKWISE, bits=bits, block=block)
    scale = 65536.0
    s1, s2 = DevScalars(1e-3, inv_scale=1.0 / scale), DevScalars(1e-3, inv_scale=1.0 / scale)
    hp = osa.optim_adamw_hp(0.9, 0.95, 1e-8)
    for t in range(1, 7):
        for i, n in enumerate(sizes):
            g = torch.from_numpy(host_normal(n, 1e-3, 943, bits, i, t)).to(DEV) * scale
            if t == 4 and i == 2:
                g[17] = float("inf")
            gb = g.to(torch.bfloat16).view(torch.int16)
            il.g[i].copy_(gb)
            sg[i].copy_(gb)
        for sc, pl in ((s1, pl_il), (s2, pl_sep)):
            sc.found_inf.zero_()
            osa.optim_check_finite(pl.handle, sc.found_inf)
            osa.optim_step_8bit_blockwise(pl.handle, hp, bits, block, sc.lr, sc.inv_scale, sc.found_inf, sc.step)
    assert int(s1.step.item()) == int(s2.step.item()) == 5
    assert all_equal(il.p, sp)
    for i, n in enumerate(sizes):
        qm, qv = sqm[i].cpu().numpy(), sqv[i].cpu().numpy()
        if bits == 4:
            qm = np.stack([qm & 0xF, qm >> 4], axis=1).ravel()[:n]
            qv = np.stack([qv & 0xF, qv >> 4], axis=1).ravel()[:n]
        assert np.array_equal(il.q[i].cpu().numpy(), interleave(qm, qv, bits)), i
        wa = np.stack([sam[i].cpu().numpy(), sav[i].cpu().numpy()], axis=1).ravel().view(np.uint32)
        assert np.array_equal(il.a[i].cpu().numpy().view(np.uint32), wa), i
