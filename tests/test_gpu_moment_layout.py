"""GPU parity of the interleaved moment layout of the AdamW / AdEMAMix steps
(plan option state_layout = OPTIM_LAYOUT_INTERLEAVED: a tensor's m, v and
AdEMAMix's m2 share one array in blocks of 1024 elements).  The layout moves
the same values as separate arrays, so each case runs both layouts on the
same inputs and checks, after every step, that params and moments agree bit
for bit, and that the interleaved run's params stay within the step bounds
of the CPU oracle.  Lists span packs of small tensors, ragged tails, an
unaligned tensor, the early-load and late kernel forms, a persistent grid,
bf16 params with remainders, bf16 grads and fp32 masters."""
import numpy as np
import pytest
import torch

import oracle as orc
import optimizer_step_adamw_amd as osa
from gpu_support import DEV, TOL_RUN, TOL_STEP1, DevScalars, relerr_tau, say, to_np_u16
from synth import host_normal

pytestmark = pytest.mark.gpu

BLK = 1024
# packs (<= 1024 elements), whole and ragged 1024-blocks, several units
RAGGED = [1, 3, 100, 256, 1000, 1023, 1024, 1025, 4095, 4097, 10007, 65539]
MID = [1 << 20, 4096 * 100 + 37, 3000]  # > 2^20 elements: the early-load form on 4096-element units


def rup(n):
    return (n + BLK - 1) // BLK * BLK


def moments_of(buf, n, K):
    """The K moment arrays of one tensor, read out of its interleaved buffer
    (copies: a moment's blocks are not contiguous)."""
    blocks = buf.view(-1, K, BLK)
    return [blocks[:, k, :].reshape(-1)[:n] for k in range(K)]


class Run:
    """Device state of one layout: param (fp32, bf16 + remainder, or model
    copy + fp32 master) and moments, sharing the gradient buffers."""

    def __init__(self, p0, g, K, il, pkind, unaligned):
        self.il, self.K, self.pkind = il, K, pkind
        sizes = [x.size for x in p0]
        dev = [torch.from_numpy(x).to(DEV) for x in p0]
        for i in unaligned:  # 4 bytes past a 16-byte boundary
            buf = torch.empty(sizes[i] + 1, dtype=torch.float32, device=DEV)
            buf[1:].copy_(dev[i])
            dev[i] = buf[1:]
        self.r = self.master = None
        if pkind == "f32":
            self.p = dev
        elif pkind == "bf16r":
            self.p = [torch.empty(n, dtype=torch.int16, device=DEV) for n in sizes]
            self.r = [torch.empty(n, dtype=torch.int16, device=DEV) for n in sizes]
            for x, b, r in zip(dev, self.p, self.r):
                osa.optim_remainder_split(x, b, r, x.numel())
        else:  # bf16 model copy of an fp32 master
            self.master = dev
            self.p = [torch.zeros(n, dtype=torch.int16, device=DEV) for n in sizes]
        if il:
            self.buf = []
            for i, n in enumerate(sizes):
                b = torch.zeros(K * rup(n) + (1 if i in unaligned else 0), device=DEV)
                self.buf.append(b[1:] if i in unaligned else b)
            self.sizes = sizes
        else:
            self.mom = []
            for i, n in enumerate(sizes):
                ms = []
                for _ in range(K):
                    b = torch.zeros(n + (1 if i in unaligned else 0), device=DEV)
                    ms.append(b[1:] if i in unaligned else b)
                self.mom.append(ms)
        self.g = g

    def moments(self, i):
        return moments_of(self.buf[i], self.sizes[i], self.K) if self.il else self.mom[i]

    def plan(self, algo, wd, grad_bf16, tile, grid):
        kw = dict(m=self.buf) if self.il else dict(m=[x[0] for x in self.mom], v=[x[1] for x in self.mom])
        if self.K == 3 and not self.il:
            kw["m2"] = [x[2] for x in self.mom]
        pdt = osa.OPTIM_F32 if self.pkind == "f32" else osa.OPTIM_BF16
        tl = osa.TensorList(self.p, self.g, remainders=self.r, master=self.master, weight_decay=wd,
                            param_dtype=pdt, grad_dtype=osa.OPTIM_BF16 if grad_bf16 else osa.OPTIM_F32, **kw)
        return osa.Plan(tl, algo, tile=tile, grid=grid,
                        state_layout=osa.OPTIM_LAYOUT_INTERLEAVED if self.il else osa.OPTIM_LAYOUT_SEPARATE)

    def master_f32(self, i):
        if self.pkind == "f32":
            return self.p[i]
        if self.pkind == "master":
            return self.master[i]
        out = torch.empty(self.p[i].numel(), dtype=torch.float32, device=DEV)
        osa.optim_remainder_reconstruct(self.p[i], self.r[i], out, out.numel())
        return out


def _run(algo, sizes, steps, *, pkind="f32", grad_bf16=False, tile=0, grid=0, unaligned=(), lr=1e-3, key=0,
         oracle=True):
    K = 3 if algo == osa.OPTIM_ALGO_ADEMAMIX else 2
    wd = [0.1 * (i % 2) for i in range(len(sizes))]
    p0 = [host_normal(n, 0.02, 960, key, i, 0) for i, n in enumerate(sizes)]
    g = [torch.zeros(n, dtype=torch.int16 if grad_bf16 else torch.float32, device=DEV) for n in sizes]
    runs = [Run(p0, g, K, il, pkind, unaligned) for il in (False, True)]
    plans = [r.plan(algo, wd, grad_bf16, tile, grid) for r in runs]
    scs = [DevScalars(lr) for _ in runs]
    lr32 = float(np.float32(lr))
    op = [x.astype(np.float64) for x in p0]
    om, ov, om2 = ([np.zeros(n) for n in sizes] for _ in range(3))
    b1, b2, b3, alpha, eps = 0.9, 0.95, 0.999, 5.0, 1e-8
    worst = 0.0
    for t in range(1, steps + 1):
        gs = []
        for i, n in enumerate(sizes):
            gh = torch.from_numpy(host_normal(n, 1e-2, 961, key, i, t)).to(DEV)
            if grad_bf16:
                g[i].copy_(gh.to(torch.bfloat16).view(torch.int16))
                gs.append(orc.bf16_bits_to_f64(to_np_u16(g[i])))
            else:
                g[i].copy_(gh)
                gs.append(gh.cpu().numpy().astype(np.float64))
        for plan, sc in zip(plans, scs):
            if K == 2:
                osa.optim_step_adamw(plan.handle, osa.optim_adamw_hp(b1, b2, eps), sc.lr, None, None, sc.step)
            else:
                osa.optim_step_ademamix(plan.handle, osa.optim_ademamix_hp(b1, b2, b3, alpha, eps), sc.lr, None,
                                        None, sc.step)
        sep, il = runs
        for i in range(len(sizes)):
            assert torch.equal(sep.p[i], il.p[i]), (t, i, "param")
            if sep.r is not None:
                assert torch.equal(sep.r[i], il.r[i]), (t, i, "remainder")
            if sep.master is not None:
                assert torch.equal(sep.master[i], il.master[i]), (t, i, "master")
            sm, im = sep.moments(i), il.moments(i)
            for k in range(K):
                assert torch.equal(sm[k], im[k]), (t, i, "moment", k)
        if oracle:
            for i in range(len(sizes)):
                if K == 2:
                    orc.adamw_step(op[i], om[i], ov[i], gs[i], lr32, b1, b2, eps, wd[i], t)
                else:
                    orc.ademamix_step(op[i], om[i], om2[i], ov[i], gs[i], lr32, b1, b2, b3, alpha, eps, wd[i], t)
            err = max(relerr_tau(il.master_f32(i).cpu().numpy(), op[i], lr32) for i in range(len(sizes)))
            worst = max(worst, err)
            assert err <= (TOL_STEP1 if t == 1 else TOL_RUN), (t, err)
    for sc in scs:
        assert int(sc.step.item()) == steps
    # the last block's slots past the tensor's end are never written
    for i, n in enumerate(sizes):
        tail = runs[1].buf[i].view(-1, K, BLK)[-1, :, n - (rup(n) - BLK):]
        assert torch.count_nonzero(tail).item() == 0, (i, "padding written")
    say(f"algo={algo} pkind={pkind} grad_bf16={grad_bf16} tile={tile} grid={grid} sizes={len(sizes)}: "
        f"layouts bit-identical over {steps} steps, worst relerr_tau {worst:.3e}")


@pytest.mark.parametrize("algo,pkind,grad_bf16", [
    (osa.OPTIM_ALGO_ADAMW, "f32", False), (osa.OPTIM_ALGO_ADAMW, "bf16r", True),
    (osa.OPTIM_ALGO_ADAMW, "master", True), (osa.OPTIM_ALGO_ADEMAMIX, "f32", False),
    (osa.OPTIM_ALGO_ADEMAMIX, "bf16r", False)])
def test_interleaved_moments_ragged_list(algo, pkind, grad_bf16):
    _run(algo, RAGGED, 6, pkind=pkind, grad_bf16=grad_bf16, unaligned=(7,) if pkind == "f32" else (), key=1)


@pytest.mark.parametrize("tile,grid", [(1024, 0), (8192, 0), (2048, 7), (4096, 0)])
@pytest.mark.parametrize("algo,pkind", [(osa.OPTIM_ALGO_ADAMW, "bf16r"), (osa.OPTIM_ALGO_ADEMAMIX, "f32")])
def test_interleaved_moments_launch_shapes(algo, pkind, tile, grid):
    _run(algo, RAGGED, 3, pkind=pkind, grad_bf16=pkind == "bf16r", tile=tile, grid=grid, key=2)


@pytest.mark.parametrize("algo,pkind", [(osa.OPTIM_ALGO_ADAMW, "f32"), (osa.OPTIM_ALGO_ADAMW, "bf16r"),
                                        (osa.OPTIM_ALGO_ADEMAMIX, "f32")])
def test_interleaved_moments_early_form(algo, pkind):
    _run(algo, MID, 3, pkind=pkind, grad_bf16=pkind == "bf16r", key=3)


@pytest.mark.parametrize("pkind", ["f32", "bf16r"])
def test_interleaved_moments_late_form(pkind):
    """More than 2^24 elements: 2048-element units without early loads."""
    _run(osa.OPTIM_ALGO_ADAMW, [(1 << 24) + 3 * 1024 + 17, 5000, 300], 2, pkind=pkind,
         grad_bf16=pkind == "bf16r", key=4, oracle=False)
