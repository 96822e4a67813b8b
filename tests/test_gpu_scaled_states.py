"""GPU parity of AdamW with 16-bit moments and a per-tensor scale
(Transformer Engine page, review thread on scaled low-precision optimizer
states).  The stored moments and scales depend only on the gradients and
the previous stored moments, so both sides follow the same fp32 recipe and
every 16-bit pattern and every scale is compared bit for bit at every step;
the parameters are held to the step bounds of the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle as orc
import optimizer_step_adamw_amd as osa
from gpu_support import DEV, TOL_RUN, TOL_STEP1, AdamState, DevScalars, relerr_tau, say, to_np_u16
from synth import host_normal

pytestmark = pytest.mark.gpu

RAGGED = [1, 7, 8, 9, 4095, 4096, 4097, 10007, 65539]
# gradient scale per tensor: 0 (all-zero moments, scale stays 1), values
# whose v would overflow fp16 unscaled, and values whose m would be fp16
# subnormals unscaled
G_STD = [1e-2, 0.0, 1e4, 1e-6, 1e-3, 1e-2, 3e1, 1e-5, 1e-2]


class ScaledState:
    def __init__(self, sizes, p0, half, param_bf16, grad_bf16):
        self.st = AdamState([torch.from_numpy(x).to(DEV) for x in p0], grad_bf16=grad_bf16,
                            param_bf16=param_bf16)
        self.st.m = [torch.zeros(n, dtype=torch.int16, device=DEV) for n in sizes]
        self.st.v = [torch.zeros(n, dtype=torch.int16, device=DEV) for n in sizes]
        self.sm = [torch.ones(1, device=DEV) for _ in sizes]
        self.sv = [torch.ones(1, device=DEV) for _ in sizes]
        self.half = half

    def tensor_list(self, wd):
        return osa.TensorList(self.st.p, self.st.g, m=self.st.m, v=self.st.v, remainders=self.st.r,
                              weight_decay=wd, scale_m=self.sm, scale_v=self.sv,
                              param_dtype=osa.OPTIM_BF16 if self.st.param_bf16 else osa.OPTIM_F32,
                              grad_dtype=osa.OPTIM_BF16 if self.st.grad_bf16 else osa.OPTIM_F32)

    def plan(self, wd, grid=0):
        return osa.Plan(self.tensor_list(wd), osa.OPTIM_ALGO_ADAMW, grid=grid,
                        state_dtype=osa.OPTIM_F16 if self.half else osa.OPTIM_BF16)


class OracleState:
    def __init__(self, sizes, p0):
        self.p = [x.astype(np.float64) for x in p0]
        self.qm = [np.zeros(n, np.uint16) for n in sizes]
        self.qv = [np.zeros(n, np.uint16) for n in sizes]
        self.sm = [np.ones(1, np.float32) for _ in sizes]
        self.sv = [np.ones(1, np.float32) for _ in sizes]


def _set_grads(S, sizes, key, t, inv):
    """Writes stored grads G (bf16 or fp32) and returns the fp32 gradient the
    step sees, G * inv (inv a power of two, so the product is exact)."""
    out = []
    for i, n in enumerate(sizes):
        std = G_STD[i % len(G_STD)]
        gh = torch.from_numpy(host_normal(n, max(std, 1e-30), 950, key, i, t)).to(DEV) * (std > 0) / inv
        if S.st.grad_bf16:
            S.st.g[i].copy_(gh.to(torch.bfloat16).view(torch.int16))
            G = orc.bf16_bits_to_f64(to_np_u16(S.st.g[i]))
        else:
            S.st.g[i].copy_(gh)
            G = S.st.g[i].cpu().numpy().astype(np.float64)
        out.append((G * inv).astype(np.float32))
    return out


def _compare(S, O, sizes, lr32, t_applied, tag):
    for i in range(len(sizes)):
        qm, qv = to_np_u16(S.st.m[i]), to_np_u16(S.st.v[i])
        assert np.array_equal(qm, O.qm[i]), (tag, i, np.flatnonzero(qm != O.qm[i])[:5])
        assert np.array_equal(qv, O.qv[i]), (tag, i, np.flatnonzero(qv != O.qv[i])[:5])
        assert S.sm[i].cpu().numpy().view(np.uint32)[0] == O.sm[i].view(np.uint32)[0], (tag, i)
        assert S.sv[i].cpu().numpy().view(np.uint32)[0] == O.sv[i].view(np.uint32)[0], (tag, i)
        err = relerr_tau(S.st.master(i).cpu().numpy(), O.p[i], lr32)
        assert err <= (TOL_STEP1 if t_applied == 1 else TOL_RUN), (tag, i, err)


@pytest.mark.parametrize("half,param_bf16,grad_bf16,grid,inv", [
    (True, False, False, 0, 1.0), (False, False, True, 0, 1.0), (True, True, True, 0, 2.0 ** -10),
    (True, False, True, 5, 1.0), (False, True, False, 0, 2.0 ** -4)])
def test_scaled_states_match_oracle(half, param_bf16, grad_bf16, grid, inv):
    sizes = RAGGED
    lr = 1e-3
    wd = [0.1 * (i % 2) for i in range(len(sizes))]
    p0 = [host_normal(n, 0.02, 951, int(half), i, 0) for i, n in enumerate(sizes)]
    S = ScaledState(sizes, p0, half, param_bf16, grad_bf16)
    plan = S.plan(wd, grid)
    sc = DevScalars(lr, None if inv == 1.0 else inv)
    O = OracleState(sizes, p0)
    lr32 = float(np.float32(lr))
    hp = osa.optim_adamw_hp(0.9, 0.999, 1e-8)
    t_or = 0
    for k in range(1, 10):
        g = _set_grads(S, sizes, int(half) * 10 + grid, k, inv)
        skip = k == 4
        sc.found_inf.fill_(1.0 if skip else 0.0)
        before = [(x.clone(), y.clone(), a.clone(), b.clone()) for x, y, a, b in zip(S.st.m, S.st.v, S.sm, S.sv)]
        osa.optim_step_adamw(plan.handle, hp, sc.lr, sc.inv_scale, sc.found_inf, sc.step)
        if skip:  # nothing moves, the scales and the step counter included
            for (x, y, a, b), m, v, sm, sv in zip(before, S.st.m, S.st.v, S.sm, S.sv):
                assert torch.equal(x, m) and torch.equal(y, v) and torch.equal(a, sm) and torch.equal(b, sv)
            assert sc.step.item() == t_or
            continue
        t_or += 1
        for i in range(len(sizes)):
            orc.adamw_scaled_step(O.p[i], O.qm[i], O.qv[i], O.sm[i], O.sv[i], g[i], half, lr32, 0.9, 0.999,
                                  1e-8, wd[i], t_or)
        assert sc.step.item() == t_or
        _compare(S, O, sizes, lr32, t_or, k)
    if half:  # the scales follow the moments' range; all-zero moments keep scale 1
        assert S.sm[1].item() == 1.0 and S.sv[1].item() == 1.0
        assert S.sv[2].item() > 1.0 and S.sm[3].item() < 1e-6
        assert np.any(np.float32(np.abs(O.qv[2].view(np.float16))) > 60000.0)
    else:
        assert all(x.item() == 1.0 for x in S.sm + S.sv)
    say(f"half={half} param_bf16={param_bf16} grad_bf16={grad_bf16} grid={grid}: "
        f"{t_or} steps, states and scales bit-exact")


@pytest.mark.parametrize("half", [True, False])
def test_scaled_states_full_size(half):
    """One 4096 x 4096 tensor and a ragged one (the benchmarked shapes), three
    steps, every stored moment compared."""
    sizes = [4096 * 4096, 4096 * 11008 // 16 + 5]
    lr = 1e-3
    p0 = [host_normal(n, 0.02, 952, int(half), i, 0) for i, n in enumerate(sizes)]
    S = ScaledState(sizes, p0, half, param_bf16=True, grad_bf16=True)
    plan = S.plan([0.1, 0.0])
    sc = DevScalars(lr)
    O = OracleState(sizes, p0)
    lr32 = float(np.float32(lr))
    hp = osa.optim_adamw_hp(0.9, 0.95, 1e-8)
    for t in range(1, 4):
        g = _set_grads(S, sizes, 7, t, 1.0)
        osa.optim_step_adamw(plan.handle, hp, sc.lr, None, None, sc.step)
        for i in range(len(sizes)):
            orc.adamw_scaled_step(O.p[i], O.qm[i], O.qv[i], O.sm[i], O.sv[i], g[i], half, lr32, 0.9, 0.95, 1e-8,
                                  [0.1, 0.0][i], t)
        _compare(S, O, sizes, lr32, t, t)
    say(f"half={half}: {sum(sizes)} elements, 3 steps bit-exact states")


def test_scaled_states_empty_and_graph():
    """An empty tensor in the list, and the step replayed from a HIP graph
    with eager work between replays."""
    sizes = [0, 4097, 3]
    p0 = [host_normal(n, 0.02, 953, 0, i, 0) for i, n in enumerate(sizes)]
    S = ScaledState(sizes, p0, True, False, False)
    plan = S.plan([0.0, 0.1, 0.1])
    sc = DevScalars(1e-3)
    hp = osa.optim_adamw_hp(0.9, 0.999, 1e-8)
    O = OracleState(sizes, p0)
    g = _set_grads(S, sizes, 3, 1, 1.0)
    torch.cuda.synchronize()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(graph, stream=cs):
            osa.optim_step_adamw(plan.handle, hp, sc.lr, None, None, sc.step)
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    assert sc.step.item() == 0  # captured, not run
    lr32 = float(np.float32(1e-3))
    for t in range(1, 5):
        graph.replay()
        torch.cuda.synchronize()
        for i in range(len(sizes)):
            orc.adamw_scaled_step(O.p[i], O.qm[i], O.qv[i], O.sm[i], O.sv[i], g[i], True, lr32, 0.9, 0.999, 1e-8,
                                  [0.0, 0.1, 0.1][i], t)
        assert sc.step.item() == t
        _compare(S, O, sizes, lr32, t, t)
        _ = torch.ones(1000, device=DEV).sum().item()  # eager work between replays
