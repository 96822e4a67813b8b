"""Every multi-kernel step (and the bf16 + remainder AdamW step with
interleaved moments), and the AMP loop around the step, captured once
in a HIP graph and replayed: each replay, with eager work and host
synchronisation between replays, must leave every buffer and device scalar
bit for bit where the same step run eagerly on a twin state leaves them.
Steps that publish through arrival counters, per-unit partial sums or
per-tensor maxima (Adam-mini, LAMB, blockwise, fp16 scaled moments) rely on
the kernels rearming their own counters, since a graph records no
memset."""
import pytest
import torch

import optimizer_step_adamw_amd as osa
from gpu_support import DEV, AdamState, DevScalars, QuantState, all_equal, say
from synth import host_normal

pytestmark = pytest.mark.gpu

SIZES = [5000, 4097, 33, 65536 + 17]
MINI = [("tok_embeddings.weight", 32 * 64), ("layers.0.attention.wq.weight", 64 * 64),
        ("layers.0.attention.wk.weight", 64 * 64), ("layers.0.feed_forward.w1.weight", 172 * 64),
        ("norm.weight", 64)]


def _p0(sizes, key):
    return [torch.from_numpy(host_normal(n, 0.02, 960, key, i, 0)).to(DEV) for i, n in enumerate(sizes)]


def _grads(sizes, key, t):
    return [torch.from_numpy(host_normal(n, 1e-3, 961, key, i, t)).to(DEV) for i, n in enumerate(sizes)]


def _capture(fn):
    torch.cuda.synchronize()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            fn()
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    return g


def _adam_like(algo, key):
    """Twin states (eager, graph) and their plans and step callables."""
    sizes = SIZES
    tw = []
    for _ in range(2):
        if algo in ("mini", "mini_segments"):
            names = [n for n, _ in MINI]
            msz = [s for _, s in MINI]
            kinds, hn, wds = osa.adam_mini_partition(names, msz, dim=64, n_heads=4, weight_decay=0.1)
            vlen = [s if k == osa.OPTIM_MINI_FULL_V else s // h for k, s, h in zip(kinds, msz, hn)]
            st = AdamState(_p0(msz, key), v_len=vlen)
            # mini_segments: every tensor its own segment (three launches each)
            plan = osa.Plan(st.tensor_list(wds, mini_kind=kinds, head_numel=hn), osa.OPTIM_ALGO_ADAM_MINI,
                            segment_bytes=1 if algo == "mini_segments" else 0)
            sizes = msz
        elif algo == "blockwise8_interleaved":
            st = QuantState(_p0(sizes, key), 8, 256)
            st.qm = [torch.zeros(2 * n, dtype=torch.uint8, device=DEV) for n in sizes]
            st.am = [torch.zeros(2 * ((n + 255) // 256), dtype=torch.float32, device=DEV) for n in sizes]
            st.qv = st.av = None
            tl = osa.TensorList(st.p, st.g, qm=st.qm, absmax_m=st.am, weight_decay=[0.01] * len(sizes))
            plan = osa.Plan(tl, osa.OPTIM_ALGO_BLOCKWISE, bits=8, block=256,
                            state_layout=osa.OPTIM_LAYOUT_INTERLEAVED)
        elif algo in ("blockwise8", "blockwise4", "blockwise_ademamix8"):
            bits = 4 if algo == "blockwise4" else 8
            block = 128 if bits == 4 else 256
            ade = algo.startswith("blockwise_ademamix")
            st = QuantState(_p0(sizes, key), bits, block, ademamix=ade)
            plan = osa.Plan(st.tensor_list([0.01] * len(sizes)),
                            osa.OPTIM_ALGO_BLOCKWISE_ADEMAMIX if ade else osa.OPTIM_ALGO_BLOCKWISE,
                            bits=bits, block=block)
        elif algo == "adamw_bf16r_interleaved":
            st = AdamState(_p0(sizes, key), param_bf16=True, moments_interleaved=True)
            plan = osa.Plan(st.tensor_list([0.1] * len(sizes)), osa.OPTIM_ALGO_ADAMW,
                            state_layout=osa.OPTIM_LAYOUT_INTERLEAVED)
        elif algo == "states16":
            st = AdamState(_p0(sizes, key))
            st.m = [torch.zeros(n, dtype=torch.int16, device=DEV) for n in sizes]
            st.v = [torch.zeros(n, dtype=torch.int16, device=DEV) for n in sizes]
            st.sm = [torch.ones(1, device=DEV) for _ in sizes]
            st.sv = [torch.ones(1, device=DEV) for _ in sizes]
            tl = osa.TensorList(st.p, st.g, m=st.m, v=st.v, weight_decay=[0.1] * len(sizes), scale_m=st.sm,
                                scale_v=st.sv)
            plan = osa.Plan(tl, osa.OPTIM_ALGO_ADAMW, state_dtype=osa.OPTIM_F16)
        else:
            st = AdamState(_p0(sizes, key), ademamix=algo == "ademamix")
            if algo == "lion":
                st.v = None
            code = dict(ademamix=osa.OPTIM_ALGO_ADEMAMIX, lion=osa.OPTIM_ALGO_LION,
                        lamb=osa.OPTIM_ALGO_LAMB)[algo]
            tl = osa.TensorList(st.p, st.g, m=st.m, v=st.v, m2=st.m2, weight_decay=[0.1] * len(sizes))
            plan = osa.Plan(tl, code)
        tw.append((st, plan, DevScalars(1e-3)))

    def step(st, plan, sc):
        hp = osa.optim_adamw_hp(0.9, 0.999, 1e-8)
        hpe = osa.optim_ademamix_hp(0.9, 0.999, 0.9999, 5.0, 1e-8)
        if algo in ("mini", "mini_segments"):
            osa.optim_step_adam_mini(plan.handle, hp, sc.lr, None, None, sc.step)
        elif algo in ("blockwise8", "blockwise8_interleaved"):
            osa.optim_step_8bit_blockwise(plan.handle, hp, 8, 256, sc.lr, None, None, sc.step)
        elif algo == "blockwise4":
            osa.optim_step_8bit_blockwise(plan.handle, hp, 4, 128, sc.lr, None, None, sc.step)
        elif algo == "blockwise_ademamix8":
            osa.optim_step_8bit_blockwise_ademamix(plan.handle, hpe, 8, 256, sc.lr, None, None, sc.step)
        elif algo in ("states16", "adamw_bf16r_interleaved"):
            osa.optim_step_adamw(plan.handle, hp, sc.lr, None, None, sc.step)
        elif algo == "ademamix":
            osa.optim_step_ademamix(plan.handle, hpe, sc.lr, None, None, sc.step)
        elif algo == "lion":
            osa.optim_step_lion(plan.handle, osa.optim_lion_hp(0.9, 0.99), sc.lr, None, None, sc.step)
        else:
            osa.optim_step_lamb(plan.handle, osa.optim_adamw_hp(0.9, 0.999, 1e-6), sc.lr, None, None, sc.step)

    return tw, sizes, step


def _buffers(st):
    out = [x for x in (getattr(st, "p", []) or [])]
    for name in ("m", "v", "m2", "r", "qm", "qv", "am", "av", "qm2", "am2", "sm", "sv"):
        out += list(getattr(st, name, None) or [])
    return out


@pytest.mark.parametrize("algo", ["ademamix", "mini", "mini_segments", "lion", "lamb", "blockwise8", "blockwise4",
                                  "blockwise_ademamix8", "blockwise8_interleaved", "states16",
                                  "adamw_bf16r_interleaved"])
def test_step_graph_replays_match_eager(algo):
    (eager, graph), sizes, step = _adam_like(algo, sum(map(ord, algo)))
    g = _capture(lambda: step(*graph))
    assert int(graph[2].step.item()) == 0  # captured, not run
    for t in range(1, 6):
        gs = _grads(sizes, 7, t)
        for st, _, _ in (eager, graph):
            for dst, x in zip(st.g, gs):
                dst.copy_(x)
        step(*eager)
        g.replay()
        torch.cuda.synchronize()
        assert all_equal(_buffers(eager[0]), _buffers(graph[0])), (algo, t)
        assert torch.equal(eager[2].step, graph[2].step) and int(graph[2].step.item()) == t, (algo, t)
        _ = torch.ones(1000, device=DEV).sum().item()  # eager work between replays
    say(f"{algo}: 5 graph replays bit-identical to the eager steps")


def test_amp_loop_graph_replays_match_eager():
    """Check + norm, clipped step, scale update in one graph; an overflow at
    replay 3 must back the scale off and skip the step, as eagerly."""
    tw = []
    for _ in range(2):
        st = AdamState(_p0(SIZES, 3), grad_bf16=True, param_bf16=True)
        plan = osa.Plan(st.tensor_list([0.1] * len(SIZES)), osa.OPTIM_ALGO_ADAMW)
        sc = DevScalars(1e-3, inv_scale=1.0 / 65536.0)
        extra = dict(scale=torch.tensor([65536.0], device=DEV), tracker=torch.zeros(1, dtype=torch.int32, device=DEV),
                     norm=torch.zeros(1, device=DEV), clip=torch.zeros(1, device=DEV))
        tw.append((st, plan, sc, extra))
    hp = osa.optim_adamw_hp(0.9, 0.95, 1e-8)

    def loop(st, plan, sc, ex):
        sc.found_inf.zero_()
        osa.optim_grad_norm(plan.handle, sc.inv_scale, 0.02, sc.found_inf, ex["norm"], ex["clip"])
        osa.optim_step_adamw(plan.handle, hp, sc.lr, ex["clip"], sc.found_inf, sc.step)
        osa.optim_scaler_update(ex["scale"], sc.inv_scale, ex["tracker"], sc.found_inf, 2.0, 0.5, 2)

    g = _capture(lambda: loop(*tw[1]))
    for t in range(1, 7):
        gs = _grads(SIZES, 4, t)
        for st, _, _, ex in tw:
            S = float(ex["scale"].item())
            for dst, x in zip(st.g, gs):
                dst.copy_((x * S).to(torch.bfloat16).view(torch.int16))
            if t == 3:
                st.g[1][100] = torch.tensor(float("inf")).to(torch.bfloat16).view(torch.int16)
        loop(*tw[0])
        g.replay()
        torch.cuda.synchronize()
        (e, _, se, xe), (r, _, sr, xr) = tw
        assert all_equal(e.buffers(), r.buffers()), t
        for a, b in ((se.step, sr.step), (se.found_inf, sr.found_inf), (se.inv_scale, sr.inv_scale),
                     (xe["scale"], xr["scale"]), (xe["tracker"], xr["tracker"]), (xe["clip"], xr["clip"]),
                     (xe["norm"], xr["norm"])):
            assert torch.equal(a, b), t
    # growth every 2 clean steps, backoff at the overflow: 65536 -> 131072 -> 65536 -> 131072
    assert int(tw[1][2].step.item()) == 5 and float(tw[1][3]["scale"].item()) == 131072.0
    say("AMP loop: 6 graph replays bit-identical to the eager loop, overflow skipped")
