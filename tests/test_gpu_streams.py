"""Distinct plans are independent: steps of four plans (AdamW, Adam-mini,
LAMB, blockwise 8-bit; each with its own workspace and arrival counters)
launched on four streams at once, from four host threads, leave every
buffer bit for bit where the same steps run one plan after another leave
them."""
import threading

import pytest
import torch

import optimizer_step_adamw_amd as osa
from gpu_support import DEV, AdamState, DevScalars, QuantState, all_equal, say
from synth import host_normal

pytestmark = pytest.mark.gpu

SIZES = [300000, 4097, 65536 + 33]
MINI = [("tok_embeddings.weight", 32 * 64), ("layers.0.attention.wq.weight", 64 * 64),
        ("layers.0.feed_forward.w1.weight", 172 * 64), ("norm.weight", 64)]
STEPS = 6


def _p0(sizes, key):
    return [torch.from_numpy(host_normal(n, 0.02, 970, key, i, 0)).to(DEV) for i, n in enumerate(sizes)]


def _make(kind):
    hp = osa.optim_adamw_hp(0.9, 0.999, 1e-8)
    if kind == "adamw":
        st = AdamState(_p0(SIZES, 1))
        plan = osa.Plan(st.tensor_list([0.1] * len(SIZES)), osa.OPTIM_ALGO_ADAMW)
        run = lambda sc, s: osa.optim_step_adamw(plan.handle, hp, sc.lr, None, None, sc.step, stream=s)
        bufs = lambda: st.buffers()
    elif kind == "mini":
        names, sizes = [n for n, _ in MINI], [s for _, s in MINI]
        kinds, hn, wds = osa.adam_mini_partition(names, sizes, dim=64, n_heads=4, weight_decay=0.1)
        vlen = [s if k == osa.OPTIM_MINI_FULL_V else s // h for k, s, h in zip(kinds, sizes, hn)]
        st = AdamState(_p0(sizes, 2), v_len=vlen)
        plan = osa.Plan(st.tensor_list(wds, mini_kind=kinds, head_numel=hn), osa.OPTIM_ALGO_ADAM_MINI)
        run = lambda sc, s: osa.optim_step_adam_mini(plan.handle, hp, sc.lr, None, None, sc.step, stream=s)
        bufs = lambda: st.buffers()
    elif kind == "lamb":
        st = AdamState(_p0(SIZES, 3))
        plan = osa.Plan(st.tensor_list([0.1] * len(SIZES)), osa.OPTIM_ALGO_LAMB)
        h6 = osa.optim_adamw_hp(0.9, 0.999, 1e-6)
        run = lambda sc, s: osa.optim_step_lamb(plan.handle, h6, sc.lr, None, None, sc.step, stream=s)
        bufs = lambda: st.buffers()
    else:
        st = QuantState(_p0(SIZES, 4), 8, 256)
        plan = osa.Plan(st.tensor_list([0.01] * len(SIZES)), osa.OPTIM_ALGO_BLOCKWISE, bits=8, block=256)
        run = lambda sc, s: osa.optim_step_8bit_blockwise(plan.handle, hp, 8, 256, sc.lr, None, None, sc.step,
                                                          stream=s)
        bufs = lambda: st.buffers()
    return dict(st=st, plan=plan, run=run, bufs=bufs, sc=DevScalars(1e-3))


def _grads(st, key, t):
    for i, dst in enumerate(st.g):
        dst.copy_(torch.from_numpy(host_normal(dst.numel(), 1e-3, 971, key, i, t)).to(DEV))


def test_plans_on_concurrent_streams_match_sequential():
    kinds = ["adamw", "mini", "lamb", "blockwise8"]
    seq = [_make(k) for k in kinds]
    par = [_make(k) for k in kinds]
    # sequential reference: one plan after another on the current stream
    for t in range(1, STEPS + 1):
        for j, x in enumerate(seq):
            _grads(x["st"], j, t)
            x["run"](x["sc"], None)
    torch.cuda.synchronize()
    # concurrent: every plan on its own stream, launched from its own thread
    streams = [torch.cuda.Stream() for _ in kinds]
    for t in range(1, STEPS + 1):
        for j, x in enumerate(par):
            _grads(x["st"], j, t)
        torch.cuda.synchronize()
        errors = []

        def worker(j):
            try:
                with torch.cuda.stream(streams[j]):
                    par[j]["run"](par[j]["sc"], streams[j])
            except Exception as e:  # surfaced below
                errors.append(e)

        threads = [threading.Thread(target=worker, args=(j,)) for j in range(len(kinds))]
        for th in threads:
            th.start()
        for th in threads:
            th.join()
        assert not errors, errors
        torch.cuda.synchronize()
    for k, a, b in zip(kinds, seq, par):
        assert all_equal(a["bufs"](), b["bufs"]()), k
        assert torch.equal(a["sc"].step, b["sc"].step) and int(b["sc"].step.item()) == STEPS, k
    say(f"{len(kinds)} plans on concurrent streams and threads: bit-identical to sequential, {STEPS} steps")
