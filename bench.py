"""Benchmark of the fused AdamW-family optimizer step on one MI355X.

Headline workload: one fp32 tensor of 4096 x 4096 elements stepped by AdamW
(lr 0.1, wd 0.1) and by AdEMAMix (beta3 0.9999, alpha 5) on the same
gradients, each optimizer with its own state.  One benchmark step = one
AdamW step + one AdEMAMix step through the C ABI (every kernel of the path:
per-step scalars, moments, bias correction, decay, update).  `value` is
optimizer element-updates per second with all inputs resident in HBM.

Secondary workloads (same JSON line, "secondary"): the 1M-element tensor,
the Llama-shaped 1.1B bf16+remainder AMP list with device cosine lr (also
timed as the full AMP loop with global-norm clipping folded into the step
and the dynamic loss-scale update), the 268M-element blockwise 8-bit and
4-bit states (2-state AdamW in both state layouts and 3-state AdEMAMix),
Adam-mini over the 7B list, Lion, LAMB and AdamW with an fp32 master and a
bf16 / fp16 model copy or with scaled 16-bit moments on the 4096 x 4096
tensor, and the headline's AdamW elements as lists of 4096 and 65536
tensors.  Gradients are drawn once per workload, outside the timed region.

Timing: HIP events on the stream the library launches on (torch's current
stream), one pair around every optimizer call inside the timed region; the
region itself is bracketed by device synchronisation.  Achieved bandwidth
counts algorithmic bytes (what the method must read and write once).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published peak
METRIC = "optimizer-step elements/s and achieved HBM GB/s (% of peak), fp32 and 8-bit"

# algorithmic bytes per element (read + write once)
B_ADAMW_F32 = 28.0            # R p g m v (16) + W p m v (12)
B_ADEMAMIX_F32 = 36.0         # + m2 read and write
B_LION_F32 = 20.0             # R p g m (12) + W p m (8)
B_ADAMW_MASTER = 30.0         # R master g m v (16) + W master, 16-bit copy, m, v (14)
B_ADAMW_STATES16 = 20.0       # R p g (8) + 16-bit m v (4); W p (4) + 16-bit m v (4)
T_ADAMW_STATES16 = 28.0       # fp16: two passes, the second re-reads g, m, v (8)
B_BF16R_AMP = 26.0 + 2.0      # R bf16 p, int16 r, bf16 g, m, v (14) + W (12); + finite check g
B_8BIT = 4 + 4 + 1 + 1 + 8 / 256 + 4 + 1 + 1 + 8 / 256
B_4BIT = 4 + 4 + 0.5 + 0.5 + 8 / 128 + 4 + 0.5 + 0.5 + 8 / 128
CLIP_MAX_NORM = 1.0           # global-norm clip of the Llama 1.1B AMP loop
C4_BETA3, C4_ALPHA = 0.9999, 5.0   # AdEMAMix on the blockwise list: the 4096^2 run's values


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--secondary", default="c1,c3,c4,c5,lion_lamb,master,states16,many",
                    help="comma list of secondary workloads (c1,c3,c4,c5,lion_lamb,master,states16,many) "
                         "or 'none'")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample (0 = skip)")
    return ap.parse_args()


class Timer:
    """Events around each call on the current stream; total from first to last."""

    def __init__(self, torch):
        self.torch = torch
        self.marks = []

    def mark(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.marks.append(e)

    def durations_ms(self):
        self.torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in zip(self.marks[:-1], self.marks[1:])]


def dist(xs):
    """Median and 10th / 90th percentiles (ms) of per-call event intervals."""
    a = sorted(xs)
    q = lambda f: a[min(len(a) - 1, int(round(f * (len(a) - 1))))]
    return dict(median_ms=q(0.5), p10_ms=q(0.1), p90_ms=q(0.9))


def run_timed(torch, calls, steps, warmup, stats=None):
    """calls: list of zero-arg functions forming one step.  The timed region
    is `steps` steps between two events, with nothing recorded between the
    calls: its mean is the step time.  A second pass of `steps` steps records
    an event after every call, for each call's mean and (into `stats`, if a
    list) its median / p10 / p90; an event between two kernels adds a few
    microseconds to the interval, so these per-call figures sit slightly
    above the kernels' own durations.  Returns (ms per step, per-call mean
    ms from the second pass, host wall ms per step of the timed region)."""
    for _ in range(warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(steps):
        for c in calls:
            c()
    b.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    ms = a.elapsed_time(b) / steps
    tm = Timer(torch)
    tm.mark()
    for _ in range(steps):
        for c in calls:
            c()
            tm.mark()
    d = tm.durations_ms()
    per_call = [sum(d[i::len(calls)]) / steps for i in range(len(calls))]
    if stats is not None:
        stats.extend(dist(d[i::len(calls)]) for i in range(len(calls)))
    return ms, per_call, wall / steps


def run_each(torch, call, steps, warmup=2):
    """Mean duration (ms) of one call run `steps` times back to back between
    two events: the kernel's launch duration as a training loop sees it, with
    no event between launches."""
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        call()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def run_timed_cold(torch, call, steps, warmup, flush_bytes=1 << 30):
    """One call per step with a 1 GiB device write between steps, outside the
    events, so the step's inputs come from HBM rather than the 256 MB
    Infinity Cache.  Returns the per-call event intervals (ms)."""
    scratch = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        call()
    out = []
    for i in range(steps):
        scratch.fill_(float(i))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        call()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b))
    del scratch
    return out


def library_sources_sha256():
    """sha256 over the library's sources and header, naming the build the
    numbers were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "optimizer_step_adamw_amd", "csrc")
    files = [os.path.join(csrc, f) for f in sorted(os.listdir(csrc))]
    files.append(os.path.join(ROOT, "include", "optim_step.h"))
    for f in files:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def environment(torch):
    """Device and software the numbers were taken on."""
    pr = torch.cuda.get_device_properties(0)
    return dict(device=pr.name, arch=getattr(pr, "gcnArchName", None), compute_units=pr.multi_processor_count,
                hbm_gib=round(pr.total_memory / 2 ** 30, 1), torch=torch.__version__,
                hip=getattr(torch.version, "hip", None), host_cpus=os.cpu_count(),
                library_sources_sha256=library_sources_sha256())


def gbs(bytes_per_step, ms):
    return bytes_per_step / (ms * 1e-3) / 1e9


# --------------------------------------------------------------------------
def adam_buffers(torch, p0_list, grad_dtype, param_bf16=False, ademamix=False, v_len=None):
    dev = "cuda"
    import optimizer_step_adamw_amd as osa
    bufs = {}
    if param_bf16:
        bufs["p"] = [torch.empty(x.numel(), dtype=torch.int16, device=dev) for x in p0_list]
        bufs["r"] = [torch.empty(x.numel(), dtype=torch.int16, device=dev) for x in p0_list]
        for x, b, r in zip(p0_list, bufs["p"], bufs["r"]):
            osa.optim_remainder_split(x, b, r, x.numel())
    else:
        bufs["p"] = [x.clone() for x in p0_list]
        bufs["r"] = None
    bufs["m"] = [torch.zeros(x.numel(), dtype=torch.float32, device=dev) for x in p0_list]
    vl = v_len or [x.numel() for x in p0_list]
    bufs["v"] = [torch.zeros(k, dtype=torch.float32, device=dev) for k in vl]
    bufs["m2"] = ([torch.zeros(x.numel(), dtype=torch.float32, device=dev) for x in p0_list]
                  if ademamix else None)
    return bufs


def scalars(torch, lr, inv_scale=None):
    dev = "cuda"
    return dict(lr=torch.tensor([lr], dtype=torch.float32, device=dev),
                step=torch.zeros(1, dtype=torch.int32, device=dev),
                found_inf=torch.zeros(1, dtype=torch.float32, device=dev),
                iter=torch.zeros(1, dtype=torch.int32, device=dev),
                inv_scale=None if inv_scale is None else
                torch.tensor([inv_scale], dtype=torch.float32, device=dev))


def bench_headline(torch, osa, synth, steps, warmup):
    wl = synth.c2_decay_stress()
    n, hp = wl.numel, wl.hp
    p0 = synth.initial_param_device(wl.tensors[0], wl.p_std, wl.index, 0, "cuda")
    g = synth.device_normal(n, wl.g_std, "cuda", wl.index, 0, 1, synth.GRAD)
    A = adam_buffers(torch, [p0], osa.OPTIM_F32)
    B = adam_buffers(torch, [p0], osa.OPTIM_F32, ademamix=True)
    del p0
    tla = osa.TensorList(A["p"], [g], m=A["m"], v=A["v"], weight_decay=[hp.wd])
    tlb = osa.TensorList(B["p"], [g], m=B["m"], v=B["v"], m2=B["m2"], weight_decay=[hp.wd])
    pa = osa.Plan(tla, osa.OPTIM_ALGO_ADAMW)
    pb = osa.Plan(tlb, osa.OPTIM_ALGO_ADEMAMIX)
    sa, sb = scalars(torch, hp.lr), scalars(torch, hp.lr)
    hpa = osa.optim_adamw_hp(hp.beta1, hp.beta2, hp.eps)
    hpb = osa.optim_ademamix_hp(hp.beta1, hp.beta2, wl.extra["beta3"], wl.extra["alpha"], hp.eps)

    def call_a():
        osa.optim_step_adamw(pa.handle, hpa, sa["lr"], None, None, sa["step"])

    def call_b():
        osa.optim_step_ademamix(pb.handle, hpb, sb["lr"], None, None, sb["step"])

    stats = []
    ms, per_call, wall = run_timed(torch, [call_a, call_b], steps, warmup, stats)
    each = [run_each(torch, call_a, steps), run_each(torch, call_b, steps)]
    ev = lambda i: dict(events_mean_ms=per_call[i], events=stats[i])
    res = dict(workload=wl.name, elements=n, ms_per_step=ms, wall_ms_per_step=wall,
               elements_per_s=2 * n / (ms * 1e-3),
               kernels={
                   "adamw_fp32": dict(ms=each[0], bytes=B_ADAMW_F32 * n,
                                      gbs=gbs(B_ADAMW_F32 * n, each[0]), **ev(0)),
                   "ademamix_fp32": dict(ms=each[1], bytes=B_ADEMAMIX_F32 * n,
                                         gbs=gbs(B_ADEMAMIX_F32 * n, each[1]), **ev(1)),
               },
               note="step time: the timed steps between two events; kernel ms: the same call run "
                    "`steps` times back to back between two events; events_*: an event after every "
                    "call (each adds a few microseconds)")
    for k in res["kernels"].values():
        k["frac"] = k["gbs"] / PEAK_HBM_GBS
    pa.close()
    pb.close()
    return res


def bench_many(torch, osa, synth, steps, warmup):
    """The headline's 16,777,216 AdamW fp32 elements as one list of many
    tensors (views of one allocation per array): 4096 tensors of 4096
    elements, and 65536 tensors of 256 (each shorter than a work unit), next
    to the single tensor -- the cost of the multi-tensor traversal."""
    n = 1 << 24
    out = {}
    for count in (1, 4096, 65536):
        size = n // count
        P = torch.randn(n, device="cuda") * 0.02
        G = torch.randn(n, device="cuda") * 1e-3
        M = torch.zeros(n, device="cuda")
        V = torch.zeros(n, device="cuda")
        views = lambda x: [x[i * size:(i + 1) * size] for i in range(count)]
        plan = osa.Plan(osa.TensorList(views(P), views(G), m=views(M), v=views(V),
                                       weight_decay=[0.1] * count), osa.OPTIM_ALGO_ADAMW)
        s = scalars(torch, 1e-3)
        h = osa.optim_adamw_hp(0.9, 0.999, 1e-8)
        ms = run_each(torch, lambda: osa.optim_step_adamw(plan.handle, h, s["lr"], None, None, s["step"]), steps)
        plan.close()
        out[f"tensors_{count}x{size}"] = dict(ms=ms, gbs=gbs(B_ADAMW_F32 * n, ms),
                                              frac=gbs(B_ADAMW_F32 * n, ms) / PEAK_HBM_GBS)
        del P, G, M, V
        torch.cuda.empty_cache()
    return dict(workload="adamw_fp32_16M_as_many_tensors", elements=n, lists=out,
                note="kernel ms: the same call run back to back on one state (a 448 MB working set "
                     "partly held by the Infinity Cache between calls)")


def bench_lion_lamb(torch, osa, synth, steps, warmup):
    """Lion and LAMB on the 4096 x 4096 tensor and gradients of the headline,
    each with its own state (beta (0.9, 0.99) for Lion; LAMB eps 1e-6)."""
    wl = synth.c2_decay_stress()
    n, hp = wl.numel, wl.hp
    p0 = synth.initial_param_device(wl.tensors[0], wl.p_std, wl.index, 0, "cuda")
    g = synth.device_normal(n, wl.g_std, "cuda", wl.index, 0, 1, synth.GRAD)
    A = adam_buffers(torch, [p0], osa.OPTIM_F32)
    B = adam_buffers(torch, [p0], osa.OPTIM_F32)
    del p0
    pl = osa.Plan(osa.TensorList(A["p"], [g], m=A["m"], weight_decay=[hp.wd]), osa.OPTIM_ALGO_LION)
    pm = osa.Plan(osa.TensorList(B["p"], [g], m=B["m"], v=B["v"], weight_decay=[hp.wd]), osa.OPTIM_ALGO_LAMB)
    sl, sm = scalars(torch, 1e-4), scalars(torch, 1e-3)
    hl = osa.optim_lion_hp(0.9, 0.99)
    hm = osa.optim_adamw_hp(hp.beta1, hp.beta2, 1e-6)
    calls = [lambda: osa.optim_step_lion(pl.handle, hl, sl["lr"], None, None, sl["step"]),
             lambda: osa.optim_step_lamb(pm.handle, hm, sm["lr"], None, None, sm["step"])]
    ms, _, _ = run_timed(torch, calls, steps, warmup)
    per_call = [run_each(torch, c, steps) for c in calls]
    pl.close()
    pm.close()
    del A, B, g
    torch.cuda.empty_cache()
    return dict(workload="lion_lamb_fp32_4096x4096", elements=n, ms_per_step=ms,
                kernels={"lion_fp32": dict(ms=per_call[0], bytes_per_element=B_LION_F32,
                                           gbs=gbs(B_LION_F32 * n, per_call[0]),
                                           frac=gbs(B_LION_F32 * n, per_call[0]) / PEAK_HBM_GBS),
                         "lamb_fp32": dict(ms=per_call[1], bytes_per_element=B_ADAMW_F32,
                                           gbs=gbs(B_ADAMW_F32 * n, per_call[1]),
                                           frac=gbs(B_ADAMW_F32 * n, per_call[1]) / PEAK_HBM_GBS,
                                           note="algorithmic 28 B/elem; the two passes move 40 B/elem "
                                                "(p, m, v read again for the per-tensor trust ratio)")})


def bench_master(torch, osa, synth, steps, warmup):
    """AdamW with an fp32 master and a bf16 or fp16 model copy on the
    4096 x 4096 tensor and gradients of the headline."""
    wl = synth.c2_decay_stress()
    n, hp = wl.numel, wl.hp
    p0 = synth.initial_param_device(wl.tensors[0], wl.p_std, wl.index, 0, "cuda")
    g = synth.device_normal(n, wl.g_std, "cuda", wl.index, 0, 1, synth.GRAD)
    out = {}
    for name, dt in (("adamw_master_bf16", osa.OPTIM_BF16), ("adamw_master_f16", osa.OPTIM_F16)):
        master = p0.clone()
        model = torch.zeros(n, dtype=torch.int16, device="cuda")
        m = torch.zeros(n, device="cuda")
        v = torch.zeros(n, device="cuda")
        plan = osa.Plan(osa.TensorList([model], [g], m=[m], v=[v], master=[master], weight_decay=[hp.wd],
                                       param_dtype=dt), osa.OPTIM_ALGO_ADAMW)
        sc = scalars(torch, hp.lr)
        h = osa.optim_adamw_hp(hp.beta1, hp.beta2, hp.eps)
        ms, _, _ = run_timed(torch, [lambda: osa.optim_step_adamw(plan.handle, h, sc["lr"], None, None,
                                                                  sc["step"])], steps, warmup)
        plan.close()
        out[name] = dict(ms=ms, bytes_per_element=B_ADAMW_MASTER, gbs=gbs(B_ADAMW_MASTER * n, ms),
                         frac=gbs(B_ADAMW_MASTER * n, ms) / PEAK_HBM_GBS)
        del master, model, m, v
    del p0, g
    torch.cuda.empty_cache()
    return dict(workload="adamw_master_copy_4096x4096", elements=n, kernels=out)


def bench_states16(torch, osa, synth, steps, warmup):
    """AdamW with fp16 or bf16 moments and per-tensor scales on the
    4096 x 4096 fp32 tensor and gradients of the headline.  frac is priced on
    the algorithmic 20 B/element; the two-pass fp16 step moves 28."""
    wl = synth.c2_decay_stress()
    n, hp = wl.numel, wl.hp
    p0 = synth.initial_param_device(wl.tensors[0], wl.p_std, wl.index, 0, "cuda")
    g = synth.device_normal(n, wl.g_std, "cuda", wl.index, 0, 1, synth.GRAD)
    out = {}
    for name, sdt in (("adamw_states_f16", osa.OPTIM_F16), ("adamw_states_bf16", osa.OPTIM_BF16)):
        p = p0.clone()
        m = torch.zeros(n, dtype=torch.int16, device="cuda")
        v = torch.zeros(n, dtype=torch.int16, device="cuda")
        sm, sv = torch.ones(1, device="cuda"), torch.ones(1, device="cuda")
        plan = osa.Plan(osa.TensorList([p], [g], m=[m], v=[v], scale_m=[sm], scale_v=[sv], weight_decay=[hp.wd]),
                        osa.OPTIM_ALGO_ADAMW, state_dtype=sdt)
        sc = scalars(torch, hp.lr)
        h = osa.optim_adamw_hp(hp.beta1, hp.beta2, hp.eps)
        ms, _, _ = run_timed(torch, [lambda: osa.optim_step_adamw(plan.handle, h, sc["lr"], None, None,
                                                                  sc["step"])], steps, warmup)
        plan.close()
        moved = T_ADAMW_STATES16 if sdt == osa.OPTIM_F16 else B_ADAMW_STATES16  # bf16: one pass
        out[name] = dict(ms=ms, bytes_per_element=B_ADAMW_STATES16, moved_per_element=moved,
                         gbs=gbs(B_ADAMW_STATES16 * n, ms), frac=gbs(B_ADAMW_STATES16 * n, ms) / PEAK_HBM_GBS)
        del p, m, v
    del p0, g
    torch.cuda.empty_cache()
    return dict(workload="adamw_scaled_states_fp32_4096x4096", elements=n, kernels=out)


def bench_c1(torch, osa, synth, steps, warmup):
    wl = synth.c1_single_tensor()
    n, hp = wl.numel, wl.hp
    p0 = synth.initial_param_device(wl.tensors[0], wl.p_std, wl.index, 0, "cuda")
    g = synth.device_normal(n, wl.g_std, "cuda", wl.index, 0, 1, synth.GRAD)
    A = adam_buffers(torch, [p0], osa.OPTIM_F32)
    plan = osa.Plan(osa.TensorList(A["p"], [g], m=A["m"], v=A["v"], weight_decay=[hp.wd]),
                    osa.OPTIM_ALGO_ADAMW)
    s = scalars(torch, hp.lr)
    h = osa.optim_adamw_hp(hp.beta1, hp.beta2, hp.eps)
    step = lambda: osa.optim_step_adamw(plan.handle, h, s["lr"], None, None, s["step"])
    stats = []
    ms, _, _ = run_timed(torch, [step], steps, warmup, stats)
    cold = dist(run_timed_cold(torch, step, steps, warmup))
    plan.close()
    return dict(workload=wl.name, elements=n, ms_per_step=ms, elements_per_s=n / (ms * 1e-3),
                gbs=gbs(B_ADAMW_F32 * n, ms), frac=gbs(B_ADAMW_F32 * n, ms) / PEAK_HBM_GBS, warm=stats[0],
                cold=dict(cold, gbs=gbs(B_ADAMW_F32 * n, cold["median_ms"])),
                note="29 MB of state: cache-resident and launch-bound when warm; cold = after a 1 GiB "
                     "write between steps, inputs from HBM")


def bench_c3(torch, osa, synth, steps, warmup):
    wl = synth.c3_llama_1b()
    hp, scale = wl.hp, wl.extra["loss_scale"]
    specs = wl.tensors
    n = wl.numel
    p0 = [synth.initial_param_device(s, wl.p_std, wl.index, i, "cuda") for i, s in enumerate(specs)]
    A = adam_buffers(torch, p0, osa.OPTIM_BF16, param_bf16=True)
    del p0
    torch.cuda.empty_cache()
    G = []
    for i, s in enumerate(specs):
        x = synth.device_normal(s.numel, wl.g_std, "cuda", wl.index, i, 0, synth.GRAD)
        G.append(x.mul_(scale).to(torch.bfloat16).view(torch.int16))
        del x
    wd = [0.0 if s.is_norm else hp.wd for s in specs]
    tl = osa.TensorList(A["p"], G, m=A["m"], v=A["v"], remainders=A["r"], weight_decay=wd,
                        param_dtype=osa.OPTIM_BF16, grad_dtype=osa.OPTIM_BF16)
    plan = osa.Plan(tl, osa.OPTIM_ALGO_ADAMW)
    s = scalars(torch, 0.0, inv_scale=1.0 / scale)
    osa.optim_plan_set_schedule(plan.handle, osa.OPTIM_SCHED_COSINE, hp.lr, 0.0, wl.steps, s["iter"])
    h = osa.optim_adamw_hp(hp.beta1, hp.beta2, hp.eps)

    def finite():
        s["found_inf"].zero_()
        osa.optim_check_finite(plan.handle, s["found_inf"])

    def step():
        osa.optim_step_adamw(plan.handle, h, s["lr"], s["inv_scale"], s["found_inf"], s["step"])

    ms, per_call, _ = run_timed(torch, [finite, step], steps, warmup)

    # the same list in the full AMP loop with clipping folded into the step:
    # check + global norm (one read of the grads), clipped step, scale update
    scale_dev = torch.tensor([scale], dtype=torch.float32, device="cuda")
    tracker = torch.zeros(1, dtype=torch.int32, device="cuda")
    norm = torch.zeros(1, dtype=torch.float32, device="cuda")
    clip = torch.zeros(1, dtype=torch.float32, device="cuda")

    def check_norm():
        s["found_inf"].zero_()
        osa.optim_grad_norm(plan.handle, s["inv_scale"], CLIP_MAX_NORM, s["found_inf"], norm, clip)

    def clipped_step():
        osa.optim_step_adamw(plan.handle, h, s["lr"], clip, s["found_inf"], s["step"])

    def scaler():
        osa.optim_scaler_update(scale_dev, s["inv_scale"], tracker, s["found_inf"], 2.0, 0.5, 2000)

    ms_c, per_c, _ = run_timed(torch, [check_norm, clipped_step, scaler], steps, warmup)
    plan.close()
    del A, G
    torch.cuda.empty_cache()
    b = B_BF16R_AMP * n
    return dict(workload=wl.name, elements=n, ms_per_step=ms, elements_per_s=n / (ms * 1e-3),
                gbs=gbs(b, ms), frac=gbs(b, ms) / PEAK_HBM_GBS,
                kernels={"check_finite_bf16": dict(ms=per_call[0], gbs=gbs(2.0 * n, per_call[0])),
                         "adamw_bf16_remainder": dict(ms=per_call[1], gbs=gbs(26.0 * n, per_call[1]))},
                amp_clip_loop=dict(
                    ms_per_step=ms_c, elements_per_s=n / (ms_c * 1e-3), gbs=gbs(b, ms_c),
                    frac=gbs(b, ms_c) / PEAK_HBM_GBS, max_norm=CLIP_MAX_NORM,
                    kernels={"check_and_norm_bf16": dict(ms=per_c[0], gbs=gbs(2.0 * n, per_c[0])),
                             "adamw_bf16_remainder_clipped": dict(ms=per_c[1], gbs=gbs(26.0 * n, per_c[1])),
                             "scaler_update": dict(ms=per_c[2])}))


def bench_c4(torch, osa, synth, steps, warmup):
    wl = synth.c4_blockwise()
    n, hp = wl.numel, wl.hp
    out = {}
    for bits, block, bpe in ((8, wl.extra["block8"], B_8BIT), (4, wl.extra["block4"], B_4BIT)):
        p = synth.initial_param_device(wl.tensors[0], wl.p_std, wl.index, 0, "cuda")
        g = synth.device_normal(n, wl.g_std, "cuda", wl.index, 0, 1, synth.GRAD)
        nb = (n * bits + 7) // 8
        qm = torch.zeros(nb, dtype=torch.uint8, device="cuda")
        qv = torch.zeros(nb, dtype=torch.uint8, device="cuda")
        am = torch.zeros(n // block, dtype=torch.float32, device="cuda")
        av = torch.zeros(n // block, dtype=torch.float32, device="cuda")
        tl = osa.TensorList([p], [g], qm=[qm], qv=[qv], absmax_m=[am], absmax_v=[av], weight_decay=[hp.wd])
        plan = osa.Plan(tl, osa.OPTIM_ALGO_BLOCKWISE, bits=bits, block=block)
        s = scalars(torch, hp.lr)
        h = osa.optim_adamw_hp(hp.beta1, hp.beta2, hp.eps)
        ms, _, _ = run_timed(torch, [lambda: osa.optim_step_8bit_blockwise(
            plan.handle, h, bits, block, s["lr"], None, None, s["step"])], steps, warmup)
        plan.close()
        out[f"blockwise_{bits}bit_block{block}"] = dict(
            elements=n, ms_per_step=ms, elements_per_s=n / (ms * 1e-3), bytes_per_element=bpe,
            gbs=gbs(bpe * n, ms), frac=gbs(bpe * n, ms) / PEAK_HBM_GBS)
        # the same states in the interleaved layout (m and v codes side by side
        # in one array, the two absmax values of a block in another)
        del qm, qv, am, av
        torch.cuda.empty_cache()
        qmv = torch.zeros(2 * nb, dtype=torch.uint8, device="cuda")
        amv = torch.zeros(2 * (n // block), dtype=torch.float32, device="cuda")
        tl = osa.TensorList([p], [g], qm=[qmv], absmax_m=[amv], weight_decay=[hp.wd])
        plan = osa.Plan(tl, osa.OPTIM_ALGO_BLOCKWISE, bits=bits, block=block,
                        state_layout=osa.OPTIM_LAYOUT_INTERLEAVED)
        s = scalars(torch, hp.lr)
        ms, _, _ = run_timed(torch, [lambda: osa.optim_step_8bit_blockwise(
            plan.handle, h, bits, block, s["lr"], None, None, s["step"])], steps, warmup)
        plan.close()
        out[f"blockwise_{bits}bit_block{block}_interleaved"] = dict(
            elements=n, ms_per_step=ms, elements_per_s=n / (ms * 1e-3), bytes_per_element=bpe,
            gbs=gbs(bpe * n, ms), frac=gbs(bpe * n, ms) / PEAK_HBM_GBS)
        del qmv, amv
        torch.cuda.empty_cache()
        qm = torch.zeros(nb, dtype=torch.uint8, device="cuda")
        qv = torch.zeros(nb, dtype=torch.uint8, device="cuda")
        am = torch.zeros(n // block, dtype=torch.float32, device="cuda")
        av = torch.zeros(n // block, dtype=torch.float32, device="cuda")
        # the same list with AdEMAMix's third state (slow EMA m2, signed codes)
        qm2 = torch.zeros(nb, dtype=torch.uint8, device="cuda")
        am2 = torch.zeros(n // block, dtype=torch.float32, device="cuda")
        tl = osa.TensorList([p], [g], qm=[qm], qv=[qv], absmax_m=[am], absmax_v=[av], qm2=[qm2],
                            absmax_m2=[am2], weight_decay=[hp.wd])
        plan = osa.Plan(tl, osa.OPTIM_ALGO_BLOCKWISE_ADEMAMIX, bits=bits, block=block)
        s = scalars(torch, hp.lr)
        he = osa.optim_ademamix_hp(hp.beta1, hp.beta2, C4_BETA3, C4_ALPHA, hp.eps)
        ms, _, _ = run_timed(torch, [lambda: osa.optim_step_8bit_blockwise_ademamix(
            plan.handle, he, bits, block, s["lr"], None, None, s["step"])], steps, warmup)
        plan.close()
        bpe3 = bpe + bits / 4 + 8 / block  # + m2 codes and absmax, read and written
        out[f"blockwise_ademamix_{bits}bit_block{block}"] = dict(
            elements=n, ms_per_step=ms, elements_per_s=n / (ms * 1e-3), bytes_per_element=bpe3,
            gbs=gbs(bpe3 * n, ms), frac=gbs(bpe3 * n, ms) / PEAK_HBM_GBS, beta3=C4_BETA3, alpha=C4_ALPHA)
        del p, g, qm, qv, am, av, qm2, am2
        torch.cuda.empty_cache()
    return dict(workload=wl.name, **out)


def bench_c5(torch, osa, synth, steps, warmup):
    wl = synth.c5_adam_mini_7b()
    hp = wl.hp
    specs = wl.tensors
    names = [s.name for s in specs]
    sizes = [s.numel for s in specs]
    kinds, hn, wds = osa.adam_mini_partition(names, sizes, dim=wl.extra["dim"], n_heads=wl.extra["n_heads"],
                                             weight_decay=hp.wd)
    vlen = [s if k == osa.OPTIM_MINI_FULL_V else s // h for k, s, h in zip(kinds, sizes, hn)]
    P = [synth.initial_param_device(s, wl.p_std, wl.index, i, "cuda") for i, s in enumerate(specs)]
    G = [synth.device_normal(s.numel, wl.g_std, "cuda", wl.index, i, 1, synth.GRAD) for i, s in enumerate(specs)]
    M = [torch.zeros(k, dtype=torch.float32, device="cuda") for k in sizes]
    V = [torch.zeros(k, dtype=torch.float32, device="cuda") for k in vlen]
    tl = osa.TensorList(P, G, m=M, v=V, weight_decay=wds, mini_kind=kinds, head_numel=hn)
    plan = osa.Plan(tl, osa.OPTIM_ALGO_ADAM_MINI)
    s = scalars(torch, hp.lr)
    h = osa.optim_adamw_hp(hp.beta1, hp.beta2, hp.eps)
    ms, _, _ = run_timed(torch, [lambda: osa.optim_step_adam_mini(plan.handle, h, s["lr"], None, None,
                                                                   s["step"])], max(3, steps // 2), 2)
    plan.close()
    n = wl.numel
    full = sum(sz for sz, k in zip(sizes, kinds) if k == osa.OPTIM_MINI_FULL_V)
    alg = 28.0 * full + 20.0 * (n - full)
    del P, G, M, V
    torch.cuda.empty_cache()
    return dict(workload=wl.name, elements=n, ms_per_step=ms, elements_per_s=n / (ms * 1e-3),
                gbs=gbs(alg, ms), frac=gbs(alg, ms) / PEAK_HBM_GBS,
                note="algorithmic bytes 28 B/elem for full-v tensors, 20 B/elem for shared-v tensors; "
                     "the kernels read g twice (block sums, then update), segment by segment, so the "
                     "second read comes mostly from the Infinity Cache")


# --------------------------------------------------------------------------
def cpu_baseline(synth, target_s):
    """The CPU oracle (scalar C, fp64, as it stands) on row slices of the
    headline tensor: AdamW + AdEMAMix, same hyperparameters.  First one
    thread on 256 rows for about half the time budget, then one thread per
    host core, each on its own 256 rows (the oracle's calls release the
    interpreter lock), for the same number of steps.  `value` is the
    all-cores rate; the single-thread rate is reported beside it."""
    import threading

    import numpy as np
    import oracle
    wl = synth.c2_decay_stress()
    hp = wl.hp
    rows = 256
    n = rows * 4096

    def state(chunk):
        p0 = synth.host_normal(n, wl.p_std, wl.index, 0, chunk, synth.P0).astype(np.float64)
        g = synth.host_normal(n, wl.g_std, wl.index, 0, chunk, synth.GRAD).astype(np.float64)
        return dict(g=g, a=(p0.copy(), np.zeros(n), np.zeros(n)),
                    b=(p0.copy(), np.zeros(n), np.zeros(n), np.zeros(n)))

    def one_step(st, t):
        pa, ma, va = st["a"]
        pb, m1, m2, nu = st["b"]
        oracle.adamw_step(pa, ma, va, st["g"], hp.lr, hp.beta1, hp.beta2, hp.eps, hp.wd, t)
        oracle.ademamix_step(pb, m1, m2, nu, st["g"], hp.lr, hp.beta1, hp.beta2, wl.extra["beta3"],
                             wl.extra["alpha"], hp.eps, hp.wd, t)

    st0 = state(0)
    steps, spent = 0, 0.0
    while spent < target_s / 2 and steps < 1000:
        t0 = time.perf_counter()
        one_step(st0, steps + 1)
        spent += time.perf_counter() - t0
        steps += 1
    single = 2 * n * steps / spent
    cores = max(1, min(os.cpu_count() or 1, 16))
    states = [state(1 + c) for c in range(cores)]

    def worker(st):
        for t in range(1, steps + 1):
            one_step(st, t)

    threads = [threading.Thread(target=worker, args=(st,)) for st in states]
    t0 = time.perf_counter()
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    wall = time.perf_counter() - t0
    return dict(value=2 * n * steps * cores / wall, unit="elements/s", cores=cores, kind="oracle",
                single_thread_value=single,
                sample=f"{rows}x4096 rows of the 4096x4096 tensor per thread, AdamW + AdEMAMix, {steps} steps: "
                       f"1 thread {spent:.1f} s, then {cores} threads {wall:.1f} s "
                       f"({os.cpu_count()} host cores visible)")


KERNEL_SOURCES = {  # kernel -> sources its device code comes from
    "adamw_fp32": ("device_common.h", "kernels_adam.hip"),
    "ademamix_fp32": ("device_common.h", "kernels_adam.hip"),
    "blockwise_8bit": ("device_common.h", "kernels_blockwise.hip"),
    "blockwise_8bit_interleaved": ("device_common.h", "kernels_blockwise.hip"),
    "blockwise_4bit": ("device_common.h", "kernels_blockwise.hip"),
    "blockwise_4bit_interleaved": ("device_common.h", "kernels_blockwise.hip"),
    "blockwise_ademamix_8bit": ("device_common.h", "kernels_blockwise.hip"),
    "blockwise_ademamix_4bit": ("device_common.h", "kernels_blockwise.hip"),
}


def kernel_sources_sha256(kernel_key):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel_key]:
        with open(os.path.join(ROOT, "optimizer_step_adamw_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_from_profile(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE scaled by a plain copy of known size), valid
    only while the kernel's sources are the ones the counters were taken on."""
    path = os.path.join(ROOT, "profiles", f"counters_{kernel_key}.txt")
    if not os.path.exists(path) or kernel_key not in KERNEL_SOURCES:
        return None
    text = open(path).read()
    m = re.search(r"kernel_sources_sha256:\s*([0-9a-f]{64})", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_sources_sha256(kernel_key):
        return None
    return float(t.group(1))


def copy_probe(torch, nbytes=256 << 20, reps=5):
    """Plain device-to-device copy of a known size: the streaming ceiling for
    context, and the known-size kernel that scales the traffic counters."""
    x = torch.randn(nbytes // 4, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        y.copy_(x)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del x, y
    return dict(bytes=2 * nbytes, ms=ms, gbs=2 * nbytes / (ms * 1e-3) / 1e9)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the optimizer step needs no cross-GPU exchange; see the sharding notes)", file=sys.stderr)
        sys.exit(2)
    import torch
    import optimizer_step_adamw_amd as osa
    import synth
    osa.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    log(f"device: {torch.cuda.get_device_name(0)}")
    copy = copy_probe(torch)
    log(f"copy probe: {json.dumps(copy)}")
    head = bench_headline(torch, osa, synth, args.steps, args.warmup)
    log(f"headline: {head['ms_per_step']:.4f} ms/step, {head['elements_per_s']:.4e} elem/s, "
        f"{json.dumps(head['kernels'])}")
    secondary = {}
    todo = [] if args.secondary == "none" else args.secondary.split(",")
    fns = dict(c1=bench_c1, c3=bench_c3, c4=bench_c4, c5=bench_c5, lion_lamb=bench_lion_lamb,
               master=bench_master, states16=bench_states16, many=bench_many)
    for key in todo:
        t0 = time.perf_counter()
        secondary[key] = fns[key](torch, osa, synth, args.steps, args.warmup)
        log(f"{key}: {json.dumps(secondary[key])} ({time.perf_counter() - t0:.1f} s)")
    dom_name = max(head["kernels"], key=lambda k: head["kernels"][k]["ms"])
    dom = head["kernels"][dom_name]
    roof = dict(bound="hbm", kernel=dom_name, achieved=dom["gbs"], peak=PEAK_HBM_GBS, unit="GB/s",
                frac=dom["gbs"] / PEAK_HBM_GBS, traffic=traffic_from_profile(dom_name),
                bytes_per_launch=dom["bytes"], launch_ms=dom["ms"])
    cpu = cpu_baseline(synth, args.cpu_seconds) if args.cpu_seconds > 0 else None
    out = {
        "metric": METRIC,
        "value": head["elements_per_s"],
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": head["workload"], "elements": head["elements"],
                   "optimizers": ["adamw", "ademamix"], "lr": 0.1, "weight_decay": 0.1,
                   "betas": [0.9, 0.999], "beta3": 0.9999, "alpha": 5.0},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": head["kernels"],
        "copy_ceiling": copy,
        "secondary": secondary,
        "environment": environment(torch),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
