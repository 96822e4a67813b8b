"""Benchmark of the fused AdamW-family optimizer step on one MI355X.

Headline workload: Adam-mini over the Llama-7B-shaped list (32 layers,
d 4096, 32 heads, ffn 11008, vocab 32000, untied output: 291 fp32 tensors,
6,738,415,616 parameters), the largest workload that fits one GPU.  One
benchmark step = one optim_step_adam_mini call through the C ABI (per-step
scalars, block sums of g^2, per-block finalize, m / p update, segment by
segment).  `value` is optimizer element-updates per second with every input
resident in HBM.

Rooflines (`rooflines`, one entry per kernel; the headline's is `roofline`):
the device duration of every launch, from the library's kernel trace (each
launch's own start and end, recorded inside the timed region, on the stream
the library launches on), against the kernel's algorithmic bytes per launch
and MI355X's 8 TB/s:
  - the Adam-mini update kernel (7B list);
  - AdamW and AdEMAMix fp32 on 4096 x 4096 (four state sets taken in turn,
    1.1 / 1.3 GB together, so no set is still in the 256 MB Infinity Cache
    when its turn comes);
  - the bf16 + int16-remainder AdamW kernel (moments in separate arrays, and
    interleaved in one array per tensor) and the non-finite check on the
    Llama-1.1B-shaped list;
  - blockwise 8-bit (block 256) and 4-bit (block 128) on 268M elements, in
    the separate and the interleaved state layout.
Each entry also carries `ceiling`: the bandwidth of the same access pattern
streamed without arithmetic by a probe kernel (probes/stream_probe.hip; same
arrays, lane layout, unit size and access kind), and `frac_of_ceiling`; and
`rw_bound`: the bandwidth its read and written bytes would reach at the
read-only and write-only probes' rates, one after the other.

Secondary workloads (`secondary`): the 1M-element tensor, the 1.1B AMP loop
with global-norm clipping and the dynamic loss scale, blockwise states in the
interleaved layout and with AdEMAMix's third state, Lion, LAMB, fp32 masters
with 16-bit model copies, scaled 16-bit moments, and 16M AdamW elements as
lists of 4096 and 65536 tensors.  Gradients are drawn once per workload,
outside the timed region.
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
B_BF16R = 26.0                # R bf16 p, int16 r, bf16 g, m, v (14) + W (12)
B_FINITE_BF16 = 2.0           # R bf16 g
B_MINI_SHARED = 20.0          # Adam-mini shared v: R p g m (12) + W p m (8)
B_MINI_FULL = 28.0            # Adam-mini full v: as AdamW
B_MINI_SUMS = 4.0             # block sums: R g
B_8BIT = 4 + 4 + 1 + 1 + 8 / 256 + 4 + 1 + 1 + 8 / 256
B_4BIT = 4 + 4 + 0.5 + 0.5 + 8 / 128 + 4 + 0.5 + 0.5 + 8 / 128
CLIP_MAX_NORM = 1.0           # global-norm clip of the Llama 1.1B AMP loop
C4_BETA3, C4_ALPHA = 0.9999, 5.0   # AdEMAMix on the blockwise list: the 4096^2 run's values
ROTATE = 4                    # state sets taken in turn for the 4096^2 rooflines


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--secondary", default="c2,c3,c4,probes,c1,amp,c4x,lion_lamb,master,states16,many",
                    help="comma list of further workloads (c2,c3,c4,probes: the rooflines and ceilings; "
                         "c1,amp,c4x,lion_lamb,master,states16,many) or 'none'")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample (0 = skip)")
    return ap.parse_args()


def dist(xs):
    """Median and 10th / 90th percentiles (ms)."""
    a = sorted(xs)
    q = lambda f: a[min(len(a) - 1, int(round(f * (len(a) - 1))))]
    return dict(median_ms=q(0.5), p10_ms=q(0.1), p90_ms=q(0.9))


def gbs(nbytes, ms):
    return nbytes / (ms * 1e-3) / 1e9


def timed_region(torch, calls, steps):
    """`steps` steps between two events on the current stream (the stream
    the library launches on), bracketed by device synchronisation; returns
    (ms per step, host wall ms per step)."""
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(steps):
        for c in calls:
            c()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps, (time.perf_counter() - t0) * 1e3 / steps


def run_timed(torch, calls, steps, warmup, plans=(), trace_cap=0):
    """calls: zero-arg functions forming one step.  `warmup` untimed steps,
    then a timed region of `steps` steps (the step time).  If `plans` are
    given, a second timed region of `steps` steps follows with their kernel
    traces on (each launch's start and end stamped by its own dispatch): the
    per-kernel durations.  The trace adds a few microseconds between
    launches but nothing to a kernel's own duration, so the step time comes
    from the untraced region.  Returns (ms per step, host wall ms per step,
    {plan: trace records}, ms per step of the traced region)."""
    import optimizer_step_adamw_amd as osa
    for _ in range(warmup):
        for c in calls:
            c()
    ms, wall = timed_region(torch, calls, steps)
    recs, ms_traced = {}, None
    if plans:
        for p in plans:
            osa.optim_plan_trace(p, trace_cap)
        ms_traced, _ = timed_region(torch, calls, steps)
        for p in plans:
            r, dropped = osa.optim_plan_trace_read(p, trace_cap)
            if dropped:
                raise RuntimeError(f"kernel trace full: {dropped} launches untraced")
            osa.optim_plan_trace(p, 0)
            recs[p] = r
    return ms, wall, recs, ms_traced


def kernel_stats(records, name=None):
    """Launch count, total / mean ms, per-launch spread and grid sizes of the
    records of one kernel (all records if name is None)."""
    sel = [r for r in records if name is None or r[0] == name]
    if not sel:
        return None
    ms = [r[2] for r in sel]
    return dict(launches=len(ms), total_ms=sum(ms), mean_ms=sum(ms) / len(ms),
                workgroups=sorted(set(r[1] for r in sel)), **dist(ms))


def roofline_entry(kernel, workload, bytes_per_launch, stats, ceiling=None, traffic=None, note=None):
    achieved = gbs(bytes_per_launch, stats["mean_ms"])
    e = dict(kernel=kernel, workload=workload, bound="hbm", achieved=achieved, peak=PEAK_HBM_GBS, unit="GB/s",
             frac=achieved / PEAK_HBM_GBS, traffic=traffic, bytes_per_launch=bytes_per_launch,
             launch_ms=stats["mean_ms"], launches=stats["launches"], workgroups=stats["workgroups"],
             launch_spread_ms=dict(p10=stats["p10_ms"], median=stats["median_ms"], p90=stats["p90_ms"]))
    if ceiling:
        e["ceiling"] = ceiling
        e["frac_of_ceiling"] = achieved / ceiling["gbs"]
    if note:
        e["note"] = note
    return e


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


def clocks():
    """The GPU's clock levels as rocm-smi reports them (read only, after the
    timed work, so the current levels are mostly idle ones): the supported
    shader-clock levels and the current shader and memory clocks; None where
    the tool is missing or says nothing."""
    import subprocess

    def smi(arg):
        for exe in ("/opt/rocm/bin/rocm-smi", "rocm-smi"):
            try:
                r = subprocess.run([exe, arg, "--json"], capture_output=True, text=True, timeout=20)
            except (OSError, subprocess.SubprocessError):
                continue
            try:
                data = json.loads(r.stdout[r.stdout.find("{"):])
            except ValueError:
                return None
            return next((v for k, v in sorted(data.items()) if k.startswith("card")), None)
        return None
    cur, lev = smi("--showclocks"), smi("--showclkfrq")
    if not cur and not lev:
        return None
    return dict(levels=lev, after_run={k: v for k, v in (cur or {}).items() if "clock" in k.lower()})


def environment(torch):
    """Device and software the numbers were taken on."""
    pr = torch.cuda.get_device_properties(0)
    return dict(device=pr.name, arch=getattr(pr, "gcnArchName", None), compute_units=pr.multi_processor_count,
                hbm_gib=round(pr.total_memory / 2 ** 30, 1), torch=torch.__version__,
                hip=getattr(torch.version, "hip", None), host_cpus=os.cpu_count(),
                clocks=clocks(), library_sources_sha256=library_sources_sha256())


KERNEL_SOURCES = {  # traffic summary name -> sources its device code comes from
    "adamw_fp32": ("device_common.h", "kernels_adam.hip"),
    "ademamix_fp32": ("device_common.h", "kernels_adam.hip"),
    "adamw_bf16_remainder": ("device_common.h", "kernels_adam.hip"),
    "adamw_bf16_remainder_interleaved": ("device_common.h", "kernels_adam.hip"),
    "adamw_fp32_packs": ("device_common.h", "kernels_adam.hip"),
    "check_finite_bf16": ("device_common.h", "kernels_util.hip"),
    "check_norm_bf16": ("device_common.h", "kernels_util.hip"),
    "mini_update": ("device_common.h", "kernels_mini.hip"),
    "mini_sumsq": ("device_common.h", "kernels_mini.hip"),
    "lion_fp32": ("device_common.h", "kernels_lion_lamb.hip"),
    "lamb_moments": ("device_common.h", "kernels_lion_lamb.hip"),
    "lamb_update": ("device_common.h", "kernels_lion_lamb.hip"),
    "scaled_bf16": ("device_common.h", "kernels_scaled.hip"),
    "scaled_f16_pass1": ("device_common.h", "kernels_scaled.hip"),
    "scaled_f16_pass2": ("device_common.h", "kernels_scaled.hip"),
    "blockwise_8bit": ("device_common.h", "kernels_blockwise.hip"),
    "blockwise_8bit_interleaved": ("device_common.h", "kernels_blockwise.hip"),
    "blockwise_4bit": ("device_common.h", "kernels_blockwise.hip"),
    "blockwise_4bit_interleaved": ("device_common.h", "kernels_blockwise.hip"),
    "blockwise_ademamix_8bit": ("device_common.h", "kernels_blockwise.hip"),
    "blockwise_ademamix_4bit": ("device_common.h", "kernels_blockwise.hip"),
}


def kernel_sources_sha256(key):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[key]:
        with open(os.path.join(ROOT, "optimizer_step_adamw_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_from_profile(key):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE scaled by a plain copy of known size), valid
    only while the kernel's sources are the ones the counters were taken on."""
    path = os.path.join(ROOT, "profiles", f"counters_{key}.txt")
    if not os.path.exists(path) or key not in KERNEL_SOURCES:
        return None
    text = open(path).read()
    m = re.search(r"kernel_sources_sha256:\s*([0-9a-f]{64})", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_sources_sha256(key):
        return None
    return float(t.group(1))


# --------------------------------------------------------------------------
def adam_buffers(torch, p0_list, param_bf16=False, ademamix=False, v_len=None):
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


def free(torch):
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------
# headline: Adam-mini, Llama-7B-shaped list
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
    plan = osa.Plan(osa.TensorList(P, G, m=M, v=V, weight_decay=wds, mini_kind=kinds, head_numel=hn),
                    osa.OPTIM_ALGO_ADAM_MINI)
    s = scalars(torch, hp.lr)
    h = osa.optim_adamw_hp(hp.beta1, hp.beta2, hp.eps)
    step = lambda: osa.optim_step_adam_mini(plan.handle, h, s["lr"], None, None, s["step"])
    ms, wall, recs, ms_traced = run_timed(torch, [step], steps, warmup, plans=[plan.handle], trace_cap=300 * steps)
    rec = recs[plan.handle]
    n = wl.numel
    full = sum(sz for sz, k in zip(sizes, kinds) if k == osa.OPTIM_MINI_FULL_V)
    shared = n - full
    alg = B_MINI_FULL * full + B_MINI_SHARED * shared
    upd, sums, fin = (kernel_stats(rec, k) for k in ("mini_update_kernel", "mini_sumsq_kernel",
                                                    "mini_finalize_kernel"))
    per_step = lambda st: st["launches"] // steps
    kern = dict(
        mini_update=dict(launches_per_step=per_step(upd), ms_per_step=upd["total_ms"] / steps,
                         bytes_per_step=alg, gbs=gbs(alg, upd["total_ms"] / steps)),
        mini_sumsq=dict(launches_per_step=per_step(sums), ms_per_step=sums["total_ms"] / steps,
                        bytes_per_step=B_MINI_SUMS * shared, gbs=gbs(B_MINI_SUMS * shared, sums["total_ms"] / steps)),
        mini_finalize=dict(launches_per_step=per_step(fin), ms_per_step=fin["total_ms"] / steps))
    kernel_ms = kernel_stats(rec)["total_ms"] / steps
    roof = roofline_entry("mini_update_kernel", wl.name, alg / per_step(upd), upd,
                          traffic=traffic_from_profile("mini_update"),
                          note="bytes per launch: the update's algorithmic bytes per step (28 B/elem full v, "
                               "20 B/elem shared v: R p g m, W p m) over its launches per step (one per "
                               "segment); g was read by the segment's block sums just before, so part of the "
                               "update's g comes from the Infinity Cache")
    plan.close()
    del P, G, M, V
    free(torch)
    return dict(workload=wl.name, elements=n, ms_per_step=ms, wall_ms_per_step=wall,
                traced_ms_per_step=ms_traced, elements_per_s=n / (ms * 1e-3), algorithmic_bytes_per_step=alg,
                gbs=gbs(alg, ms), frac=gbs(alg, ms) / PEAK_HBM_GBS,
                kernel_ms_per_step=kernel_ms, kernels=kern, roofline=roof,
                note="step bytes: 28 B/elem for the 2 full-v tensors, 20 B/elem for the 289 shared-v tensors "
                     "(the block-sum pass's read of g is not counted)")


# --------------------------------------------------------------------------
# 4096 x 4096: AdamW and AdEMAMix, four state sets in turn
def bench_c2(torch, osa, synth, steps, warmup):
    wl = synth.c2_decay_stress()
    n, hp = wl.numel, wl.hp
    out = {}
    for ade in (False, True):
        sets = []
        for k in range(ROTATE):
            p0 = synth.initial_param_device(wl.tensors[0], wl.p_std, wl.index, 0, "cuda")
            g = synth.device_normal(n, wl.g_std, "cuda", wl.index, 0, 1 + k, synth.GRAD)
            B = adam_buffers(torch, [p0], ademamix=ade)
            del p0
            tl = osa.TensorList(B["p"], [g], m=B["m"], v=B["v"], m2=B["m2"], weight_decay=[hp.wd])
            plan = osa.Plan(tl, osa.OPTIM_ALGO_ADEMAMIX if ade else osa.OPTIM_ALGO_ADAMW)
            sets.append((plan, scalars(torch, hp.lr), B, g))
        if ade:
            h = osa.optim_ademamix_hp(hp.beta1, hp.beta2, wl.extra["beta3"], wl.extra["alpha"], hp.eps)
            fn = osa.optim_step_ademamix
        else:
            h = osa.optim_adamw_hp(hp.beta1, hp.beta2, hp.eps)
            fn = osa.optim_step_adamw
        calls = [(lambda pl=pl, sc=sc: fn(pl.handle, h, sc["lr"], None, None, sc["step"]))
                 for pl, sc, _, _ in sets]
        ms, _, recs, _ = run_timed(torch, calls, steps, warmup, plans=[x[0].handle for x in sets], trace_cap=4 * steps)
        rec = [r for v in recs.values() for r in v]
        name = "ademamix_fp32" if ade else "adamw_fp32"
        bpe = B_ADEMAMIX_F32 if ade else B_ADAMW_F32
        out[name] = dict(stats=kernel_stats(rec), bytes=bpe * n, ms_per_call=ms / ROTATE)
        for pl, _, _, _ in sets:
            pl.close()
        del sets
        free(torch)
    return dict(workload=wl.name, elements=n, rotate=ROTATE, kernels=out)


# --------------------------------------------------------------------------
# Llama 1.1B: bf16 params + int16 remainders, bf16 grads x 65536, AMP, cosine lr
def c3_state(torch, osa, synth, interleaved=False):
    """interleaved: the moments of each tensor in one array, in blocks of 1024
    elements (the plan's interleaved moment layout)."""
    wl = synth.c3_llama_1b()
    hp, scale = wl.hp, wl.extra["loss_scale"]
    specs = wl.tensors
    p0 = [synth.initial_param_device(s, wl.p_std, wl.index, i, "cuda") for i, s in enumerate(specs)]
    A = adam_buffers(torch, p0, param_bf16=True)
    del p0
    if interleaved:
        A["m"] = [torch.zeros(2 * ((x.numel() + 1023) // 1024 * 1024), device="cuda") for x in A["p"]]
        A["v"] = None
    free(torch)
    G = []
    for i, s in enumerate(specs):
        x = synth.device_normal(s.numel, wl.g_std, "cuda", wl.index, i, 0, synth.GRAD)
        G.append(x.mul_(scale).to(torch.bfloat16).view(torch.int16))
        del x
    wd = [0.0 if s.is_norm else hp.wd for s in specs]
    tl = osa.TensorList(A["p"], G, m=A["m"], v=A["v"], remainders=A["r"], weight_decay=wd,
                        param_dtype=osa.OPTIM_BF16, grad_dtype=osa.OPTIM_BF16)
    plan = osa.Plan(tl, osa.OPTIM_ALGO_ADAMW,
                    state_layout=osa.OPTIM_LAYOUT_INTERLEAVED if interleaved else osa.OPTIM_LAYOUT_SEPARATE)
    s = scalars(torch, 0.0, inv_scale=1.0 / scale)
    osa.optim_plan_set_schedule(plan.handle, osa.OPTIM_SCHED_COSINE, hp.lr, 0.0, wl.steps, s["iter"])
    h = osa.optim_adamw_hp(hp.beta1, hp.beta2, hp.eps)
    return wl, plan, s, h, (A, G)


def bench_c3(torch, osa, synth, steps, warmup):
    wl, plan, s, h, keep = c3_state(torch, osa, synth)
    n = wl.numel

    def finite():
        s["found_inf"].zero_()
        osa.optim_check_finite(plan.handle, s["found_inf"])

    def step():
        osa.optim_step_adamw(plan.handle, h, s["lr"], s["inv_scale"], s["found_inf"], s["step"])

    ms, _, recs, _ = run_timed(torch, [finite, step], steps, warmup, plans=[plan.handle], trace_cap=4 * steps)
    rec = recs[plan.handle]
    plan.close()
    del keep
    free(torch)
    # the same step with the moments interleaved (one array per tensor)
    _, plan, s, h, keep = c3_state(torch, osa, synth, interleaved=True)
    ms_il, _, recs, _ = run_timed(torch, [finite, step], steps, warmup, plans=[plan.handle], trace_cap=4 * steps)
    rec_il = recs[plan.handle]
    plan.close()
    del keep
    free(torch)
    b = (B_BF16R + B_FINITE_BF16) * n
    return dict(workload=wl.name, elements=n, ms_per_step=ms, elements_per_s=n / (ms * 1e-3),
                gbs=gbs(b, ms), frac=gbs(b, ms) / PEAK_HBM_GBS,
                interleaved_moments=dict(ms_per_step=ms_il, elements_per_s=n / (ms_il * 1e-3)),
                kernels=dict(adamw_bf16_remainder=dict(stats=kernel_stats(rec, "adam_kernel"), bytes=B_BF16R * n),
                             adamw_bf16_remainder_interleaved=dict(stats=kernel_stats(rec_il, "adam_kernel"),
                                                                   bytes=B_BF16R * n),
                             check_finite_bf16=dict(stats=kernel_stats(rec, "finite_kernel"),
                                                    bytes=B_FINITE_BF16 * n)))


def bench_amp(torch, osa, synth, steps, warmup):
    """The 1.1B list in the full AMP loop with clipping folded into the step:
    check + global norm (one read of the grads), clipped step, scale update."""
    wl, plan, s, h, keep = c3_state(torch, osa, synth)
    n = wl.numel
    scale_dev = torch.tensor([wl.extra["loss_scale"]], dtype=torch.float32, device="cuda")
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

    ms, _, recs, _ = run_timed(torch, [check_norm, clipped_step, scaler], steps, warmup, plans=[plan.handle],
                            trace_cap=8 * steps)
    rec = recs[plan.handle]
    plan.close()
    del keep
    free(torch)
    b = (B_BF16R + B_FINITE_BF16) * n
    ks = {k: kernel_stats(rec, k) for k in ("finite_kernel", "norm_stage1_kernel", "norm_finalize_kernel",
                                            "adam_kernel")}
    return dict(workload=wl.name + "_clip_loop", elements=n, ms_per_step=ms, elements_per_s=n / (ms * 1e-3),
                gbs=gbs(b, ms), frac=gbs(b, ms) / PEAK_HBM_GBS, max_norm=CLIP_MAX_NORM,
                kernels={k: dict(mean_ms=v["mean_ms"], launches=v["launches"]) for k, v in ks.items() if v},
                check_and_norm_gbs=gbs(B_FINITE_BF16 * n, ks["finite_kernel"]["mean_ms"]))


# --------------------------------------------------------------------------
# blockwise 8-bit / 4-bit states, 268M elements
def bench_blockwise(torch, osa, synth, steps, warmup, interleaved=False, ademamix=False):
    wl = synth.c4_blockwise()
    n, hp = wl.numel, wl.hp
    out = {}
    for bits, block, bpe in ((8, wl.extra["block8"], B_8BIT), (4, wl.extra["block4"], B_4BIT)):
        p = synth.initial_param_device(wl.tensors[0], wl.p_std, wl.index, 0, "cuda")
        g = synth.device_normal(n, wl.g_std, "cuda", wl.index, 0, 1, synth.GRAD)
        nb = (n * bits + 7) // 8
        keep = []
        if interleaved:
            qmv = torch.zeros(2 * nb, dtype=torch.uint8, device="cuda")
            amv = torch.zeros(2 * (n // block), dtype=torch.float32, device="cuda")
            keep += [qmv, amv]
            tl = osa.TensorList([p], [g], qm=[qmv], absmax_m=[amv], weight_decay=[hp.wd])
            plan = osa.Plan(tl, osa.OPTIM_ALGO_BLOCKWISE, bits=bits, block=block,
                            state_layout=osa.OPTIM_LAYOUT_INTERLEAVED)
        else:
            mk = lambda: torch.zeros(nb, dtype=torch.uint8, device="cuda")
            ak = lambda: torch.zeros(n // block, dtype=torch.float32, device="cuda")
            qm, qv, am, av = mk(), mk(), ak(), ak()
            keep += [qm, qv, am, av]
            kw = {}
            if ademamix:
                qm2, am2 = mk(), ak()
                keep += [qm2, am2]
                kw = dict(qm2=[qm2], absmax_m2=[am2])
            tl = osa.TensorList([p], [g], qm=[qm], qv=[qv], absmax_m=[am], absmax_v=[av], weight_decay=[hp.wd], **kw)
            plan = osa.Plan(tl, osa.OPTIM_ALGO_BLOCKWISE_ADEMAMIX if ademamix else osa.OPTIM_ALGO_BLOCKWISE,
                            bits=bits, block=block)
        s = scalars(torch, hp.lr)
        if ademamix:
            he = osa.optim_ademamix_hp(hp.beta1, hp.beta2, C4_BETA3, C4_ALPHA, hp.eps)
            call = lambda: osa.optim_step_8bit_blockwise_ademamix(plan.handle, he, bits, block, s["lr"], None, None,
                                                                  s["step"])
            bpe = bpe + bits / 4 + 8 / block  # + m2 codes and absmax, read and written
        else:
            h = osa.optim_adamw_hp(hp.beta1, hp.beta2, hp.eps)
            call = lambda: osa.optim_step_8bit_blockwise(plan.handle, h, bits, block, s["lr"], None, None, s["step"])
        ms, _, recs, _ = run_timed(torch, [call], steps, warmup, plans=[plan.handle], trace_cap=2 * steps)
        st = kernel_stats(recs[plan.handle])
        plan.close()
        name = ("blockwise_ademamix_" if ademamix else "blockwise_") + f"{bits}bit" + \
               ("_interleaved" if interleaved else "")
        out[name] = dict(elements=n, block=block, ms_per_step=ms, elements_per_s=n / (ms * 1e-3),
                         bytes_per_element=bpe, stats=st, bytes=bpe * n,
                         gbs=gbs(bpe * n, st["mean_ms"]), frac=gbs(bpe * n, st["mean_ms"]) / PEAK_HBM_GBS)
        del p, g, keep, tl
        free(torch)
    return dict(workload=wl.name, kernels=out)


# --------------------------------------------------------------------------
# access-pattern ceilings
# read / written bytes per element of each roofline workload (the
# Adam-mini update: per element of the 7B list, full-v and shared-v mixed)
_C5_N, _C5_FULL = 6738415616, 2 * 32000 * 4096
RW_SPLIT = {
    "adam_mini_llama7b": ((16.0 * _C5_FULL + 12.0 * (_C5_N - _C5_FULL)) / _C5_N,
                          (12.0 * _C5_FULL + 8.0 * (_C5_N - _C5_FULL)) / _C5_N),
    "adamw_fp32_4096x4096": (16.0, 12.0),
    "ademamix_fp32_4096x4096": (20.0, 16.0),
    "adamw_bf16_remainder_llama1b": (14.0, 12.0),
    "adamw_bf16_remainder_interleaved_llama1b": (14.0, 12.0),
    "check_finite_bf16_llama1b": (2.0, 0.0),
    "blockwise_8bit_268M": (4 + 4 + 1 + 1 + 8 / 256, 4 + 1 + 1 + 8 / 256),
    "blockwise_4bit_268M": (4 + 4 + 0.5 + 0.5 + 8 / 128, 4 + 0.5 + 0.5 + 8 / 128),
    "blockwise_8bit_interleaved_268M": (4 + 4 + 1 + 1 + 8 / 256, 4 + 1 + 1 + 8 / 256),
    "blockwise_4bit_interleaved_268M": (4 + 4 + 0.5 + 0.5 + 8 / 128, 4 + 0.5 + 0.5 + 8 / 128),
}


def rw_bound(ceil, split):
    """The bandwidth a kernel reading R and writing W bytes per element would
    reach if its reads ran at the read-only probe's rate and its writes at the
    write-only probe's, one after the other: (R + W) / (R / read + W / write)."""
    if not split or "read_fp32_268M" not in ceil or "write_fp32_268M" not in ceil:
        return None
    r, w = split
    rd = ceil["read_fp32_268M"]["gbs"]
    wr = max(ceil["write_fp32_268M"]["gbs"], ceil.get("write_fp32_ordinary_268M", {}).get("gbs", 0.0))
    return dict(gbs=(r + w) / (r / rd + w / wr), read_gbs=rd, write_gbs=wr, read_bytes=r, write_bytes=w)


def probe_time(torch, fn, reps, warmup=2):
    """Mean ms of one probe launch (events around each launch on the current
    stream; each probe is one kernel)."""
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    ev = []
    for i in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn(i)
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / reps


def bench_probes(torch, reps):
    import probes
    out = {}
    f32 = lambda k: torch.empty(k, dtype=torch.float32, device="cuda").normal_()
    # 4096^2 AdamW / AdEMAMix patterns: four array sets in turn, units of 4096
    # (the kernels' form at this size)
    n = 1 << 24
    for name, arrays, bpe in (("adamw_4096x4096", 4, B_ADAMW_F32), ("ademamix_4096x4096", 5, B_ADEMAMIX_F32)):
        sets = [[f32(n) for _ in range(arrays)] for _ in range(ROTATE)]
        if arrays == 4:
            fn = lambda i: probes.call("probe_adamw", *sets[i % ROTATE], n, 4)
        else:
            fn = lambda i: probes.call("probe_ademamix", *sets[i % ROTATE], n, 4)
        ms = probe_time(torch, fn, 4 * reps)
        out[name] = dict(ms=ms, bytes=bpe * n, gbs=gbs(bpe * n, ms))
        del sets
        free(torch)
    n = 1 << 28
    # Llama-1.1B bf16 + remainder pattern (2048-element units)
    h16 = lambda: torch.empty(n, dtype=torch.int16, device="cuda").random_(-30000, 30000)
    arr = [h16(), h16(), h16(), f32(n), f32(n)]
    ms = probe_time(torch, lambda i: probes.call("probe_bf16r", *arr, n, 0), reps)
    out["bf16r_268M"] = dict(ms=ms, bytes=B_BF16R * n, gbs=gbs(B_BF16R * n, ms))
    # the same with m and v interleaved in one array of 2n floats
    mv = f32(2 * n)
    ms = probe_time(torch, lambda i: probes.call("probe_bf16r", arr[0], arr[1], arr[2], mv, None, n, 1), reps)
    out["bf16r_il_268M"] = dict(ms=ms, bytes=B_BF16R * n, gbs=gbs(B_BF16R * n, ms))
    del mv
    sink = torch.zeros(n // 32768, dtype=torch.int32, device="cuda")
    ms = probe_time(torch, lambda i: probes.call("probe_read", arr[2], n, 2, sink), reps)
    out["read_bf16_268M"] = dict(ms=ms, bytes=2.0 * n, gbs=gbs(2.0 * n, ms))
    ms = probe_time(torch, lambda i: probes.call("probe_read", arr[3], n, 4, sink), reps)
    out["read_fp32_268M"] = dict(ms=ms, bytes=4.0 * n, gbs=gbs(4.0 * n, ms))
    del arr
    free(torch)
    # Adam-mini update pattern with g from HBM (R p g m, W p m; units of 4096)
    arr = [f32(n), f32(n), f32(n)]
    ms = probe_time(torch, lambda i: probes.call("probe_mini", *arr, n), reps)
    out["mini_3r2w_268M"] = dict(ms=ms, bytes=B_MINI_SHARED * n, gbs=gbs(B_MINI_SHARED * n, ms))
    ms = probe_time(torch, lambda i: probes.call("probe_copy", arr[0], arr[1], n), reps)
    out["copy_268M"] = dict(ms=ms, bytes=8.0 * n, gbs=gbs(8.0 * n, ms))
    # one write-only stream, non-temporal stores (as the step kernels) and ordinary ones
    for nt, key in ((1, "write_fp32_268M"), (0, "write_fp32_ordinary_268M")):
        ms = probe_time(torch, lambda i: probes.call("probe_write", arr[2], n, nt), reps)
        out[key] = dict(ms=ms, bytes=4.0 * n, gbs=gbs(4.0 * n, ms))
    del arr
    free(torch)
    # blockwise separate layout: 8-bit block 256 on 4096-element units, 4-bit
    # block 128 on 8192 (the step's units), 2 rows of loads in flight or the
    # whole unit; the better one is the ceiling
    for bits, block, bpe, unit_rows in ((8, 256, B_8BIT, 4), (4, 128, B_4BIT, 8)):
        nb = n * bits // 8
        arr = [f32(n), f32(n), torch.zeros(nb, dtype=torch.uint8, device="cuda"),
               torch.zeros(nb, dtype=torch.uint8, device="cuda"),
               torch.zeros(n // block, device="cuda"), torch.zeros(n // block, device="cuda")]
        best = None
        for rows in (2, unit_rows):
            ms = probe_time(torch, lambda i: probes.call("probe_blockwise", *arr, n, bits, unit_rows, rows), reps)
            e = dict(ms=ms, bytes=bpe * n, gbs=gbs(bpe * n, ms), unit=unit_rows * 1024, rows_in_flight=rows)
            best = e if best is None or e["gbs"] > best["gbs"] else best
        out[f"blockwise_{bits}bit_268M"] = best
        del arr
        free(torch)
    return out


# --------------------------------------------------------------------------
# secondary workloads
def bench_c1(torch, osa, synth, steps, warmup):
    """The 1M-element tensor (29 MB of state): warm (cache-resident, launch
    bound) and cold (a 1 GiB device write between steps, outside the events)."""
    wl = synth.c1_single_tensor()
    n, hp = wl.numel, wl.hp
    p0 = synth.initial_param_device(wl.tensors[0], wl.p_std, wl.index, 0, "cuda")
    g = synth.device_normal(n, wl.g_std, "cuda", wl.index, 0, 1, synth.GRAD)
    A = adam_buffers(torch, [p0])
    plan = osa.Plan(osa.TensorList(A["p"], [g], m=A["m"], v=A["v"], weight_decay=[hp.wd]), osa.OPTIM_ALGO_ADAMW)
    s = scalars(torch, hp.lr)
    h = osa.optim_adamw_hp(hp.beta1, hp.beta2, hp.eps)
    step = lambda: osa.optim_step_adamw(plan.handle, h, s["lr"], None, None, s["step"])
    ms, _, recs, _ = run_timed(torch, [step], steps, warmup, plans=[plan.handle], trace_cap=2 * steps)
    warm = kernel_stats(recs[plan.handle])
    scratch = torch.empty((1 << 30) // 4, dtype=torch.float32, device="cuda")
    osa.optim_plan_trace(plan.handle, 2 * steps)
    for i in range(steps):
        scratch.fill_(float(i))
        step()
    cold = kernel_stats(osa.optim_plan_trace_read(plan.handle)[0])
    osa.optim_plan_trace(plan.handle, 0)
    plan.close()
    del scratch
    free(torch)
    return dict(workload=wl.name, elements=n, ms_per_step=ms, elements_per_s=n / (ms * 1e-3),
                warm=dict(warm, gbs=gbs(B_ADAMW_F32 * n, warm["mean_ms"])),
                cold=dict(cold, gbs=gbs(B_ADAMW_F32 * n, cold["mean_ms"])),
                note="kernel durations from the trace; warm = back to back (29 MB in the Infinity Cache), "
                     "cold = after a 1 GiB write")


def bench_lion_lamb(torch, osa, synth, steps, warmup):
    """Lion and LAMB on the 4096 x 4096 tensor (beta (0.9, 0.99) for Lion;
    LAMB eps 1e-6), each kernel timed from the trace."""
    wl = synth.c2_decay_stress()
    n, hp = wl.numel, wl.hp
    p0 = synth.initial_param_device(wl.tensors[0], wl.p_std, wl.index, 0, "cuda")
    g = synth.device_normal(n, wl.g_std, "cuda", wl.index, 0, 1, synth.GRAD)
    A = adam_buffers(torch, [p0])
    B = adam_buffers(torch, [p0])
    del p0
    pl = osa.Plan(osa.TensorList(A["p"], [g], m=A["m"], weight_decay=[hp.wd]), osa.OPTIM_ALGO_LION)
    pm = osa.Plan(osa.TensorList(B["p"], [g], m=B["m"], v=B["v"], weight_decay=[hp.wd]), osa.OPTIM_ALGO_LAMB)
    sl, sm = scalars(torch, 1e-4), scalars(torch, 1e-3)
    hl = osa.optim_lion_hp(0.9, 0.99)
    hm = osa.optim_adamw_hp(hp.beta1, hp.beta2, 1e-6)
    calls = [lambda: osa.optim_step_lion(pl.handle, hl, sl["lr"], None, None, sl["step"]),
             lambda: osa.optim_step_lamb(pm.handle, hm, sm["lr"], None, None, sm["step"])]
    ms, _, recs, _ = run_timed(torch, calls, steps, warmup, plans=[pl.handle, pm.handle], trace_cap=4 * steps)
    lion = kernel_stats(recs[pl.handle])
    lamb = {k: kernel_stats(recs[pm.handle], k) for k in ("lamb_moments_kernel", "lamb_trust_kernel",
                                                         "lamb_update_kernel")}
    lamb_ms = sum(v["mean_ms"] for v in lamb.values())
    pl.close()
    pm.close()
    del A, B, g
    free(torch)
    return dict(workload="lion_lamb_fp32_4096x4096", elements=n, ms_per_step=ms,
                kernels={"lion_fp32": dict(mean_ms=lion["mean_ms"], gbs=gbs(B_LION_F32 * n, lion["mean_ms"]),
                                           frac=gbs(B_LION_F32 * n, lion["mean_ms"]) / PEAK_HBM_GBS),
                         "lamb_fp32": dict(ms=lamb_ms, passes={k: v["mean_ms"] for k, v in lamb.items()},
                                           gbs=gbs(B_ADAMW_F32 * n, lamb_ms),
                                           frac=gbs(B_ADAMW_F32 * n, lamb_ms) / PEAK_HBM_GBS,
                                           note="algorithmic 28 B/elem; the two passes move 40 B/elem")},
                note="back to back on one state each (the state partly stays in the Infinity Cache)")


def bench_master(torch, osa, synth, steps, warmup):
    """AdamW with an fp32 master and a bf16 or fp16 model copy, 4096 x 4096."""
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
        _, _, recs, _ = run_timed(torch, [lambda: osa.optim_step_adamw(plan.handle, h, sc["lr"], None, None, sc["step"])],
                               steps, warmup, plans=[plan.handle], trace_cap=2 * steps)
        st = kernel_stats(recs[plan.handle])
        plan.close()
        out[name] = dict(mean_ms=st["mean_ms"], bytes_per_element=B_ADAMW_MASTER,
                         gbs=gbs(B_ADAMW_MASTER * n, st["mean_ms"]),
                         frac=gbs(B_ADAMW_MASTER * n, st["mean_ms"]) / PEAK_HBM_GBS)
        del master, model, m, v
    del p0, g
    free(torch)
    return dict(workload="adamw_master_copy_4096x4096", elements=n, kernels=out)


def bench_states16(torch, osa, synth, steps, warmup):
    """AdamW with fp16 or bf16 moments and per-tensor scales, 4096 x 4096;
    frac on the algorithmic 20 B/element (the two-pass fp16 step moves 28)."""
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
        ms, _, recs, _ = run_timed(torch, [lambda: osa.optim_step_adamw(plan.handle, h, sc["lr"], None, None,
                                                                     sc["step"])],
                                steps, warmup, plans=[plan.handle], trace_cap=4 * steps)
        kt = kernel_stats(recs[plan.handle])["total_ms"] / steps
        plan.close()
        moved = T_ADAMW_STATES16 if sdt == osa.OPTIM_F16 else B_ADAMW_STATES16
        out[name] = dict(kernel_ms_per_step=kt, bytes_per_element=B_ADAMW_STATES16, moved_per_element=moved,
                         gbs=gbs(B_ADAMW_STATES16 * n, kt), frac=gbs(B_ADAMW_STATES16 * n, kt) / PEAK_HBM_GBS)
        del p, m, v
    del p0, g
    free(torch)
    return dict(workload="adamw_scaled_states_fp32_4096x4096", elements=n, kernels=out)


def bench_many(torch, osa, synth, steps, warmup):
    """16,777,216 AdamW fp32 elements as one tensor, as 4096 tensors of 4096
    and as 65536 of 256 (views of one allocation per array), four state sets
    in turn: the cost of the multi-tensor traversal."""
    n = 1 << 24
    out = {}
    for count in (1, 4096, 65536):
        size = n // count
        sets = []
        for k in range(ROTATE):
            P = torch.randn(n, device="cuda") * 0.02
            G = torch.randn(n, device="cuda") * 1e-3
            M = torch.zeros(n, device="cuda")
            V = torch.zeros(n, device="cuda")
            views = lambda x: [x[i * size:(i + 1) * size] for i in range(count)]
            plan = osa.Plan(osa.TensorList(views(P), views(G), m=views(M), v=views(V),
                                           weight_decay=[0.1] * count), osa.OPTIM_ALGO_ADAMW)
            sets.append((plan, scalars(torch, 1e-3), (P, G, M, V)))
        h = osa.optim_adamw_hp(0.9, 0.999, 1e-8)
        calls = [(lambda pl=pl, s=s: osa.optim_step_adamw(pl.handle, h, s["lr"], None, None, s["step"]))
                 for pl, s, _ in sets]
        _, _, recs, _ = run_timed(torch, calls, steps, warmup, plans=[x[0].handle for x in sets], trace_cap=2 * steps)
        st = kernel_stats([r for v in recs.values() for r in v])
        out[f"tensors_{count}x{size}"] = dict(mean_ms=st["mean_ms"], gbs=gbs(B_ADAMW_F32 * n, st["mean_ms"]),
                                              frac=gbs(B_ADAMW_F32 * n, st["mean_ms"]) / PEAK_HBM_GBS,
                                              workgroups=st["workgroups"])
        if count == 65536:  # packs of small tensors: the pack kernel's own counters
            out[f"tensors_{count}x{size}"]["traffic"] = traffic_from_profile("adamw_fp32_packs")
        for pl, _, _ in sets:
            pl.close()
        del sets
        free(torch)
    return dict(workload="adamw_fp32_16M_as_many_tensors", elements=n, rotate=ROTATE, lists=out)


# --------------------------------------------------------------------------
def cpu_baseline(synth, target_s):
    """The CPU oracle (scalar C, fp64, as it stands) on a sample of the 7B
    Adam-mini list, per thread: two q-projection head blocks (2 x 524,288
    elements, shared v per block), a 1,048,576-element slice of a w1 matrix
    as one shared-v block, one norm (4096, no decay) and a 1,048,576-element
    slice of the embedding (full v), same hyperparameters and distributions.
    First one thread for about half the time budget, then one thread per
    host core (each on its own sample) for the same number of steps; `value`
    is the all-cores rate in element updates per second."""
    import threading

    import numpy as np
    import oracle
    wl = synth.c5_adam_mini_7b()
    hp = wl.hp
    head = wl.extra["dim"] * wl.extra["dim"] // wl.extra["n_heads"]
    parts = [("head", 2 * head, head, hp.wd, False), ("scalar", 1 << 20, 1 << 20, hp.wd, False),
             ("norm", 4096, 4096, 0.0, True), ("full", 1 << 20, 1, hp.wd, False)]
    per_step = sum(p[1] for p in parts)

    def state(chunk):
        st = []
        for j, (_, n, block, wd, is_norm) in enumerate(parts):
            p0 = (np.ones(n) if is_norm else
                  synth.host_normal(n, wl.p_std, wl.index, 100 + chunk, j, synth.P0).astype(np.float64))
            g = synth.host_normal(n, wl.g_std, wl.index, 100 + chunk, j, synth.GRAD).astype(np.float64)
            v = np.zeros(n if block == 1 else n // block)
            st.append((p0, np.zeros(n), v, g, block, wd))
        return st

    def one_step(st, t):
        for p, m, v, g, block, wd in st:
            if block == 1:
                oracle.adamw_step(p, m, v, g, hp.lr, hp.beta1, hp.beta2, hp.eps, wd, t)
            else:
                oracle.adam_mini_step(p, m, v, g, block, hp.lr, hp.beta1, hp.beta2, hp.eps, wd, t)

    st0 = state(0)
    steps, spent = 0, 0.0
    while spent < target_s / 2 and steps < 1000:
        t0 = time.perf_counter()
        one_step(st0, steps + 1)
        spent += time.perf_counter() - t0
        steps += 1
    single = per_step * steps / spent
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
    return dict(value=per_step * steps * cores / wall, unit="elements/s", cores=cores, kind="oracle",
                single_thread_value=single,
                sample=f"per thread {per_step} elements of the 7B Adam-mini list (2 q head blocks of {head}, "
                       f"a 1M slice of w1 as one shared-v block, a 4096 norm, a 1M embedding slice with full v), "
                       f"{steps} steps: 1 thread {spent:.1f} s, then {cores} threads {wall:.1f} s "
                       f"({os.cpu_count()} host cores visible)")


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
    head = bench_c5(torch, osa, synth, args.steps, args.warmup)
    log(f"headline c5: {head['ms_per_step']:.3f} ms/step, {head['elements_per_s']:.4e} elem/s, "
        f"update {head['roofline']['achieved']:.0f} GB/s")
    todo = [] if args.secondary == "none" else [k for k in args.secondary.split(",") if k]
    res = {}
    fns = dict(c2=bench_c2, c3=bench_c3, c4=bench_blockwise, c1=bench_c1, amp=bench_amp,
               c4x=lambda *a: dict(interleaved=bench_blockwise(*a, interleaved=True),
                                   ademamix=bench_blockwise(*a, ademamix=True)),
               lion_lamb=bench_lion_lamb, master=bench_master, states16=bench_states16, many=bench_many)
    for key in todo:
        t0 = time.perf_counter()
        if key == "probes":
            res[key] = bench_probes(torch, max(5, args.steps // 2))
        else:
            res[key] = fns[key](torch, osa, synth, args.steps, args.warmup)
        log(f"{key}: {json.dumps(res[key])} ({time.perf_counter() - t0:.1f} s)")
    ceil = res.get("probes", {})
    # per-kernel rooflines, each against its access pattern's ceiling
    roofs = [dict(head["roofline"], ceiling=ceil.get("mini_3r2w_268M"),
                  frac_of_ceiling=(head["roofline"]["achieved"] / ceil["mini_3r2w_268M"]["gbs"]
                                   if "mini_3r2w_268M" in ceil else None))]
    if "c2" in res:
        c2 = res["c2"]
        for k, pk in (("adamw_fp32", "adamw_4096x4096"), ("ademamix_fp32", "ademamix_4096x4096")):
            e = c2["kernels"][k]
            roofs.append(roofline_entry("adam_kernel", f"{k}_4096x4096", e["bytes"], e["stats"], ceil.get(pk),
                                        traffic_from_profile(k),
                                        note=f"{ROTATE} state sets taken in turn (none stays in the Infinity Cache)"))
    if "c3" in res:
        for k, pk in (("adamw_bf16_remainder", "bf16r_268M"), ("adamw_bf16_remainder_interleaved", "bf16r_il_268M"),
                      ("check_finite_bf16", "read_bf16_268M")):
            e = res["c3"]["kernels"][k]
            roofs.append(roofline_entry("adam_kernel" if k.startswith("adamw") else "finite_kernel",
                                        f"{k}_llama1b", e["bytes"], e["stats"], ceil.get(pk),
                                        traffic_from_profile(k)))
    if "c4" in res:
        for k, pk in (("blockwise_8bit", "blockwise_8bit_268M"), ("blockwise_4bit", "blockwise_4bit_268M")):
            e = res["c4"]["kernels"][k]
            roofs.append(roofline_entry("blockwise_kernel", f"{k}_268M", e["bytes"], e["stats"], ceil.get(pk),
                                        traffic_from_profile(k)))
    if "c4x" in res:  # the same steps with each element's m and v codes side by side
        for k in ("blockwise_8bit_interleaved", "blockwise_4bit_interleaved"):
            e = res["c4x"]["interleaved"]["kernels"][k]
            roofs.append(roofline_entry("blockwise_kernel", f"{k}_268M", e["bytes"], e["stats"], None,
                                        traffic_from_profile(k)))
    for e in roofs:
        rw = rw_bound(ceil, RW_SPLIT.get(e["workload"]))
        if rw:
            e["rw_bound"] = dict(rw, frac=e["achieved"] / rw["gbs"])
    roof = roofs[0]
    cpu = cpu_baseline(synth, args.cpu_seconds) if args.cpu_seconds > 0 else None
    wl_c5 = synth.c5_adam_mini_7b()
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
        "config": {"workload": head["workload"], "elements": head["elements"], "tensors": len(wl_c5.tensors),
                   "optimizer": "adam_mini", "lr": wl_c5.hp.lr, "betas": [wl_c5.hp.beta1, wl_c5.hp.beta2],
                   "eps": wl_c5.hp.eps, "weight_decay": wl_c5.hp.wd, "layers": 32, "dim": 4096, "n_heads": 32,
                   "ffn": 11008, "vocab": 32000},
        "roofline": roof,
        "rooflines": roofs,
        "cpu_baseline": cpu,
        "headline": head,
        "ceilings": ceil,
        "secondary": {k: v for k, v in res.items() if k != "probes"},
        "environment": environment(torch),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
