"""C-ABI checks that need no GPU: the library loads, exports every function
the header declares, and its host-only entry points (codebook, plan sizing
and validation) behave.  Device pointers here are fake integers: the
size query validates and lays out a plan without touching the device."""
import os
import re

import numpy as np
import pytest

import optimizer_step_adamw_amd as osa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(osa.LIB_PATH):
        osa.build_library()
    return osa.lib()


def header_functions():
    text = open(os.path.join(ROOT, "include", "optim_step.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(optim_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_function(L):
    declared = header_functions()
    assert len(declared) == 23, declared
    assert sorted(osa.EXPORTED) == declared
    for name in declared:
        assert hasattr(L, name), name


@pytest.mark.parametrize("bits,signed", [(8, True), (8, False), (4, True), (4, False)])
def test_codebook_matches_oracle(L, orc, bits, signed):
    """Two independent implementations of the same map definition."""
    vals, thr = osa.optim_quant_codebook(bits, signed)
    mb = bits - 1 if signed else bits
    M = orc.dynamic_map(mb)
    assert np.array_equal(vals.view(np.uint32), M.view(np.uint32))
    assert np.array_equal(thr[1:].view(np.uint32), orc.thresholds(M)[1:].view(np.uint32))


class Fake:
    """Non-overlapping fake device addresses."""

    def __init__(self):
        self.next = 1 << 40

    def __call__(self, nbytes, misalign=0):
        a = self.next + misalign
        self.next += ((nbytes + 4095) // 4096 + 1) * 4096
        return a


def fake_list(sizes, algo=osa.OPTIM_ALGO_ADAMW, fake=None, **kw):
    fake = fake or Fake()
    n = len(sizes)
    args = dict(params=[fake(4 * s) for s in sizes], grads=[fake(4 * s) for s in sizes],
                m=[fake(4 * s) for s in sizes], v=[fake(4 * s) for s in sizes],
                weight_decay=[0.01] * n, numel=sizes)
    if algo == osa.OPTIM_ALGO_ADEMAMIX:
        args["m2"] = [fake(4 * s) for s in sizes]
    args.update(kw)
    return osa.TensorList(**args)


def ws(tl, algo, opts=None):
    return osa.optim_plan_workspace_size(tl, algo, opts)


def expect_error(code, fn):
    with pytest.raises(osa.OptimError) as ei:
        fn()
    assert ei.value.code == code, str(ei.value)
    assert len(str(ei.value)) > 20


def test_workspace_size_grows_with_units(L):
    a = ws(fake_list([4096]), osa.OPTIM_ALGO_ADAMW)
    b = ws(fake_list([4096] * 300), osa.OPTIM_ALGO_ADAMW)
    assert 0 < a < b
    assert ws(osa.TensorList([], [], weight_decay=[], numel=[]), osa.OPTIM_ALGO_ADAMW) > 0


def test_validation_codes(L):
    f = Fake()
    expect_error(osa.OPTIM_EINVAL, lambda: ws(fake_list([-1]), osa.OPTIM_ALGO_ADAMW))
    expect_error(osa.OPTIM_EINVAL, lambda: ws(fake_list([(1 << 48) + 1]), osa.OPTIM_ALGO_ADAMW))
    assert ws(fake_list([(1 << 33) + 5]), osa.OPTIM_ALGO_ADAMW) > 0  # beyond 32-bit element counts
    expect_error(osa.OPTIM_EALIGN, lambda: ws(
        fake_list([8], params=[f(32, misalign=2)]), osa.OPTIM_ALGO_ADAMW))
    # a gradient that aliases another tensor's moment buffer
    fk = Fake()
    tl = fake_list([1024, 1024], fake=fk)
    m0 = tl.struct.m[0]
    expect_error(osa.OPTIM_EINVAL, lambda: ws(
        fake_list([1024, 1024], grads=[f(4096), m0 + 64]), osa.OPTIM_ALGO_ADAMW))
    expect_error(osa.OPTIM_EINVAL, lambda: ws(fake_list([8], weight_decay=[-0.1]), osa.OPTIM_ALGO_ADAMW))
    expect_error(osa.OPTIM_EINVAL, lambda: ws(fake_list([8]), osa.OPTIM_ALGO_ADEMAMIX))  # no m2
    expect_error(osa.OPTIM_EUNSUPPORTED, lambda: ws(
        fake_list([8] * 65, weight_decay=[i * 1e-3 for i in range(65)]), osa.OPTIM_ALGO_ADAMW))
    expect_error(osa.OPTIM_EUNSUPPORTED, lambda: ws(
        fake_list([8], param_dtype=osa.OPTIM_BF16), osa.OPTIM_ALGO_ADAMW))  # no remainder
    expect_error(osa.OPTIM_EDTYPE, lambda: ws(fake_list([8], grad_dtype=7), osa.OPTIM_ALGO_ADAMW))
    expect_error(osa.OPTIM_EINVAL, lambda: ws(fake_list([8]), 9))


def test_adam_mini_validation(L):
    kinds = [osa.OPTIM_MINI_HEAD]
    ok = fake_list([4096], mini_kind=kinds, head_numel=[512])
    assert ws(ok, osa.OPTIM_ALGO_ADAM_MINI) > 0
    expect_error(osa.OPTIM_EINVAL, lambda: ws(
        fake_list([4096], mini_kind=kinds, head_numel=[500]), osa.OPTIM_ALGO_ADAM_MINI))
    expect_error(osa.OPTIM_EINVAL, lambda: ws(
        fake_list([4096], mini_kind=[7], head_numel=[0]), osa.OPTIM_ALGO_ADAM_MINI))
    # launch segments: any positive gradient-byte bound (0 = default), never negative
    seg = lambda b: osa.optim_plan_opts(0, 0, 0, 0, 0, b)
    for b in (0, 1, 1 << 40):
        assert ws(ok, osa.OPTIM_ALGO_ADAM_MINI, seg(b)) == ws(ok, osa.OPTIM_ALGO_ADAM_MINI)
    expect_error(osa.OPTIM_EINVAL, lambda: ws(ok, osa.OPTIM_ALGO_ADAM_MINI, seg(-1)))


def test_blockwise_validation(L):
    f = Fake()
    n = 1000
    kw = dict(m=None, v=None, qm=[f(n)], qv=[f(n)], absmax_m=[f(64)], absmax_v=[f(64)])
    for bits, block in ((8, 256), (8, 64), (4, 128), (4, 512)):
        assert ws(fake_list([n], fake=f, **kw), osa.OPTIM_ALGO_BLOCKWISE,
                  osa.optim_plan_opts(bits, block, 0, 0)) > 0
    for bits, block in ((8, 512), (4, 64), (6, 256), (8, 100)):
        expect_error(osa.OPTIM_EINVAL, lambda: ws(
            fake_list([n], fake=f, **kw), osa.OPTIM_ALGO_BLOCKWISE, osa.optim_plan_opts(bits, block, 0, 0)))
    expect_error(osa.OPTIM_EINVAL, lambda: ws(fake_list([n], fake=f, **kw), osa.OPTIM_ALGO_BLOCKWISE, None))
    # the codes of one tensor overlapping its own parameter
    expect_error(osa.OPTIM_EINVAL, lambda: ws(
        fake_list([n], **kw), osa.OPTIM_ALGO_BLOCKWISE, osa.optim_plan_opts(8, 256, 0, 0)))


def test_blockwise_interleaved_layout_validation(L):
    """Interleaved state: codes of m and v in qm (2 bytes an element at 8
    bits, 1 at 4), (absmax m, absmax v) pairs in absmax_m; qv and absmax_v
    absent; the 2-state blockwise step only."""
    f = Fake()
    n = 1000
    il = lambda bits, block: osa.optim_plan_opts(bits, block, 0, 0, 0, 0, osa.OPTIM_LAYOUT_INTERLEAVED)
    kw = lambda **o: {**dict(m=None, v=None, qm=[f(2 * n)], absmax_m=[f(64)]), **o}
    for bits, block in ((8, 256), (8, 64), (4, 128), (4, 512)):
        assert ws(fake_list([n], fake=f, **kw()), osa.OPTIM_ALGO_BLOCKWISE, il(bits, block)) > 0
    # qv / absmax_v given, absmax only 4-byte aligned, codes overlapping the next tensor's
    expect_error(osa.OPTIM_EINVAL, lambda: ws(fake_list([n], fake=f, **kw(qv=[f(n)])), osa.OPTIM_ALGO_BLOCKWISE,
                                              il(8, 256)))
    expect_error(osa.OPTIM_EINVAL, lambda: ws(fake_list([n], fake=f, **kw(absmax_v=[f(64)])),
                                              osa.OPTIM_ALGO_BLOCKWISE, il(8, 256)))
    expect_error(osa.OPTIM_EALIGN, lambda: ws(fake_list([n], fake=f, **kw(absmax_m=[f(64, misalign=4)])),
                                              osa.OPTIM_ALGO_BLOCKWISE, il(8, 256)))
    q = f(4 * n)
    expect_error(osa.OPTIM_EINVAL, lambda: ws(  # 8-bit codes take 2n bytes: q + n overlaps
        fake_list([n, n], fake=f, m=None, v=None, qm=[q, q + n], absmax_m=[f(64), f(64)]),
        osa.OPTIM_ALGO_BLOCKWISE, il(8, 256)))
    assert ws(fake_list([n, n], fake=f, m=None, v=None, qm=[q, q + 2 * n], absmax_m=[f(64), f(64)]),
              osa.OPTIM_ALGO_BLOCKWISE, il(8, 256)) > 0
    # other algorithms, unknown layouts
    expect_error(osa.OPTIM_EUNSUPPORTED, lambda: ws(
        fake_list([n], fake=f, **kw(qm2=[f(n)], absmax_m2=[f(64)])), osa.OPTIM_ALGO_BLOCKWISE_ADEMAMIX, il(8, 256)))
    expect_error(osa.OPTIM_EUNSUPPORTED, lambda: ws(fake_list([n], fake=f, v=None), osa.OPTIM_ALGO_LION,
                                                    osa.optim_plan_opts(0, 0, 0, 0, 0, 0, 1)))
    expect_error(osa.OPTIM_EINVAL, lambda: ws(fake_list([n], fake=f, **kw()), osa.OPTIM_ALGO_BLOCKWISE,
                                              osa.optim_plan_opts(8, 256, 0, 0, 0, 0, 2)))


def test_interleaved_moment_layout_validation(L):
    """AdamW / AdEMAMix with interleaved moments: m holds K * 1024 *
    ceil(numel / 1024) floats (K = 2, or 3 with m2), v and m2 absent; the
    other algorithms and 16-bit moments refuse the layout."""
    f = Fake()
    il = lambda sdt=0: osa.optim_plan_opts(0, 0, 0, 0, sdt, 0, osa.OPTIM_LAYOUT_INTERLEAVED)
    n = 1000  # one block: the buffer is K * 1024 floats
    assert ws(fake_list([n], fake=f, v=None, m=[f(2 * 4096)]), osa.OPTIM_ALGO_ADAMW, il()) > 0
    assert ws(fake_list([n], fake=f, v=None, m=[f(3 * 4096)]), osa.OPTIM_ALGO_ADEMAMIX, il()) > 0
    # v or m2 given, m misaligned
    expect_error(osa.OPTIM_EINVAL, lambda: ws(fake_list([n], fake=f), osa.OPTIM_ALGO_ADAMW, il()))
    expect_error(osa.OPTIM_EINVAL, lambda: ws(fake_list([n], fake=f, v=None, m2=[f(4 * n)]),
                                              osa.OPTIM_ALGO_ADEMAMIX, il()))
    expect_error(osa.OPTIM_EALIGN, lambda: ws(fake_list([n], fake=f, v=None, m=[f(8192, misalign=2)]),
                                              osa.OPTIM_ALGO_ADAMW, il()))
    # two tensors of 1500 elements: each buffer spans 2 * 2048 floats, so
    # buffers 2 * 1500 floats apart overlap and 2 * 2048 apart do not
    k = 1500
    base = f(4 * 2 * 2048 * 2)
    expect_error(osa.OPTIM_EINVAL, lambda: ws(fake_list([k, k], fake=f, v=None, m=[base, base + 4 * 2 * k]),
                                              osa.OPTIM_ALGO_ADAMW, il()))
    assert ws(fake_list([k, k], fake=f, v=None, m=[base, base + 4 * 2 * 2048]), osa.OPTIM_ALGO_ADAMW, il()) > 0
    # not for Lion, LAMB, Adam-mini or 16-bit moments
    for algo in (osa.OPTIM_ALGO_LION, osa.OPTIM_ALGO_LAMB):
        expect_error(osa.OPTIM_EUNSUPPORTED, lambda: ws(fake_list([n], fake=f, v=None), algo, il()))
    expect_error(osa.OPTIM_EUNSUPPORTED, lambda: ws(
        fake_list([4096], fake=f, v=None, mini_kind=[osa.OPTIM_MINI_FULL_V], head_numel=[0]),
        osa.OPTIM_ALGO_ADAM_MINI, il()))
    expect_error(osa.OPTIM_EUNSUPPORTED, lambda: ws(
        fake_list([n], fake=f, v=None, scale_m=[f(4)], scale_v=[f(4)]), osa.OPTIM_ALGO_ADAMW, il(osa.OPTIM_F16)))


def test_tile_bounds(L):
    """Work units are a power of two of at least one group of 4 elements per
    lane (1024); blockwise rows need 2048."""
    f = Fake()
    for tile in (1024, 2048, 1 << 24):
        assert ws(fake_list([5000]), osa.OPTIM_ALGO_ADAMW, osa.optim_plan_opts(0, 0, 0, tile)) > 0
    for tile in (512, 3072, 1 << 25, -4):
        expect_error(osa.OPTIM_EINVAL, lambda: ws(
            fake_list([5000]), osa.OPTIM_ALGO_ADAMW, osa.optim_plan_opts(0, 0, 0, tile)))
    n = 1000
    kw = dict(m=None, v=None, qm=[f(n)], qv=[f(n)], absmax_m=[f(64)], absmax_v=[f(64)])
    assert ws(fake_list([n], fake=f, **kw), osa.OPTIM_ALGO_BLOCKWISE, osa.optim_plan_opts(8, 256, 0, 2048)) > 0
    expect_error(osa.OPTIM_EINVAL, lambda: ws(
        fake_list([n], fake=f, **kw), osa.OPTIM_ALGO_BLOCKWISE, osa.optim_plan_opts(8, 256, 0, 1024)))


def test_scaler_and_norm_validation_without_device(L):
    """Argument errors come back before any device work."""
    a = 1 << 40
    expect_error(osa.OPTIM_EINVAL, lambda: osa.optim_scaler_update(None, None, a, a, 2.0, 0.5, 10, 0))
    expect_error(osa.OPTIM_EINVAL, lambda: osa.optim_scaler_update(a, None, a, a, 1.0, 0.5, 10, 0))
    expect_error(osa.OPTIM_EINVAL, lambda: osa.optim_scaler_update(a, None, a, a, 2.0, 1.0, 10, 0))
    expect_error(osa.OPTIM_EINVAL, lambda: osa.optim_scaler_update(a, None, a, a, 2.0, 0.5, 0, 0))
    expect_error(osa.OPTIM_EALIGN, lambda: osa.optim_scaler_update(a + 2, None, a, a, 2.0, 0.5, 10, 0))
    expect_error(osa.OPTIM_EINVAL, lambda: osa.optim_grad_norm(None, None, 1.0, a, None, a, 0))


def test_blockwise_ademamix_validation(L):
    f = Fake()
    n = 1000
    kw = dict(m=None, v=None, qm=[f(n)], qv=[f(n)], absmax_m=[f(64)], absmax_v=[f(64)])
    opts = osa.optim_plan_opts(8, 256, 0, 0)
    expect_error(osa.OPTIM_EINVAL, lambda: ws(fake_list([n], fake=f, **kw), osa.OPTIM_ALGO_BLOCKWISE_ADEMAMIX, opts))
    full = dict(kw, qm2=[f(n)], absmax_m2=[f(64)])
    assert ws(fake_list([n], fake=f, **full), osa.OPTIM_ALGO_BLOCKWISE_ADEMAMIX, opts) > 0
    # m2's codes overlapping m's
    bad = dict(kw, qm2=[kw["qm"][0] + 8], absmax_m2=[f(64)])
    expect_error(osa.OPTIM_EINVAL, lambda: ws(fake_list([n], fake=f, **bad), osa.OPTIM_ALGO_BLOCKWISE_ADEMAMIX, opts))
    expect_error(osa.OPTIM_EINVAL, lambda: ws(fake_list([n], fake=f, **full), 5, opts))


def test_lion_and_lamb_validation(L):
    f = Fake()
    n = 1000
    lion = dict(m=[f(4 * n)], v=None)
    assert ws(fake_list([n], fake=f, **lion), osa.OPTIM_ALGO_LION) > 0
    expect_error(osa.OPTIM_EINVAL, lambda: ws(fake_list([n], fake=f, m=None, v=None), osa.OPTIM_ALGO_LION))
    assert ws(fake_list([n], fake=f), osa.OPTIM_ALGO_LAMB) > 0
    expect_error(osa.OPTIM_EINVAL, lambda: ws(fake_list([n], fake=f, v=None), osa.OPTIM_ALGO_LAMB))
    expect_error(osa.OPTIM_EINVAL, lambda: ws(fake_list([n], fake=f), 7))
    # LAMB keeps two partial sums per unit: its workspace exceeds AdamW's
    assert ws(fake_list([1 << 20], fake=f), osa.OPTIM_ALGO_LAMB) > ws(fake_list([1 << 20], fake=f),
                                                                         osa.OPTIM_ALGO_ADAMW)


def test_master_weight_validation(L):
    f = Fake()
    n = 1000
    mw = dict(params=[f(2 * n)], master=[f(4 * n)])
    for dt in (osa.OPTIM_BF16, osa.OPTIM_F16):
        for algo in (osa.OPTIM_ALGO_ADAMW, osa.OPTIM_ALGO_ADEMAMIX):
            extra = dict(m2=[f(4 * n)]) if algo == osa.OPTIM_ALGO_ADEMAMIX else {}
            assert ws(fake_list([n], fake=f, param_dtype=dt, **mw, **extra), algo) > 0
    expect_error(osa.OPTIM_EINVAL, lambda: ws(fake_list([n], fake=f, master=[f(4 * n)]), osa.OPTIM_ALGO_ADAMW))
    expect_error(osa.OPTIM_EUNSUPPORTED, lambda: ws(
        fake_list([n], fake=f, params=[f(2 * n)], param_dtype=osa.OPTIM_F16), osa.OPTIM_ALGO_ADAMW))
    expect_error(osa.OPTIM_EUNSUPPORTED, lambda: ws(
        fake_list([n], fake=f, param_dtype=osa.OPTIM_BF16, v=None, **mw), osa.OPTIM_ALGO_LION))
    expect_error(osa.OPTIM_EINVAL, lambda: ws(
        fake_list([n], fake=f, param_dtype=osa.OPTIM_BF16, remainders=[f(2 * n)], **mw), osa.OPTIM_ALGO_ADAMW))
    p = f(4 * n)
    expect_error(osa.OPTIM_EINVAL, lambda: ws(  # master overlapping the model copy
        fake_list([n], fake=f, params=[p], master=[p + 16], param_dtype=osa.OPTIM_BF16), osa.OPTIM_ALGO_ADAMW))
    expect_error(osa.OPTIM_EDTYPE, lambda: ws(fake_list([n], fake=f, param_dtype=3), osa.OPTIM_ALGO_ADAMW))


def test_scaled_state_validation(L):
    f = Fake()
    n = 1000
    opts = lambda sdt: osa.optim_plan_opts(0, 0, 0, 0, sdt)
    s16 = lambda **kw: fake_list([n], fake=f, **{**dict(m=[f(2 * n)], v=[f(2 * n)], scale_m=[f(4)],
                                                    scale_v=[f(4)]), **kw})
    for sdt in (osa.OPTIM_F16, osa.OPTIM_BF16):
        assert ws(s16(), osa.OPTIM_ALGO_ADAMW, opts(sdt)) > 0
        assert ws(s16(param_dtype=osa.OPTIM_BF16, params=[f(2 * n)], remainders=[f(2 * n)]),
                  osa.OPTIM_ALGO_ADAMW, opts(sdt)) > 0
        # a 16-bit moment needs 2-byte alignment only
        assert ws(s16(m=[f(2 * n, misalign=2)]), osa.OPTIM_ALGO_ADAMW, opts(sdt)) > 0
        expect_error(osa.OPTIM_EALIGN, lambda: ws(s16(m=[f(2 * n, misalign=1)]), osa.OPTIM_ALGO_ADAMW, opts(sdt)))
        expect_error(osa.OPTIM_EALIGN, lambda: ws(s16(scale_v=[f(4, misalign=2)]), osa.OPTIM_ALGO_ADAMW,
                                                  opts(sdt)))
        expect_error(osa.OPTIM_EINVAL, lambda: ws(  # the scales are required
            fake_list([n], fake=f, m=[f(2 * n)], v=[f(2 * n)]), osa.OPTIM_ALGO_ADAMW, opts(sdt)))
        expect_error(osa.OPTIM_EUNSUPPORTED, lambda: ws(
            s16(m2=[f(4 * n)]), osa.OPTIM_ALGO_ADEMAMIX, opts(sdt)))
        expect_error(osa.OPTIM_EUNSUPPORTED, lambda: ws(
            s16(param_dtype=osa.OPTIM_BF16, params=[f(2 * n)], master=[f(4 * n)]), osa.OPTIM_ALGO_ADAMW, opts(sdt)))
        sm = f(4)
        expect_error(osa.OPTIM_EINVAL, lambda: ws(  # a scale shared by two tensors
            fake_list([n, n], fake=f, m=[f(2 * n), f(2 * n)], v=[f(2 * n), f(2 * n)], scale_m=[sm, sm],
                      scale_v=[f(4), f(4)]), osa.OPTIM_ALGO_ADAMW, opts(sdt)))
    expect_error(osa.OPTIM_EDTYPE, lambda: ws(s16(), osa.OPTIM_ALGO_ADAMW, opts(3)))
    # the 16-bit moments halve the state footprint, the scales are per tensor
    assert ws(s16(), osa.OPTIM_ALGO_ADAMW, opts(osa.OPTIM_F16)) >= ws(fake_list([n]), osa.OPTIM_ALGO_ADAMW)


def test_null_plan_is_rejected_without_device(L):
    expect_error(osa.OPTIM_EINVAL, lambda: osa.optim_step_adamw(
        None, osa.optim_adamw_hp(0.9, 0.999, 1e-8), 1 << 40, None, None, 1 << 41, 0))
    expect_error(osa.OPTIM_EINVAL, lambda: osa.optim_plan_set_schedule(None, 1, 1e-3, 0.0, 10, 1 << 40))
    expect_error(osa.OPTIM_EINVAL, lambda: osa.optim_remainder_split(0, 0, 0, -1, 0))


def test_product_partition_by_name():
    names = ["tok_embeddings.weight", "layers.0.attention.wq.weight", "layers.0.attention.wk.weight",
             "layers.0.attention.wv.weight", "layers.0.attention_norm.weight", "output.weight"]
    numels = [32 * 64, 64 * 64, 64 * 64, 64 * 64, 64, 32 * 64]
    kinds, heads, wds = osa.adam_mini_partition(names, numels, dim=64, n_heads=4, weight_decay=0.1)
    assert kinds == [0, 1, 1, 2, 2, 0]
    assert heads[1] == heads[2] == 1024 and heads[3] == 4096 and heads[4] == 64
    assert wds == [0.1, 0.1, 0.1, 0.1, 0.0, 0.1]
    with pytest.raises(ValueError):
        osa.adam_mini_partition(names, numels, dim=10, n_heads=3, weight_decay=0.1)


def test_missing_library_raises_without_fallback():
    """With the built library absent every entry point raises: there is no
    CPU or torch fallback (checked in a fresh interpreter)."""
    import subprocess
    import sys
    code = ("import optimizer_step_adamw_amd as osa\n"
            "osa.LIB_PATH = '/nonexistent/liboptim_step.so'\n"
            "osa._lib = None\n"
            "try:\n"
            "    osa.optim_plan_workspace_size(osa.TensorList([], [], weight_decay=[], numel=[]), osa.OPTIM_ALGO_ADAMW)\n"
            "except RuntimeError as e:\n"
            "    print('raised:', 'no fallback' in str(e))\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert "raised: True" in out.stdout, (out.stdout, out.stderr)


def test_static_plan_refuses_oversize_and_invalid_lists_on_the_host(L):
    """optim_plan_create_static validates and sizes the plan before it
    touches any device: an invalid list and a plan larger than the static
    workspace are refused with no device call (fake pointers, no GPU)."""
    big = [1 << 34]  # Adam-mini SCALAR: one partial sum per 4096-element unit
    tl = fake_list(big, mini_kind=[osa.OPTIM_MINI_SCALAR], head_numel=big)
    need = ws(tl, osa.OPTIM_ALGO_ADAM_MINI)
    assert need > osa.OPTIM_STATIC_WORKSPACE_BYTES
    with pytest.raises(osa.OptimError) as ei:
        osa.optim_plan_create_static(tl, osa.OPTIM_ALGO_ADAM_MINI, None, stream=0)
    assert ei.value.code == osa.OPTIM_EWORKSPACE
    assert str(need) in str(ei.value) and str(osa.OPTIM_STATIC_WORKSPACE_BYTES) in str(ei.value)
    expect_error(osa.OPTIM_EINVAL, lambda: osa.optim_plan_create_static(
        fake_list([4096], weight_decay=[-1.0]), osa.OPTIM_ALGO_ADAMW, None, stream=0))


def test_static_workspace_holds_the_7b_adam_mini_plan(L):
    """The static workspace is sized for the largest list of the benchmark
    workloads: the Llama-7B-shaped Adam-mini plan (one partial sum per
    4096-element unit) fits it."""
    import synth
    wl = synth.c5_adam_mini_7b()
    names = [t.name for t in wl.tensors]
    sizes = [t.numel for t in wl.tensors]
    kinds, heads, wds = osa.adam_mini_partition(names, sizes, dim=4096, n_heads=32, weight_decay=0.1)
    fake = Fake()
    vlen = [n if k == osa.OPTIM_MINI_FULL_V else n // h for n, k, h in zip(sizes, kinds, heads)]
    tl = osa.TensorList([fake(4 * n) for n in sizes], [fake(4 * n) for n in sizes],
                        m=[fake(4 * n) for n in sizes], v=[fake(4 * k) for k in vlen], weight_decay=wds,
                        mini_kind=kinds, head_numel=heads, numel=sizes)
    need = ws(tl, osa.OPTIM_ALGO_ADAM_MINI)
    assert 8 << 20 < need <= osa.OPTIM_STATIC_WORKSPACE_BYTES, need


def test_binding_refuses_host_and_strided_tensors():
    """The kernels walk numel() elements from each tensor's address, so the
    binding refuses a tensor that is not on the GPU, or not contiguous,
    before the library sees it."""
    import torch
    host = torch.zeros(16)
    with pytest.raises(ValueError, match="GPU tensor"):
        osa.TensorList([host], [host], m=[host], v=[host], weight_decay=[0.0])
    strided = torch.zeros(4, 4).t()

    class Cuda:  # a stand-in that claims the GPU but is a transposed view
        is_cuda = True

        def __init__(self, t):
            self.t = t
            self.shape = t.shape

        def is_contiguous(self):
            return self.t.is_contiguous()

        def stride(self):
            return self.t.stride()

        def data_ptr(self):
            return self.t.data_ptr()

    with pytest.raises(ValueError, match="contiguous"):
        osa.optim_step_adamw(None, osa.optim_adamw_hp(0.9, 0.999, 1e-8), Cuda(strided), None, None, None)


def test_trace_calls_refuse_bad_arguments_on_the_host(L):
    """The kernel-trace entry points validate before touching a device."""
    import ctypes
    count, dropped = ctypes.c_int32(-1), ctypes.c_int64(-1)
    recs = (osa.optim_kernel_time * 4)()
    assert L.optim_plan_trace(None, 16) == osa.OPTIM_EINVAL
    assert b"plan" in L.optim_last_error()
    assert L.optim_plan_trace_read(None, recs, 4, ctypes.byref(count), ctypes.byref(dropped)) == osa.OPTIM_EINVAL
    assert count.value == -1  # nothing written on an error
    assert L.optim_plan_destroy(None) == osa.OPTIM_OK  # destroying NULL is a no-op
