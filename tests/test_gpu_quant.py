"""GPU checks of the blockwise quantizer through optim_quantize_blockwise /
optim_dequantize_blockwise, which run the same device code as the 8-bit /
4-bit step: exhaustive over every fp32 magnitude in [0, 1] against the
threshold rule, and bit-exact round trips against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle as orc
import optimizer_step_adamw_amd as osa
from gpu_support import DEV, QuantState, say
from synth import host_normal

pytestmark = pytest.mark.gpu


def _plan(bits, block):
    qs = QuantState([torch.zeros(block, device=DEV)], bits, block)
    return qs, osa.Plan(qs.tensor_list([0.0]), osa.OPTIM_ALGO_BLOCKWISE, bits=bits, block=block)


def _unpack(codes_dev, bits, n):
    c = codes_dev.cpu().numpy()
    return orc.unpack_nibbles(c, n) if bits == 4 else c[:n]


@pytest.mark.parametrize("bits,block,signed", [(8, 256, True), (8, 256, False), (4, 128, True),
                                               (4, 128, False)])
def test_quantizer_exhaustive_unit_interval(bits, block, signed):
    """Every fp32 a in [0, 1], placed in blocks whose absmax is exactly 1.0 (so
    the normalisation is exact): the code index is the largest j with
    T[j] <= a, T being the oracle's thresholds (torch.searchsorted referee)."""
    mb = bits - 1 if signed else bits
    T = torch.from_numpy(orc.thresholds(orc.dynamic_map(mb))[1:].copy()).to(DEV)
    qs, plan = _plan(bits, block)
    per = block - 1
    top = 0x3F800000  # bit pattern of 1.0
    CH = per * (1 << 18)
    mask = (1 << bits) - 1
    for s in range(0, top + 1, CH):
        k = min(CH, top + 1 - s)
        a = torch.arange(s, s + k, dtype=torch.int32, device=DEV).view(torch.float32)
        nb = (k + per - 1) // per
        flat = torch.zeros(nb * per, dtype=torch.float32, device=DEV)
        flat[:k] = a
        x = torch.ones(nb, block, dtype=torch.float32, device=DEV)
        x[:, :per] = flat.view(nb, per)
        del flat
        n = nb * block
        codes = torch.empty((n * bits + 7) // 8, dtype=torch.uint8, device=DEV)
        absmax = torch.empty(nb, dtype=torch.float32, device=DEV)
        osa.optim_quantize_blockwise(plan.handle, signed, x, n, codes, absmax)
        if bits == 8:
            got = codes.to(torch.int64)
        else:
            got = torch.stack([codes & 15, codes >> 4], 1).reshape(-1).to(torch.int64)
        got = got.view(nb, block)[:, :per].reshape(-1)[:k] & mask
        want = torch.searchsorted(T, a, right=True)
        bad = (got != want).nonzero()
        assert bad.numel() == 0, (s, a[bad[:5, 0]].tolist(), got[bad[:5, 0]].tolist(), want[bad[:5, 0]].tolist())
        assert torch.all(absmax == 1.0)
    say(f"{bits}-bit {'signed' if signed else 'unsigned'}: all fp32 in [0,1] agree with the threshold rule")


@pytest.mark.parametrize("bits,block", [(8, 256), (8, 64), (4, 128), (4, 512)])
def test_quantize_roundtrip_matches_oracle(bits, block):
    for n in (1, 77, block, 3 * block + 5, 40000 + 3):
        x = host_normal(n, 1e-3, 950, bits, block, n)
        x[::7] = 0.0
        qs, plan = _plan(bits, block)
        for signed in (True, False):
            xs = x if signed else np.abs(x)
            mb = bits - 1 if signed else bits
            codes = torch.empty((n * bits + 7) // 8, dtype=torch.uint8, device=DEV)
            absmax = torch.empty((n + block - 1) // block, dtype=torch.float32, device=DEV)
            xd = torch.from_numpy(xs).to(DEV)
            osa.optim_quantize_blockwise(plan.handle, signed, xd, n, codes, absmax)
            oc, oa = orc.quantize(xs, block, mb, signed)
            assert np.array_equal(_unpack(codes, bits, n), oc), (bits, block, n, signed)
            if bits == 4:
                assert np.array_equal(codes.cpu().numpy(), orc.pack_nibbles(oc))
            assert np.array_equal(absmax.cpu().numpy().view(np.uint32), oa.view(np.uint32))
            back = torch.empty(n, dtype=torch.float32, device=DEV)
            osa.optim_dequantize_blockwise(plan.handle, signed, codes, absmax, n, back)
            ob = orc.dequantize(oc, oa, block, mb, signed)
            assert np.array_equal(back.cpu().numpy().view(np.uint32), ob.view(np.uint32))
