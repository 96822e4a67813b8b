"""Device checks of the step library's numeric helpers (through the probe
library, which compiles the library's device header with its flags).

recip_rn, the blockwise quantizer's reciprocal of a block maximum: Markstein's
correction of the hardware reciprocal inside [2^-126, 2^126] must equal the
IEEE quotient 1/a bit for bit -- the quantizer's codes are specified with
r = fl32(1/A) -- and the IEEE division serves the rest.  Checked for every
positive fp32 input."""
import pytest
import torch

import probes
from gpu_support import DEV, say

pytestmark = pytest.mark.gpu


def test_recip_rn_equals_ieee_division_for_every_positive_float():
    print("case: recip_rn over all 2^32 fp32 patterns", flush=True)
    L = probes.lib()
    bad = torch.zeros(1, dtype=torch.int64, device=DEV)
    fast = torch.zeros(1, dtype=torch.int64, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    assert L.check_recip_rn(0, 256, bad.data_ptr(), fast.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    # the fast path covers exponents -126 .. 125 and the single value 2^126
    assert int(fast.item()) >= 252 << 23, int(fast.item())
    assert int(bad.item()) == 0, int(bad.item())
    say(f"recip_rn: {int(fast.item())} inputs on the fast path, none differs from 1/a")
