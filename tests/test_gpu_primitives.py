"""Every binary32 bit pattern through the device's division, square root and
bf16 rounding -- the helpers every kernel uses (brq_fp32_primitive) --
against the host's correctly rounded operations with the same flushes
(oracle.prim_sweep): the report's §2 "The same operation compiles to
different instructions" and §2.1 Table 1.  2^32 inputs per primitive, in
16 slices of 2^28; results must agree bit for bit, except that a NaN
result may carry any NaN payload."""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SLICE = 1 << 28


@pytest.fixture(scope="module")
def brq():
    import bitwise_reproducible_int8_amd as m
    m.lib()
    return m


def _nan32(u):
    return ((u & 0x7F800000) == 0x7F800000) & ((u & 0x007FFFFF) != 0)


def _nan16(u):
    return ((u & 0x7F80) == 0x7F80) & ((u & 0x007F) != 0)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("prim,name", [(0, "sqrt"), (1, "rcp"), (2, "rsqrt"), (3, "bf16_cvt"),
                                       (4, "bf16_int")])
def test_primitive_exhaustive(brq, orc, prim, name):
    host_prim = prim if prim < 3 else 3
    isnan = _nan32 if prim < 3 else _nan16
    out = torch.empty(SLICE, dtype=torch.int32, device="cuda:0")
    host = np.empty(SLICE, np.uint32)
    for k in range(1 << 32 >> 28):
        first = k * SLICE
        print(f"primitive {name} slice {k}", file=sys.stderr, flush=True)
        brq.fp32_primitive(prim, first, SLICE, out=out)
        g = out.cpu().numpy().view(np.uint32)
        orc.prim_sweep(host_prim, first, SLICE, out=host)
        bad = np.nonzero(g != host)[0]
        if bad.size:
            both_nan = isnan(g[bad]) & isnan(host[bad])
            real = bad[~both_nan]
            assert real.size == 0, (
                f"{name}: {real.size} inputs differ in slice {k}; first input "
                f"{first + int(real[0]):#010x}: device {int(g[real[0]]):#x} host "
                f"{int(host[real[0]]):#x}")
