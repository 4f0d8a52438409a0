"""The allocation-free quantiser entry point, brq_quantize_lsq_static, called
through the C ABI: its outputs equal brq_quantize_lsq's (with a caller
workspace) and the oracle's, bit for bit, on two calls in a row, the second
with a smaller input, so the shared static scratch is reused with stale
contents from the first call."""
import ctypes as C

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def brq():
    import bitwise_reproducible_int8_amd as m
    m.lib()
    return m


def _static(brq, x, per_row, col_mul, want_t, tune=None):
    from tests.gpu_util import to_dev
    X = to_dev(x)
    rows, cols = X.shape
    ns = rows if per_row else 1
    dev = X.device
    q = torch.empty((rows, cols), dtype=torch.int8, device=dev)
    qt = torch.empty((cols, rows), dtype=torch.int8, device=dev) if want_t else None
    scale = torch.empty(ns, dtype=torch.float32, device=dev)
    amax = torch.empty(ns, dtype=torch.float32, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    cm = None if col_mul is None else to_dev(col_mul)
    tn = None if tune is None else C.byref(brq.Tune(**tune))
    st = brq.lib().brq_quantize_lsq_static(
        X.data_ptr(), brq._fp_code(X), rows, cols, brq.PER_ROW if per_row else brq.PER_TENSOR,
        None if cm is None else cm.data_ptr(), q.data_ptr(), None if qt is None else qt.data_ptr(),
        scale.data_ptr(), amax.data_ptr(), flags.data_ptr(), tn,
        torch.cuda.current_stream().cuda_stream)
    assert st == 0, brq.lib().brq_status_string(st)
    torch.cuda.synchronize()
    return q, qt, scale, amax, flags


CASES = [
    # first call large, second smaller (stale scratch from the first)
    [((2048, 4096), True, False, "cm"), ((96, 264), True, False, None)],
    [((1024, 2048), False, False, None), ((64, 256), False, False, "cm")],
    [((3072, 2048), True, True, None), ((16, 264), True, True, None)],  # per row
]


@pytest.mark.parametrize("calls", CASES, ids=["bf16-cm", "fp32", "per-row"])
def test_static_scratch_matches_workspace_entry_point(brq, orc, syn, calls):
    from tests.gpu_util import assert_bitwise, to_dev
    for k, (shape, bf16, per_row, cm) in enumerate(calls):
        x = syn.normal(shape, 1.0, tag=700 + k, bf16=bf16)
        col = syn.normal((shape[1],), 0.01, mean=0.02, tag=710 + k) if cm else None
        want_t = shape[0] % 16 == 0 and shape[1] % 16 == 0
        for tune in (None, {"chunk_log2": 10}):
            q, qt, s, a, fl = _static(brq, x, per_row, col, want_t, tune)
            wq, wqt, ws_, wa = brq.quantize_lsq(to_dev(x), per_row=per_row,
                                                col_mul=None if col is None else to_dev(col),
                                                want_t=want_t, tune=tune)
            torch.cuda.synchronize()
            tag = f"call {k} {shape} tune={tune}"
            assert_bitwise(q, wq.cpu().numpy(), f"q {tag}")
            assert_bitwise(s, ws_.cpu().numpy(), f"scale {tag}")
            assert_bitwise(a, wa.cpu().numpy(), f"amax {tag}")
            if want_t:
                assert_bitwise(qt, wqt.cpu().numpy(), f"q_t {tag}")
            oq, oqt, os_, oa, ofl = orc.quantize_lsq(x, per_row=per_row, col_mul=col,
                                                     want_t=want_t)
            assert_bitwise(q, oq, f"q vs oracle {tag}")
            assert_bitwise(s, os_, f"scale vs oracle {tag}")
            assert int(fl.item()) == ofl == 0


def test_static_scratch_rejects_oversize(brq):
    x = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda:0")
    q = torch.empty((64, 64), dtype=torch.int8, device="cuda:0")
    s = torch.empty(1, dtype=torch.float32, device="cuda:0")
    # declared far larger than the buffers: refused before any launch
    st = brq.lib().brq_quantize_lsq_static(x.data_ptr(), brq.BF16, 1 << 20, 1 << 14, brq.PER_TENSOR,
                                           None, q.data_ptr(), None, s.data_ptr(), None, None,
                                           None, torch.cuda.current_stream().cuda_stream)
    assert st == brq.E_SCRATCH
