"""GPU parity of the optimizer step (AdamW, global-norm clip, spike skip)
through the C ABI against the CPU oracle, bit for bit: the device decision
over a norm sequence, the elementwise update over ragged sizes, both
parameter and gradient dtypes, clipped and unclipped, with and without
weight decay, and a skipped step."""
import sys

import numpy as np
import pytest
import torch

import brq_synth as syn
import oracle as orc
from tests.gpu_util import DEV, assert_bitwise, to_dev, to_np

pytestmark = pytest.mark.gpu

brq = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global brq
    import bitwise_reproducible_int8_amd as m
    m.lib()
    brq = m
    yield


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def test_adamw_decide_sequence():
    norms = [0.3, 1.0, 1.0000001, 2.5, 5.0, 5.78, 0.4, 0.4, 0.4, 0.4, 0.4, 0.4, 6.88, 0.2, 7.0,
             0.2, 0.2, 0.2, 0.2, 0.2, float("inf"), 0.2, float("nan"), 0.2, 0.2, 0.2, 0.2, 0.2,
             0.0, 1e-30]
    say("adamw_decide", len(norms))
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    fl = torch.zeros(1, dtype=torch.int32, device=DEV)
    ctl = torch.empty(2, dtype=torch.float32, device=DEV)
    ost = 0
    for n in norms:
        nt = torch.tensor([n], dtype=torch.float32, device=DEV)
        fl.zero_()
        brq.adamw_decide(nt, st, out=ctl, flags=fl)
        ap, cl, ost, ofl = orc.adamw_decide(np.float32(n), ost)
        assert_bitwise(ctl, np.array([ap, cl], np.float32), f"ctl at norm {n}")
        assert int(st.item()) == ost, n
        assert int(fl.item()) == ofl, n


ADAMW_CASES = [
    # n, param bf16, grad bf16, step t, weight decay, norm scale (clip when > 1)
    (1, True, False, 1, 0.1, 1.0),
    (7, True, False, 3, 0.1, 1.0),
    (8, False, False, 2, 0.0, 1.0),
    (1000, True, True, 5, 0.1, 1.0),
    (4099, True, False, 7, 0.1, 3.5),
    (4099, False, True, 1, 0.1, 2.0),
    (65539, True, False, 12, 0.0, 1.0),
    (65536 + 8, True, False, 100, 0.1, 1.7),
]


@pytest.mark.parametrize("n,pb,gb,t,wd,clip_norm", ADAMW_CASES)
def test_adamw_step(n, pb, gb, t, wd, clip_norm):
    say("adamw_step", n, pb, gb, t, wd, clip_norm)
    p, g, m, v = syn.optimizer_group(n, grad_std=1e-3, param_bf16=pb, grad_bf16=gb, group=n % 7)
    lr = 3e-4
    bc = orc.adamw_bias_corrections(t)
    assert brq.adamw_bias_corrections(t) == (float(bc[0]), float(bc[1]))
    # the decision as the oracle makes it for this norm
    ap, cl, _, _ = orc.adamw_decide(np.float32(clip_norm), 0)
    want_p, want_m, want_v = orc.adamw_step(p, g, m, v, lr, bc[0], bc[1], ap, cl, wd=wd)
    dp, dg, dm, dv = to_dev(p), to_dev(g), to_dev(m), to_dev(v)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    ctl = brq.adamw_decide(torch.tensor([clip_norm], dtype=torch.float32, device=DEV), st)
    assert_bitwise(ctl, np.array([ap, cl], np.float32), "ctl")
    brq.adamw_step(dp, dg, dm, dv, ctl, lr, bc, weight_decay=wd)
    assert_bitwise(dp, want_p, f"param n={n}")
    assert_bitwise(dm, want_m, f"m n={n}")
    assert_bitwise(dv, want_v, f"v n={n}")


def test_adamw_skipped_step_writes_nothing():
    n = 4099
    p, g, m, v = syn.optimizer_group(n, grad_std=1e-3, group=3)
    dp, dg, dm, dv = to_dev(p), to_dev(g), to_dev(m), to_dev(v)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    ctl = brq.adamw_decide(torch.tensor([9.0], dtype=torch.float32, device=DEV), st)
    assert int(st.item()) == 4
    brq.adamw_step(dp, dg, dm, dv, ctl, 1e-3, brq.adamw_bias_corrections(1))
    for a, b, nm in ((dp, p, "p"), (dm, m, "m"), (dv, v, "v")):
        assert_bitwise(a, b, nm)


def test_adamw_two_steps_carry_state():
    """Two consecutive steps on the same buffers (moments carried over,
    parameter rounded to bf16 in between) equal two oracle steps."""
    n = 10000
    p, g, m, v = syn.optimizer_group(n, grad_std=1e-3, group=5)
    g2 = syn.normal((n,), 2e-3, tag=syn.tag_for(47, syn.TAG_DY))
    dp, dm, dv = to_dev(p), to_dev(m), to_dev(v)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    op, om, ov = p, m, v
    for t, grad, norm in ((1, g, 0.8), (2, g2, 1.3)):
        bc = orc.adamw_bias_corrections(t)
        ap, cl, _, _ = orc.adamw_decide(np.float32(norm), 0)
        op, om, ov = orc.adamw_step(op, grad, om, ov, 1e-3, bc[0], bc[1], ap, cl)
        ctl = brq.adamw_decide(torch.tensor([norm], dtype=torch.float32, device=DEV), st)
        brq.adamw_step(dp, to_dev(grad), dm, dv, ctl, 1e-3, brq.adamw_bias_corrections(t))
    assert_bitwise(dp, op, "p")
    assert_bitwise(dm, om, "m")
    assert_bitwise(dv, ov, "v")


def test_adamw_argument_errors():
    n = 64
    p = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    g = torch.zeros(n, dtype=torch.float32, device=DEV)
    m = torch.zeros(n, dtype=torch.float32, device=DEV)
    ctl = torch.tensor([1.0, 1.0], device=DEV)
    with pytest.raises(brq.BrqError):
        brq.adamw_step(p, g, m, torch.zeros(n - 1, device=DEV), ctl, 1e-3, (0.1, 0.05))
    with pytest.raises(brq.BrqError):
        brq.adamw_step(p, g, m.to(torch.bfloat16), m, ctl, 1e-3, (0.1, 0.05))
    with pytest.raises(brq.BrqError):
        brq.adamw_bias_corrections(0)
