"""GPU parity of the exact-statistic quantiser (brq_quantize_lsq_exact)
against the oracle, bit for bit: layer-like data, values spanning the whole
binary32 exponent range (carries through every container), container sums
past 2^64, specials, per-row groups, the layer's full activation and
gradient shapes, and order independence.
"""
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


def wide_range(shape, seed, lo=1, hi=254):
    """fp32 values with random signs, fractions and biased exponents in
    [lo, hi], plus zeros and subnormals."""
    rng = np.random.default_rng(seed)
    n = int(np.prod(shape))
    e = rng.integers(lo, hi + 1, size=n).astype(np.uint32)
    u = (e << 23) | rng.integers(0, 1 << 23, size=n).astype(np.uint32)
    u |= rng.integers(0, 2, size=n).astype(np.uint32) << 31
    z = rng.random(n) < 0.05
    u[z] = rng.integers(0, 1 << 23, size=int(z.sum())).astype(np.uint32)
    return u.view(np.float32).reshape(shape)


def check(x, col=None, per_row=False, want_t=None, name=""):
    if want_t is None:
        want_t = x.shape[0] % 16 == 0 and x.shape[1] % 16 == 0
    q, qt, s, amax, fl = orc.quantize_lsq(x, per_row=per_row, col_mul=col, want_t=want_t,
                                          exact=True)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    gq, gqt, gs, gamax = brq.quantize_lsq(to_dev(x), per_row=per_row,
                                          col_mul=None if col is None else to_dev(col),
                                          want_t=want_t, flags=flags, exact=True)
    assert_bitwise(gs, s, name + " scale")
    assert_bitwise(gq, q, name + " q")
    if fl == 0:
        assert_bitwise(gamax, amax, name + " amax")
    if want_t:
        assert_bitwise(gqt, qt, name + " q_t")
    assert int(flags.item()) == fl, name
    return gs


CASES = [
    ((64, 256), False, None),
    ((100, 264), True, None),
    ((257, 520), False, None),
    ((300, 512), True, "cm"),
    ((64, 256), False, "cm"),
    ((1024, 2048), True, None),     # 2^21 values: many work-groups per partial level
    ((1536, 1000), False, "cm"),
]


@pytest.mark.parametrize("shape,bf16,cm", CASES)
def test_exact_per_tensor(shape, bf16, cm):
    say("exact_per_tensor", shape, bf16, cm)
    x = syn.normal(shape, 1.0, tag=211, bf16=bf16)
    col = syn.normal((shape[1],), 0.01, mean=0.02, tag=212) if cm else None
    check(x, col, name=f"{shape}")


@pytest.mark.parametrize("seed,lo,hi", [(1, 1, 254), (2, 100, 160), (3, 1, 40), (4, 200, 254),
                                        (5, 120, 136)])
def test_exact_wide_range(seed, lo, hi):
    """Every digit and carry of the fixed-point sum, per-tensor and per-row;
    the (4) case overflows to +inf and raises the flag."""
    say("exact_wide_range", seed, lo, hi)
    x = wide_range((96, 1024), seed, lo, hi)
    check(x, name=f"wide {seed}")
    check(x[:, :512].copy(), per_row=True, name=f"wide rows {seed}")


def test_exact_container_past_2_64():
    """2^26 equal values of (2^24 - 1) * 2^15 units each: the digit's total
    needs 65 bits.  S = n * v rounded once, checked against its closed
    form too."""
    say("exact_container_past_2_64")
    u = np.uint32((128 << 23) | 0x7fffff)  # e - 1 = 127 = 15 (mod 16): the widest term
    x = np.full((16384, 4096), u, np.uint32).view(np.float32)
    gs = check(x, want_t=False, name="2^26 equal")
    v = float(x[0, 0])
    S = np.float32(float(v) * 2.0 ** 26)  # n a power of two: exact scaling
    want_s, _ = orc.lsq_scale(S, x.size)
    assert to_np(gs)[0] == want_s


def test_exact_specials_and_edges():
    say("exact_specials")
    z = np.zeros((32, 64), np.float32)
    check(z, name="zeros")
    check(z, per_row=True, name="zero rows")
    e = torch.empty((0, 64), dtype=torch.float32, device=DEV)
    _, _, gs, _ = brq.quantize_lsq(e, exact=True)
    assert float(gs.item()) == 0.0
    for val in (np.inf, -np.inf, np.nan):
        bad = np.ones((16, 64), np.float32)
        bad[3, 5] = val
        for per_row in (False, True):
            flags = torch.zeros(1, dtype=torch.int32, device=DEV)
            brq.quantize_lsq(to_dev(bad), per_row=per_row, flags=flags, exact=True)
            assert int(flags.item()) == brq.FLAG_NONFINITE, (val, per_row)
    sub = np.full((16, 64), 1.0, np.float32)
    sub[0, :16] = np.float32(1e-40)
    sub[1, :16] = -np.float32(1e-40)
    check(sub, name="subnormal inputs")
    # subnormals alone (they would sum to a normal): S = 0, step 0
    only = np.full((16, 64), np.float32(1e-39), np.float32)
    check(only, name="subnormal only")
    # the smallest normals: the sum's last bits sit at the bottom of the range
    tiny = np.full((16, 64), np.float32(2.0 ** -126), np.float32)
    tiny[::2, ::3] = np.float32(2.0 ** -126 * (1 + 2.0 ** -23))
    check(tiny, name="smallest normals")


def test_exact_differs_from_tree_where_the_tree_rounds():
    """A large value and many small ones: the tree loses the small ones,
    the exact sum keeps them; the GPU follows the exact definition."""
    say("exact_vs_tree")
    x = np.full((64, 256), np.float32(2.0 ** -24), np.float32)
    x[0, 0] = 1.0
    s_exact = orc.quantize_lsq(x, exact=True)[2][0]
    s_tree = orc.quantize_lsq(x)[2][0]
    assert s_exact != s_tree
    gs = check(x, name="big+small")
    assert to_np(gs)[0] == s_exact


@pytest.mark.parametrize("shape,bf16", [((256, 256), False), ((3072, 2048), True),
                                        ((48, 8192), True), ((16, 264), True), ((5, 16384), True),
                                        ((33, 100), False), ((40, 16384), False)])
def test_exact_per_row(shape, bf16):
    say("exact_per_row", shape, bf16)
    w = syn.normal(shape, 0.02, tag=213, bf16=bf16)
    check(w, per_row=True, name=f"rows {shape}")


def test_exact_order_free():
    """Any permutation of the values gives the same step size."""
    say("exact_order_free")
    x = wide_range((512, 512), 9, 90, 170)
    _, _, s0, _ = brq.quantize_lsq(to_dev(x), exact=True)
    rng = np.random.default_rng(10)
    for _ in range(3):
        p = x.reshape(-1)[rng.permutation(x.size)].reshape(x.shape)
        _, _, s1, _ = brq.quantize_lsq(to_dev(p), exact=True)
        assert_bitwise(s1, to_np(s0), "permuted scale")


@pytest.mark.parametrize("which", ["x_attn", "x_down", "dy_gate"])
def test_exact_layer_shapes(which):
    """The layer's full activation inputs (32768 x 2048 and 32768 x 8192
    bf16) and one gradient with its per-channel weight steps folded in."""
    say("exact_layer_shapes", which)
    col = None
    if which.startswith("x_"):
        x = syn.layer_input(which)
    else:
        i = [n for n, *_ in syn.LAYER_LINEARS].index("gate")
        x = syn.layer_dy(i)
        w = syn.layer_weight(i)
        col = orc.quantize_lsq(w, per_row=True, exact=True)[2]
    check(x, col, want_t=False, name=which)
