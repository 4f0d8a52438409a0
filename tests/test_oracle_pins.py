"""Pins of the CPU oracle against values fixed outside it.

Every check here compares the oracle with something it does not compute
itself: hand-derived vectors (tests/golden), exact rational arithmetic
(tests/_exact.py), numpy/scipy integer algebra, fp64 bounds, Python's
hashlib (FIPS 180-4) and mathematical invariants.
"""
import hashlib
import math
import os
import struct
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

from tests import _exact as X

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(x):
    return np.float32(x)


def _bits(f):
    return struct.unpack("<I", struct.pack("<f", float(f)))[0]


def bits(f):
    return struct.unpack("<I", struct.pack("<f", float(f)))[0]


# --------------------------------------------------------------------------
# arithmetic model: flush, bf16 widen / narrow
# --------------------------------------------------------------------------
def test_flush_directed(orc):
    tiny = X.bits_to_float(0x00000001)
    assert orc.flush(tiny) == 0.0 and math.copysign(1, orc.flush(tiny)) == 1
    assert orc.flush(-tiny) == 0.0 and math.copysign(1, orc.flush(-tiny)) == -1
    big_sub = X.bits_to_float(0x007FFFFF)
    assert orc.flush(big_sub) == 0.0
    fmin = X.bits_to_float(0x00800000)
    assert orc.flush(fmin) == fmin
    assert orc.flush(-fmin) == -fmin
    assert orc.flush(1.5) == 1.5


def test_bf16_widen_exhaustive(orc):
    h = np.arange(65536, dtype=np.uint32)
    want = (h << 16).astype(np.uint32)
    sub = ((h & 0x7F80) == 0)
    want[sub] &= 0x80000000
    L = orc.lib()
    got = np.array([bits(L.orc_bf16_to_f32(int(v))) for v in range(65536)], np.uint32)
    nan = ((h & 0x7F80) == 0x7F80) & ((h & 0x7F) != 0)
    assert np.array_equal(got[~nan], want[~nan])


def _bf16_rne_exact(f):
    """Nearest bf16 to a finite float32, ties to even, by exact comparison."""
    fr = Fraction(float(f))
    u = bits(f)
    lo = u & 0xFFFF0000
    hi = (lo + 0x10000) & 0xFFFFFFFF
    a, b = Fraction(X.bits_to_float(lo)), Fraction(X.bits_to_float(hi)) if (hi & 0x7F800000) != 0x7F800000 else None
    if b is None:  # next step is infinity: compare against the overflow midpoint
        return lo >> 16 if (u & 0xFFFF) < 0x8000 or ((u & 0xFFFF) == 0x8000 and ((lo >> 16) & 1) == 0) else hi >> 16
    da, db = abs(fr - a), abs(b - fr)
    if da < db or (da == db and ((lo >> 16) & 1) == 0):
        return lo >> 16
    return hi >> 16


def test_bf16_narrow_rne(orc):
    rng = np.random.default_rng(1)
    vals = list(rng.standard_normal(2000).astype(np.float32))
    # crafted ties: low half exactly 0x8000 with even and odd upper halves
    for up in (0x3F80, 0x3F81, 0xBF80, 0xBF81, 0x4000, 0x7F7F):
        vals.append(np.float32(X.bits_to_float((up << 16) | 0x8000)))
        vals.append(np.float32(X.bits_to_float((up << 16) | 0x7FFF)))
        vals.append(np.float32(X.bits_to_float((up << 16) | 0x8001)))
    for v in vals:
        assert orc.f32_to_bf16(float(v)) == _bf16_rne_exact(v), hex(bits(v))
    assert orc.f32_to_bf16(X.bits_to_float(0x3F808000)) == 0x3F80
    assert orc.f32_to_bf16(X.bits_to_float(0x3F818000)) == 0x3F82


# --------------------------------------------------------------------------
# LSQ constant
# --------------------------------------------------------------------------
def _golden_kv(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if "=" in line:
            k, v = line.split("=")
            out[k.strip()] = int(v.strip(), 16)
    return out


def _next_up(f):
    return np.nextafter(np.float32(f), np.float32(np.inf))


def _next_down(f):
    return np.nextafter(np.float32(f), np.float32(-np.inf))


def test_prim_sweep_host_correctly_rounded(orc):
    """The host side of the device primitive sweep: square root and
    reciprocal correctly rounded (checked in exact rationals), with the
    model's flushes, and bf16 rounding as the scalar routine."""
    rng = np.random.default_rng(17)
    pats = rng.integers(0, 2 ** 32, 6000, dtype=np.uint64).astype(np.uint32)
    edge = np.array([0, 1, 0x007FFFFF, 0x00800000, 0x00800001, 0x3F800000, 0x3F800001,
                     0x7F7FFFFF, 0x7F800000, 0x7FC00000, 0x80000000, 0x80800000, 0xFF800000,
                     0x1F800000, 0x7E800000, 0x7E7FFFFF, 0x00400000],
                    np.uint32)
    pats = np.concatenate([pats, edge])
    for p in pats:
        x = X.bits_to_float(int(p))
        xd = 0.0 if (int(p) & 0x7F800000) == 0 else x  # DAZ (sign is irrelevant below)
        sq = orc.prim_sweep(0, int(p), 1)[0]
        rc = orc.prim_sweep(1, int(p), 1)[0]
        r = X.bits_to_float(int(sq))
        if math.isnan(xd) or xd < 0:
            assert math.isnan(r)
        elif math.isinf(xd) or xd == 0:
            assert r == math.sqrt(xd)
        else:
            fx = Fraction(xd)
            assert Fraction(float(r)) > 0
            lo = (Fraction(float(_next_down(r))) + Fraction(float(r))) / 2
            hi = (Fraction(float(r)) + Fraction(float(_next_up(r)))) / 2
            assert lo * lo <= fx <= hi * hi, (hex(int(p)), r)
        q = X.bits_to_float(int(rc))
        if math.isnan(xd):
            assert math.isnan(q)
        elif math.isinf(xd):
            assert q == 0.0
        elif xd == 0:
            assert math.isinf(q)
        else:
            want = X.op(Fraction(1) / Fraction(xd))
            if want == 0:  # 1/x subnormal: flushed to a zero with x's sign
                assert q == 0.0 and math.copysign(1, q) == math.copysign(1, xd), hex(int(p))
            else:
                assert _bits(q) == X.float_to_bits(float(want)), (hex(int(p)), q, float(want))
        assert orc.prim_sweep(3, int(p), 1)[0] == orc.f32_to_bf16(x) or math.isnan(x)


def test_lsq_k2_constant(orc):
    g = _golden_kv("lsq_constants.txt")
    getcontext().prec = 100
    s = X.round_binary32(Fraction(Decimal(127).sqrt()))
    assert X.float_to_bits(float(s)) == g["sqrt127_bits"]
    r = X.round_binary32(1 / s)
    assert X.float_to_bits(float(r)) == g["recip_sqrt127_bits"]
    assert X.float_to_bits(float(2 * r)) == g["k2_bits"]
    assert bits(orc.lsq_k2()) == g["k2_bits"]


def test_reciprocal_multiply_differs_from_divide():
    """App. A.3: x/d and x*fl(1/d) disagree by up to one ulp when d is not a
    power of two; that is why every average multiplies by a reciprocal."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal(10000).astype(np.float32)
    d = np.float32(3.0)
    a = x / d
    b = x * (np.float32(1.0) / d)
    diff = np.abs(a.view(np.int32).astype(np.int64) - b.view(np.int32).astype(np.int64))
    assert diff.max() == 1 and (diff > 0).any()
    assert np.array_equal(x / np.float32(4.0), x * np.float32(0.25))


# --------------------------------------------------------------------------
# canonical tree
# --------------------------------------------------------------------------
def _golden_tree():
    rows = []
    for line in open(os.path.join(GOLDEN, "tree_vectors.txt")):
        if line.startswith("#") or not line.strip():
            continue
        exp, leaves, _ = line.split(";", 2)
        rows.append((float(exp), [float(t) for t in leaves.split()]))
    return rows


@pytest.mark.parametrize("recursive", [False, True])
def test_tree_golden(orc, recursive):
    for exp, leaves in _golden_tree():
        got = orc.tree_sum(np.array(leaves, np.float32), recursive=recursive)
        assert bits(got) == bits(exp), (leaves, got, exp)


def test_tree_powers_of_two_closed_form(orc):
    for j in range(0, 21, 4):
        for k in (0, 3, 20, 60):
            n = 1 << j
            leaves = np.full(n, np.float32(2.0 ** -k))
            assert orc.tree_sum(leaves) == np.float32(n * 2.0 ** -k)


def test_tree_two_codings_agree(orc):
    rng = np.random.default_rng(7)
    for n in list(range(1, 130)) + [4096 + 1664, 3 * 4096 + 1]:
        leaves = (rng.standard_normal(n) * np.exp(rng.uniform(-20, 20, n))).astype(np.float32)
        a = orc.tree_sum(leaves)
        b = orc.tree_sum(leaves, recursive=True)
        assert bits(a) == bits(b), n


def test_tree_matches_exact_rational_emulation(orc):
    """Each node is one binary32 RNE addition of its two children."""
    rng = np.random.default_rng(11)
    for n in (1, 2, 3, 5, 17, 33, 64, 100):
        leaves = (rng.standard_normal(n) * np.exp(rng.uniform(-8, 8, n))).astype(np.float32)
        level = [Fraction(float(v)) for v in leaves]
        while len(level) > 1:
            nxt = [X.op(level[2 * i] + level[2 * i + 1]) for i in range(len(level) // 2)]
            if len(level) % 2:
                nxt.append(level[-1])
            level = nxt
        assert float(orc.tree_sum(leaves)) == float(level[0]), n


def test_tree_chunk_decomposition(orc):
    """Summing aligned 2^c chunks by the tree and then the chunk sums by the
    same tree gives the whole-tensor tree: the GPU relies on this.  Checked
    on a config-4-like tail (n = 4096*c + 1664)."""
    rng = np.random.default_rng(5)
    n = 4096 * 5 + 1664
    leaves = (rng.standard_normal(n) ** 2).astype(np.float32)
    for c in (6, 9, 12):
        C = 1 << c
        parts = np.array([orc.tree_sum(leaves[i:i + C]) for i in range(0, n, C)], np.float32)
        assert bits(orc.tree_sum(parts)) == bits(orc.tree_sum(leaves)), c


# --------------------------------------------------------------------------
# quantiser
# --------------------------------------------------------------------------
def test_quant_dequant_invariant(orc):
    """quantise(dequant(q)) == q for every code and step sizes across many
    binades (|error| of the two roundings is far below 1/2)."""
    rng = np.random.default_rng(3)
    qs = np.arange(-127, 128)
    for e in range(-60, 61, 7):
        for _ in range(3):
            s = np.float32(rng.uniform(1, 2) * 2.0 ** e)
            r = np.float32(1) / s
            for q in qs:
                x = np.float32(q) * s
                assert orc.quant1(float(x), float(r)) == q, (q, s)


@pytest.mark.parametrize("xr,q", [(2.5, 2), (3.5, 4), (-2.5, -2), (-3.5, -4), (0.5, 0),
                                  (1.5, 2), (-0.5, 0), (126.5, 126), (127.5, 127),
                                  (128.0, 127), (1e30, 127), (-127.5, -127), (-1e30, -127),
                                  (0.49999997, 0)])
def test_quant_ties_and_clamp(orc, xr, q):
    assert orc.quant1(xr, 1.0) == q


def test_quant_exhaustive_bf16_vs_fp64(orc):
    """All finite bf16 inputs x with a fixed r: the oracle's code equals the
    fp64 evaluation (exact product of two binary32 values, rounded once to
    binary32 then to the nearest integer, ties to even, clamped)."""
    L = orc.lib()
    h = np.arange(65536, dtype=np.uint32)
    fin = (h & 0x7F80) != 0x7F80
    xs = (h[fin] << 16).view(np.float32)
    xs = np.where((h[fin] & 0x7F80) == 0, np.float32(0) * np.sign(xs), xs).astype(np.float32)
    for r in (np.float32(5.634), np.float32(0.01171875), np.float32(1234.5)):
        with np.errstate(over="ignore"):
            prod = (xs.astype(np.float64) * np.float64(r)).astype(np.float32)
        want = np.clip(np.rint(prod.astype(np.float64)), -127, 127).astype(np.int64)
        got = np.array([L.orc_quant1(float(v), float(r)) for v in xs], np.int64)
        assert np.array_equal(got, want)


def test_lsq_scale_formula_bound(orc, syn):
    """s = 2*mean|x|/sqrt(127) within a few ulp of the exact real value."""
    x = syn.normal((64, 256), 1.0, tag=91)
    q, _, s, amax, fl = orc.quantize_lsq(x)
    exact = 2 * np.abs(x.astype(np.float64)).mean() / math.sqrt(127)
    assert fl == 0
    assert abs(float(s[0]) - exact) <= 4 * np.spacing(np.float32(exact))
    assert amax[0] == np.abs(x).max()
    # codes: fp64 single-rounding evaluation with the oracle's scale
    r = np.float32(1) / s[0]
    prod = (x.astype(np.float64) * np.float64(r)).astype(np.float32)
    want = np.clip(np.rint(prod.astype(np.float64)), -127, 127).astype(np.int8)
    assert np.array_equal(q, want)


def test_lsq_per_row_and_transpose(orc, syn):
    w = syn.normal((32, 256), 0.02, tag=92)
    q, qt, s, amax, _ = orc.quantize_lsq(w, per_row=True, want_t=True)
    assert np.array_equal(qt, q.T)
    for r in range(32):
        q1, _, s1, a1, _ = orc.quantize_lsq(w[r:r + 1])
        assert np.array_equal(q1[0], q[r]) and s1[0] == s[r] and a1[0] == amax[r]


def test_lsq_zero_tensor_and_flags(orc):
    z = np.zeros((4, 64), np.float32)
    q, _, s, amax, fl = orc.quantize_lsq(z)
    assert s[0] == 0 and not q.any() and fl == 0 and amax[0] == 0
    z[1, 3] = np.inf
    assert orc.quantize_lsq(z)[4] == orc.FLAG_NONFINITE
    z[1, 3] = np.nan
    assert orc.quantize_lsq(z)[4] == orc.FLAG_NONFINITE


def test_lsq_col_mul_is_elementwise_product(orc, syn):
    x = syn.normal((16, 64), 1e-3, tag=93)
    cm = syn.normal((64,), 0.01, mean=0.02, tag=94)
    a = orc.quantize_lsq(x, col_mul=cm)
    prod = (x.astype(np.float64) * cm.astype(np.float64)[None, :]).astype(np.float32)
    b = orc.quantize_lsq(prod)
    assert np.array_equal(a[0], b[0]) and a[2][0] == b[2][0]


def test_lsq_daz_on_input(orc):
    x = np.full((1, 64), 1.0, np.float32)
    x[0, :8] = X.bits_to_float(0x00000005)      # subnormals read as zero
    x[0, 8:16] = -X.bits_to_float(0x00400000)
    q, _, s, amax, _ = orc.quantize_lsq(x)
    y = np.full((1, 64), 1.0, np.float32)
    y[0, :16] = 0
    q2, _, s2, _, _ = orc.quantize_lsq(y)
    assert np.array_equal(q, q2) and s[0] == s2[0]


def test_lsq_mean_is_reciprocal_multiply(orc):
    """App. A.3: the mean multiplies by fl(1/n).  For n = 3 and an exactly
    summed S, fl(S*fl(1/3)) and fl(S/3) differ for some S; the oracle's step
    size must follow the reciprocal product, evaluated here in exact
    rationals."""
    k2 = Fraction(orc.lsq_k2())
    inv3 = X.op(Fraction(1, 3))
    hits = 0
    for S in range(1, 4000):
        rm, dv = X.op(S * inv3), X.op(Fraction(S, 3))
        if rm == dv:
            continue
        x = np.array([[float(S), 0.0, 0.0]], np.float32)
        _, _, s, _, _ = orc.quantize_lsq(x)
        assert Fraction(float(s[0])) == X.op(rm * k2), S
        hits += 1
        if hits == 20:
            break
    assert hits == 20


def test_f32_subnormal_inputs_read_as_zero(orc):
    """Table 1: subnormals are flushed everywhere, inputs included.  A row of
    fp32 subnormals normalises to zero (rstd = 1/sqrt(eps) would otherwise
    lift x*rstd into the normal range)."""
    D = 64
    sub = X.bits_to_float(0x00100000)           # 2^-129 * 1.0: subnormal
    x = np.full((2, D), sub, np.float32)
    x[1] = -sub
    g = np.ones(D, np.float32)
    y, rstd, _ = orc.rmsnorm_fwd(x, g, 1e-6)
    assert not y.any() and np.all(np.signbit(y[1])) and not np.any(np.signbit(y[0]))
    assert np.all(rstd == rstd[0])
    # bf16 subnormal rows behave the same
    xb = np.full((1, D), 0x0040, np.uint16)
    yb, _, _ = orc.rmsnorm_fwd(xb, np.full(D, 0x3F80, np.uint16), 1e-6)
    assert not yb.any()
    # fp32 subnormal dy in the fp WHT: rotated values are exactly zero
    d = np.full((4, 3), sub, np.float32)
    _, s_v, v, _ = orc.wht_fp_quant(d, 4, want_v=True)
    assert not v.any() and s_v == 0


def test_bf16_input_equals_widened_f32(orc, syn):
    xb = syn.normal((8, 128), 1.0, tag=95, bf16=True)
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    a, b = orc.quantize_lsq(xb), orc.quantize_lsq(xf)
    assert np.array_equal(a[0], b[0]) and a[2][0] == b[2][0]


# --------------------------------------------------------------------------
# int8 GEMMs
# --------------------------------------------------------------------------
def _codes(rng, shape):
    return rng.integers(-127, 128, size=shape, dtype=np.int64).astype(np.int8)


def test_qgemm_fwd_exact_int(orc):
    rng = np.random.default_rng(21)
    for M, N, K in [(1, 1, 1), (3, 5, 7), (17, 33, 64), (8, 8, 4096)]:
        qx, qw = _codes(rng, (M, K)), _codes(rng, (N, K))
        acc = qx.astype(np.int64) @ qw.astype(np.int64).T
        y = orc.qgemm_fwd(qx, np.float32(1.0), qw, np.ones(N, np.float32))
        assert np.array_equal(y, acc.astype(np.float32))  # |acc| < 2^24: exact
        # the fp64 dot is a second, independent evaluation
        assert np.array_equal(y.astype(np.float64), qx.astype(np.float64) @ qw.astype(np.float64).T)


def test_qgemm_fwd_extreme_acc(orc):
    """K = 131071 codes of -128 keep acc = 2^14 * K = 2^31 - 2^14 < 2^31 (the
    int32 bound for any int8 code); that value is a multiple of 2^7, the
    binary32 spacing there, so it converts exactly."""
    K = 131071
    qx = np.full((2, K), -128, np.int8)
    qx[1] = 127
    qw = np.full((2, K), -128, np.int8)
    qw[1] = 127
    y = orc.qgemm_fwd(qx, np.float32(1.0), qw, np.ones(2, np.float32))
    assert 128 * 128 * K == 2 ** 31 - 2 ** 14
    assert y[0, 0] == np.float32(2 ** 31 - 2 ** 14)
    assert y[0, 1] == np.float32(-128 * 127 * K) and y[1, 1] == np.float32(127 * 127 * K)


def test_qgemm_fwd_epilogue_closed_form(orc):
    # acc = 2^j exactly; scales powers of two: y = 2^(j+a+b) exactly
    qx = np.zeros((1, 64), np.int8)
    qx[0, 0] = 64
    qw = np.zeros((3, 64), np.int8)
    qw[:, 0] = [1, 2, 4]
    sx = np.float32(2.0 ** -3)
    sw = np.array([2.0 ** -1, 2.0 ** -2, 2.0 ** 5], np.float32)
    y = orc.qgemm_fwd(qx, sx, qw, sw)
    assert list(y[0]) == [64 * 1 * 2.0 ** -4, 64 * 2 * 2.0 ** -5, 64 * 4 * 2.0 ** 2]
    # per-tensor weight scale: one value for every column
    y1 = orc.qgemm_fwd(qx, sx, qw, np.float32(0.5))
    assert list(y1[0]) == [64 * 1 * 2.0 ** -4, 64 * 2 * 2.0 ** -4, 64 * 4 * 2.0 ** -4]


def test_qgemm_fwd_rounding_of_acc(orc):
    """int32 -> binary32 rounds to nearest even: acc = 2^24 + 1 -> 2^24."""
    K = 1041
    qx = np.full((1, K), 127, np.int8)
    qw = np.full((1, K), 127, np.int8)
    acc = 127 * 127 * K  # 16790529
    y = orc.qgemm_fwd(qx, np.float32(1.0), qw, np.float32(1.0))
    assert float(y[0, 0]) == float(X.round_binary32(Fraction(acc)))


def test_qgemm_bwd_dx_exact_int(orc):
    rng = np.random.default_rng(22)
    for M, N, K in [(1, 1, 1), (5, 9, 3), (16, 64, 48)]:
        qg, qw = _codes(rng, (M, N)), _codes(rng, (N, K))
        acc = qg.astype(np.int64) @ qw.astype(np.int64)
        dx = orc.qgemm_bwd_dx(qg, np.float32(0.25), qw)
        assert np.array_equal(dx, (acc * 0.25).astype(np.float32))


# --------------------------------------------------------------------------
# Walsh-Hadamard rotations
# --------------------------------------------------------------------------
@pytest.mark.parametrize("b", [1, 2, 4, 8, 64, 128])
def test_wht_int_matches_sylvester(orc, b):
    H = scipy.linalg.hadamard(b).astype(np.int64)
    assert np.array_equal(H @ H.T, b * np.eye(b, dtype=np.int64))
    rng = np.random.default_rng(b)
    M, K = 2 * b, 24
    qx = _codes(rng, (M, K))
    u = orc.wht_int(qx, b)
    want = np.concatenate([H @ qx[i:i + b].astype(np.int64) for i in range(0, M, b)])
    assert np.array_equal(u, want)


def test_wht_int_involution(orc):
    """H (H v) = b v, exactly, on inputs small enough to stay int8."""
    b = 8
    rng = np.random.default_rng(2)
    qx = rng.integers(-3, 4, size=(16, 10)).astype(np.int8)
    u = orc.wht_int(qx, b)
    assert np.abs(u).max() <= 127
    uu = orc.wht_int(u.astype(np.int8), b)
    assert np.array_equal(uu, b * qx.astype(np.int32))


def test_wht_int_quant_statistic(orc):
    rng = np.random.default_rng(9)
    qx = _codes(rng, (128, 64))
    b = 64
    q_u, s_u, S = orc.wht_int_quant(qx, b)
    u = orc.wht_int(qx, b).astype(np.int64)
    assert S == np.abs(u).sum()
    exact = 2 * (S / u.size) / math.sqrt(127)
    assert abs(float(s_u) - exact) <= 4 * np.spacing(np.float32(exact))
    r = np.float32(1) / np.float32(s_u)
    prod = (u.astype(np.float64) * np.float64(r)).astype(np.float32)
    assert np.array_equal(q_u, np.clip(np.rint(prod.astype(np.float64)), -127, 127).astype(np.int8))


@pytest.mark.parametrize("b", [2, 16, 64, 128])
def test_wht_fp_integer_inputs_exact(orc, b):
    """Integer-valued inputs stay exact in binary32: the fp butterfly must
    equal the Sylvester transform."""
    H = scipy.linalg.hadamard(b).astype(np.int64)
    rng = np.random.default_rng(b + 1)
    M, N = 2 * b, 12
    d = rng.integers(-1000, 1001, size=(M, N))
    _, _, v, fl = orc.wht_fp_quant(d.astype(np.float32), b, want_v=True)
    want = np.concatenate([H @ d[i:i + b] for i in range(0, M, b)])
    assert fl == 0 and np.array_equal(v, want.astype(np.float32))


def test_wht_fp_random_within_bound(orc, syn):
    b = 128
    H = scipy.linalg.hadamard(b).astype(np.float64)
    dy = syn.normal((256, 16), 1e-3, tag=97)
    _, _, v, _ = orc.wht_fp_quant(dy, b, want_v=True)
    d64 = dy.astype(np.float64)
    want = np.concatenate([H @ d64[i:i + b] for i in range(0, 256, b)])
    l1 = np.concatenate([np.abs(H) @ np.abs(d64[i:i + b]) for i in range(0, 256, b)])
    bound = math.log2(b) * 2.0 ** -24 * l1 * 1.01
    assert np.all(np.abs(v - want) <= bound)


def test_wht_fp_bf16_and_f32_agree(orc, syn):
    dyb = syn.normal((128, 32), 1e-3, tag=98, bf16=True)
    dyf = (dyb.astype(np.uint32) << 16).view(np.float32)
    a = orc.wht_fp_quant(dyb, 64)
    b = orc.wht_fp_quant(dyf, 64)
    assert np.array_equal(a[0], b[0]) and a[1] == b[1]


def test_wht_rejects_ragged_blocks(orc):
    """The rotations need a power-of-two block dividing the rotated
    dimension; anything else is refused before the C loops run."""
    q = np.zeros((64, 32), np.int8)
    dy = np.zeros((64, 32), np.float32)
    for call in (lambda: orc.wht_int(q, 128), lambda: orc.wht_int_quant(q, 128),
                 lambda: orc.wht_fp_quant(dy, 128), lambda: orc.wht_fp_quant(dy, 24),
                 lambda: orc.qgemm_bwd_dw_wht(q, np.ones(1, np.float32), dy, 128),
                 lambda: orc.wht_fp_rows_quant(dy, 64)):
        with pytest.raises(ValueError):
            call()


def test_dw_gemm_rotation_identity(orc):
    """(H qx)^T (H qv) = b * qx^T qv in integers; with unit scales the dW
    GEMM returns acc * 2^-log2(b) exactly (checks transposition/indexing)."""
    b = 16
    rng = np.random.default_rng(4)
    M, N, K = 32, 6, 5
    qx = rng.integers(-5, 6, size=(M, K)).astype(np.int8)
    qv = rng.integers(-5, 6, size=(M, N)).astype(np.int8)
    u = orc.wht_int(qx, b)
    hv = orc.wht_int(qv, b)
    lhs = hv.T.astype(np.int64) @ u.astype(np.int64)
    rhs = b * (qv.T.astype(np.int64) @ qx.astype(np.int64))
    assert np.array_equal(lhs, rhs)
    dw = orc.dw_gemm(hv.astype(np.int8), u.astype(np.int8), 1.0, 1.0, 1.0, b)
    assert np.abs(hv).max() <= 127 and np.abs(u).max() <= 127
    assert np.array_equal(dw, (qv.T.astype(np.int64) @ qx.astype(np.int64)).astype(np.float32))


def test_dw_gemm_row_range(orc):
    rng = np.random.default_rng(6)
    qv, qu = _codes(rng, (64, 10)), _codes(rng, (64, 7))
    full = orc.dw_gemm(qv, qu, 0.5, 0.25, 2.0, 64)
    part = orc.dw_gemm(qv, qu, 0.5, 0.25, 2.0, 64, 3, 8)
    assert np.array_equal(part[3:8], full[3:8]) and not part[:3].any()


def test_dw_wht_reduces_error(orc, syn):
    """§3.2 "int8 computation": rotating along tokens before int8
    quantisation of the weight gradient cuts its relative error (the pages
    report ~5% -> ~1% at their shapes).  b = 1 is the unrotated case."""
    M, K, N = 2048, 64, 32
    x = syn.normal((M, K), 1.0, tag=101)
    dy = syn.student_t3((M, N), 1e-3, tag=102)
    qx, _, sx, _, _ = orc.quantize_lsq(x)
    xhat = qx.astype(np.float64) * float(sx[0])
    ref = dy.astype(np.float64).T @ xhat
    err = {}
    for b in (1, 128):
        dw, _, _, _ = orc.qgemm_bwd_dw_wht(qx, sx, dy, b)
        err[b] = np.linalg.norm(dw - ref) / np.linalg.norm(ref)
    # heavy-tailed gradients: rotation at least halves the error; what is
    # left is the LSQ step's own noise floor (step ~0.14 sigma after the
    # rotation Gaussianises the tensor: ~4% per quantised operand)
    assert err[128] < 0.5 * err[1]
    assert err[128] < 0.07 and err[1] > 0.10


# --------------------------------------------------------------------------
# RMSNorm and grad-norm
# --------------------------------------------------------------------------
def test_rmsnorm_pm1_rows_closed_form(orc):
    D = 2048
    rng = np.random.default_rng(12)
    x = np.where(rng.random((4, D)) < 0.5, -1.0, 1.0).astype(np.float32)
    g = np.ones(D, np.float32)
    y, rstd, fl = orc.rmsnorm_fwd(x, g, 1e-6)
    getcontext().prec = 100
    eps = Fraction(float(np.float32(1e-6)))
    ms_eps = X.op(1 + eps)                      # ss = D exactly, ms = 1 exactly
    sq = X.round_binary32(Fraction((Decimal(ms_eps.numerator) / Decimal(ms_eps.denominator)).sqrt()))
    want = X.op(1 / sq)
    assert fl == 0 and np.all(rstd == np.float32(float(want)))
    assert np.array_equal(y, x * rstd[:, None])


def test_rmsnorm_y_grouping_closed_form(orc, syn):
    """y = fl(fl(x * rstd) * g), not fl(x * fl(rstd * g)).  Rows of 1536
    entries +-1, 192 entries +-1.5 and 320 entries +-0.5 have sum of squares
    2048 exactly (every partial sum is a multiple of 1/4), so ms = 1 and
    rstd = fl(1/fl(sqrt(fl(1 + 1e-6)))) = 1 - 2^-21 (fl(1 + 1e-6) =
    1 + 2^-20, its square root rounds to 1 + 2^-21, whose reciprocal rounds
    to 1 - 2^-21).  Then x * rstd is exact for these x, and y is the one
    rounding of an exact product, computed in double (48-bit products are
    exact there).  For x = +-1.5 the other grouping rounds twice and differs
    for some g."""
    D = 2048
    rng = np.random.default_rng(3)
    T = 16
    x = np.empty((T, D), np.float32)
    for t in range(T):
        row = np.array([1.0] * 1536 + [1.5] * 192 + [0.5] * 320, np.float32)
        rng.shuffle(row)
        x[t] = row * rng.choice([-1.0, 1.0], size=D).astype(np.float32)
    g = syn.normal((D,), 0.1, mean=1.0, tag=5)
    y, rstd, fl = orc.rmsnorm_fwd(x, g, 1e-6)
    r = np.float32(1.0 - 2.0 ** -21)
    assert fl == 0 and np.all(rstd == r)
    xr = x.astype(np.float64) * np.float64(r)
    assert np.array_equal(xr.astype(np.float32).astype(np.float64), xr)  # x * rstd exact
    want = (xr * g.astype(np.float64)[None, :]).astype(np.float32)
    assert np.array_equal(y.view(np.uint32), want.view(np.uint32))
    other = (x * (r * g).astype(np.float32)[None, :]).astype(np.float32)
    assert np.any(other.view(np.uint32) != want.view(np.uint32))


def test_rmsnorm_fwd_fp64_bound(orc, syn):
    x = syn.normal((16, 512), 1.0, tag=111)
    g = syn.normal((512,), 0.1, mean=1.0, tag=112)
    y, rstd, _ = orc.rmsnorm_fwd(x, g, 1e-6)
    x64 = x.astype(np.float64)
    r64 = 1 / np.sqrt((x64 ** 2).mean(1) + float(np.float32(1e-6)))
    assert np.allclose(rstd, r64, rtol=4e-7, atol=0)
    assert np.allclose(y, x64 * r64[:, None] * g.astype(np.float64), rtol=1e-6, atol=0)


def test_rmsnorm_bf16_io(orc, syn):
    x = syn.normal((8, 256), 1.0, tag=113, bf16=True)
    g = syn.normal((256,), 0.1, mean=1.0, tag=114, bf16=True)
    y, rstd, _ = orc.rmsnorm_fwd(x, g, 1e-6)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    gf = (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    yf = (y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = xf / np.sqrt((xf ** 2).mean(1, keepdims=True) + 1e-6) * gf
    assert np.all(np.abs(yf - ref) <= np.abs(ref) * 2.0 ** -8 * 1.01 + 1e-30)


def test_rmsnorm_subnormal_inputs_flush(orc):
    D = 64
    x = np.ones((1, D), np.uint16) * 0x3F80      # bf16 1.0
    x[0, :5] = [0x0001, 0x8001, 0x007F, 0x807F, 0x0040]
    g = np.ones(D, np.uint16) * 0x3F80
    y, rstd, _ = orc.rmsnorm_fwd(x, g, 1e-6)
    x2 = x.copy()
    x2[0, :5] = [0x0000, 0x8000, 0x0000, 0x8000, 0x0000]
    y2, rstd2, _ = orc.rmsnorm_fwd(x2, g, 1e-6)
    assert np.array_equal(y, y2) and rstd[0] == rstd2[0]
    assert list(y[0, :2]) == [0x0000, 0x8000]  # signed zeros kept


def test_rmsnorm_bwd_fp64(orc, syn):
    T, D = 32, 256
    x = syn.normal((T, D), 1.0, tag=115)
    g = syn.normal((D,), 0.1, mean=1.0, tag=116)
    dy = syn.normal((T, D), 1e-3, tag=117)
    _, rstd, _ = orc.rmsnorm_fwd(x, g, 1e-6)
    dx, dg = orc.rmsnorm_bwd(x, g, rstd, dy)
    x64, g64, dy64 = (a.astype(np.float64) for a in (x, g, dy))
    r = 1 / np.sqrt((x64 ** 2).mean(1, keepdims=True) + float(np.float32(1e-6)))
    xh = x64 * r
    d = dy64 * g64
    dx_ref = r * (d - xh * (d * xh).mean(1, keepdims=True))
    dg_ref = (dy64 * xh).sum(0)
    assert np.allclose(dx, dx_ref, rtol=1e-4, atol=1e-9)
    assert np.allclose(dg, dg_ref, rtol=1e-4, atol=1e-9)
    # with g = 1 the gradient is orthogonal to x-hat (up to rounding)
    dx1, _ = orc.rmsnorm_bwd(x, np.ones(D, np.float32), rstd, dy)
    assert np.all(np.abs((dx1 * xh).sum(1)) < 1e-6 * np.abs(dx1).sum(1).max())


def test_grad_norm_closed_form(orc):
    for n, v, ss in [(1 << 16, 2.0 ** -8, 1.0), (1 << 20, 2.0 ** -10, 1.0), (12, 3.0, 108.0)]:
        a = np.full(n, v, np.float32)
        s, nrm, fl = orc.grad_norm(a)
        assert s == ss and nrm == np.float32(math.sqrt(ss)) and fl == 0


def test_grad_norm_tail_order(orc):
    """n = 4096*2 + 1664 leaves: squares of 2^12 then ones; the tree adds the
    tail subtree last, so the ones' sum (exact) meets 2^24 once."""
    n = 4096 * 2 + 1664
    v = np.ones(n, np.float32)
    v[0] = 4096.0
    s, _, _ = orc.grad_norm(v)
    # left subtree [0,8192): 2^24 + 8191 ones -> exact sum within each
    # aligned 2^j block that excludes leaf 0; exact-rational emulation:
    level = [Fraction(float(np.float32(t) * np.float32(t))) for t in v]
    while len(level) > 1:
        nxt = [X.op(level[2 * i] + level[2 * i + 1]) for i in range(len(level) // 2)]
        if len(level) % 2:
            nxt.append(level[-1])
        level = nxt
    assert float(s) == float(level[0])


def test_grad_norm_fp64_bound(orc, syn):
    v = syn.normal((100003,), 1e-4, tag=121)
    s, nrm, _ = orc.grad_norm(v)
    ref = (v.astype(np.float64) ** 2).sum()
    # pairwise tree error bound: ceil(log2 n) * u * sum + one rounding per square
    assert abs(float(s) - ref) <= (17 + 1) * 2.0 ** -24 * ref
    assert abs(float(nrm) - math.sqrt(ref)) <= 10 * 2.0 ** -24 * math.sqrt(ref)


def test_grad_norm_nonfinite_flag(orc):
    v = np.ones(100, np.float32)
    v[50] = np.float32(2e19)  # square overflows
    assert orc.grad_norm(v)[2] == orc.FLAG_NONFINITE


# --------------------------------------------------------------------------
# hash
# --------------------------------------------------------------------------
def test_sha256_vs_hashlib(orc):
    rng = np.random.default_rng(13)
    for n in list(range(0, 130)) + [4095, 4096, 4097, 65536 + 17]:
        m = rng.integers(0, 256, size=n, dtype=np.uint8).tobytes()
        assert orc.sha256(m) == hashlib.sha256(m).digest(), n


def _merkle_py(b: bytes) -> bytes:
    leaves = [b[i:i + 4096] for i in range(0, len(b), 4096)] or [b""]
    d = [hashlib.sha256(x).digest() for x in leaves]
    while len(d) > 1:
        d = [hashlib.sha256(b"".join(d[i:i + 128])).digest() for i in range(0, len(d), 128)]
    return d[0]


def _tensor_digest_py(name, a, code):
    h = b"BRQ1" + bytes([code, a.ndim]) + b"".join(struct.pack("<Q", s) for s in a.shape)
    h += struct.pack("<H", len(name)) + name.encode() + _merkle_py(a.tobytes())
    return hashlib.sha256(h).digest()


def test_merkle_vs_python(orc):
    rng = np.random.default_rng(14)
    for n in (0, 1, 4096, 4097, 4096 * 128, 4096 * 128 + 1, 4096 * 129 * 3 + 5):
        a = rng.integers(0, 256, size=n, dtype=np.uint8)
        assert orc.merkle_root(a) == _merkle_py(a.tobytes()), n


def test_hash_state_vs_python(orc):
    rng = np.random.default_rng(15)
    ts = [("y", rng.standard_normal((33, 70)).astype(np.float32), 0),
          ("dw", rng.standard_normal((5, 4096 * 3 + 1)).astype(np.float32), 0),
          ("x", rng.integers(0, 65535, size=(7, 9), dtype=np.uint16), 1),
          ("q", rng.integers(-127, 128, size=(0, 4), dtype=np.int64).astype(np.int8), 2)]
    want = hashlib.sha256(b"".join(_tensor_digest_py(n, a, c) for n, a, c in ts)).digest()
    assert orc.hash_state(ts) == want
    # one flipped bit anywhere changes the state digest
    ts[1][1].view(np.uint8).reshape(-1)[12345] ^= 1
    assert orc.hash_state(ts) != want


# --------------------------------------------------------------------------
# input generator (shared with the GPU path; holds no method arithmetic)
# --------------------------------------------------------------------------
def test_philox_known_answers(syn):
    for line in open(os.path.join(GOLDEN, "philox_kat.txt")):
        if line.startswith("#") or not line.strip():
            continue
        lhs, rhs = line.split("->")
        w = [int(t, 16) for t in lhs.split()]
        want = [int(t, 16) for t in rhs.split()]
        assert list(syn.philox4x32_10(w[:4], w[4:])) == want


def test_generator_counter_based(syn):
    a = syn.normal((1000,), 1.0, tag=77)
    b = syn.normal((1500,), 1.0, tag=77)
    assert np.array_equal(a, b[:1000])       # value i depends on (seed, tag, i) only
    c = syn.normal((1000,), 1.0, tag=78)
    assert not np.array_equal(a, c)


# --------------------------------------------------------------------------
# optimizer: AdamW, global-norm clip, spike skip (report §3.2 "Optimizer",
# "Optimizer-state precision"; §3.4.2 "Gradient behavior, Clipping, and
# Spike Protocol")
# --------------------------------------------------------------------------
def test_adamw_bias_corrections_exact_and_bounded(orc):
    b1, b2 = Fraction(float(f32(0.9))), Fraction(float(f32(0.95)))
    # t = 1: 1 - beta is exact in binary32 (Sterbenz)
    bc1, bc2 = orc.adamw_bias_corrections(1)
    assert Fraction(float(bc1)) == 1 - b1 and Fraction(float(bc2)) == 1 - b2
    # t > 1: within t half-ulp relative errors of the exact power, plus the
    # final rounding
    for t in (2, 3, 10, 100, 1000):
        bc1, bc2 = orc.adamw_bias_corrections(t)
        for bc, b in ((bc1, b1), (bc2, b2)):
            exact = 1 - b ** t
            bound = (b ** t) * Fraction(t, 2 ** 23) + Fraction(float(np.spacing(f32(bc))))
            assert abs(Fraction(float(bc)) - exact) <= bound, (t, float(bc), float(exact))
    # very long runs: beta^t flushes to zero, the correction is 1
    assert orc.adamw_bias_corrections(100000) == (f32(1.0), f32(1.0))


def test_adamw_decide_spike_protocol(orc):
    """A pre-clip norm above 5 skips five optimizer steps (this one and the
    next four); two spikes skip ten; a norm in (1, 5] is clipped to 1; a norm
    of at most 1 is left alone.  A non-finite norm counts as a spike (the
    reading for a case the pages leave open)."""
    norms = [0.3, 1.0, 2.5, 5.0, 5.78, 0.4, 0.4, 0.4, 0.4, 0.4, 0.4, 6.88, 0.2, 7.0, 0.2,
             0.2, 0.2, 0.2, 0.2, 0.2, float("inf"), 0.2, 0.2, 0.2, 0.2, 0.2]
    # the protocol written out independently: remaining skips after a spike
    expect, remaining = [], 0
    for n in norms:
        if not math.isfinite(n) or n > 5.0:
            remaining = 5
        if remaining:
            remaining -= 1
            expect.append("skip")
        else:
            expect.append("clip" if n > 1.0 else "keep")
    st, skipped, got = 0, 0, []
    for n in norms:
        ap, cl, st, fl = orc.adamw_decide(n, st)
        assert fl == (0 if math.isfinite(n) else 1)
        if ap == 0.0:
            got.append("skip")
            skipped += 1
            assert cl == 0.0
        elif cl != 1.0:
            got.append("clip")
            # the clipped gradient has norm 1 up to the rounding of 1 / norm
            assert abs(float(cl) * n - 1.0) <= 2.0 ** -23, (n, cl)
        else:
            got.append("keep")
            assert cl == 1.0
    assert got == expect
    # the pages' run: two spikes, ten skipped steps; here a third spike lands
    # inside the second window and restarts it, and the inf adds a fourth
    assert expect.count("skip") == skipped == 5 + 2 + 5 + 5


def _adamw_f64(p, g, m, v, lr, t, wd, beta1=0.9, beta2=0.95, eps=1e-8):
    """The same update in binary64 from the same binary32 inputs."""
    b1, b2, e = float(f32(beta1)), float(f32(beta2)), float(f32(eps))
    p, g, m, v = (np.asarray(a, np.float64) for a in (p, g, m, v))
    m2 = b1 * m + (1 - b1) * g
    v2 = b2 * v + (1 - b2) * g * g
    mh = m2 / (1 - b1 ** t)
    vh = v2 / (1 - b2 ** t)
    u = mh / (np.sqrt(vh) + e)
    return p - float(f32(lr)) * (u + float(f32(wd)) * p), m2, v2, u


def test_adamw_step_fp32_param_vs_fp64(orc):
    rng = np.random.default_rng(11)
    n = 4096
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = (np.abs(rng.standard_normal(n)) * 1e-7 + 1e-9).astype(np.float32)
    lr, t = 3e-4, 7
    bc1, bc2 = orc.adamw_bias_corrections(t)
    p1, m1, v1 = orc.adamw_step(p, g, m, v, lr, bc1, bc2)
    pe, me, ve, ue = _adamw_f64(p, g, m, v, lr, t, 0.1)
    # moments: two products and a sum, each rounded once -- half an ulp of
    # each product and of the sum (the terms may cancel)
    b1, b2 = float(f32(0.9)), float(f32(0.95))
    tm = (np.abs(b1 * m.astype(np.float64)) + np.abs((1 - b1) * g.astype(np.float64))) * 2.0 ** -24
    tv = (np.abs(b2 * v.astype(np.float64)) + (1 - b2) * g.astype(np.float64) ** 2 * 2) * 2.0 ** -24
    assert np.all(np.abs(m1 - me) <= tm + np.spacing(np.abs(m1)) / 2)
    assert np.all(np.abs(v1 - ve) <= tv + np.spacing(np.abs(v1)) / 2)
    # parameter: one rounding of p plus lr times the few-ulp error of u
    tol = np.spacing(np.abs(p1)) + float(lr) * np.abs(ue) * 16 * 2.0 ** -24
    assert np.all(np.abs(p1 - pe) <= tol)
    # and it moved against the gradient direction of u for every element
    assert np.all(np.sign(p - p1) == np.sign(ue + 0.1 * p))


def test_adamw_step_bf16_param_rounds_once(orc):
    rng = np.random.default_rng(12)
    n = 4096
    pf = (rng.standard_normal(n) * 0.02).astype(np.float32)
    pb = np.array([orc.f32_to_bf16(float(x)) for x in pf], np.uint16)
    pw = np.array([orc.bf16_to_f32(int(h)) for h in pb], np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    lr, t = 1e-3, 1
    bc1, bc2 = orc.adamw_bias_corrections(t)
    p1, _, _ = orc.adamw_step(pb, g, m, v, lr, bc1, bc2)
    pe, _, _, ue = _adamw_f64(pw, g, m, v, lr, t, 0.1)
    # first step from zero moments: u = g / (|g| + eps), +-1 up to eps/|g|
    assert np.all(np.abs(np.abs(ue) - 1.0) <= 1e-8 / np.abs(g) + 1e-6)
    # the bf16 result is one of the two bf16 neighbours of the exact value,
    # and the nearest whenever the exact value is not within 2^-14 relative
    # of a rounding boundary
    got = np.array([orc.bf16_to_f32(int(h)) for h in p1], np.float64)
    ulp = np.array([float(np.spacing(np.float32(abs(x)))) * 65536 for x in pe])
    assert np.all(np.abs(got - pe) <= ulp)
    nearest = np.array([orc.bf16_to_f32(orc.f32_to_bf16(float(x))) for x in pe], np.float64)
    frac = np.abs(pe / ulp - np.round(pe / ulp))
    safe = np.abs(frac - 0.5) > 1e-3
    assert np.all(got[safe] == nearest[safe])


def test_adamw_zero_gradient_and_skip_are_identities(orc):
    rng = np.random.default_rng(13)
    n = 257
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    z = np.zeros(n, np.float32)
    bc1, bc2 = orc.adamw_bias_corrections(3)
    # zero gradient, zero moments, no weight decay: u = 0 / (0 + eps) = 0
    p1, m1, v1 = orc.adamw_step(p, z, z, z, 3e-4, bc1, bc2, wd=0.0)
    assert np.array_equal(p1.view(np.uint32), p.view(np.uint32))
    assert not m1.any() and not v1.any()
    # a skipped step changes nothing at all
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = (np.abs(rng.standard_normal(n)) * 1e-7).astype(np.float32)
    p2, m2, v2 = orc.adamw_step(p, g, m, v, 3e-4, bc1, bc2, apply=0.0, clip=0.0)
    for a, b in ((p2, p), (m2, m), (v2, v)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    # decay alone (zero gradient and moments) shrinks every weight toward 0
    p3, _, _ = orc.adamw_step(p, z, z, z, 0.1, bc1, bc2, wd=0.5)
    assert np.all(np.abs(p3) <= np.abs(p)) and np.all(np.sign(p3) * np.sign(p) >= 0)


def test_bf16_array_rounding_matches_torch(orc):
    """The GEMMs' bf16-output variant rounds each fp32 result once to
    nearest even: the oracle's array rounding equals torch's independent
    float32 -> bfloat16 conversion, ties and extremes included."""
    import torch
    rng = np.random.default_rng(21)
    a = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000).astype(np.float32),
        np.array([1.00390625, 1.01171875, -1.00390625, 3.4e38, -3.4e38, 0.0, -0.0, 1e-38, 6e-39], np.float32),
    ]).astype(np.float32)
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.to_bf16(a)
    finite = np.isfinite(a)
    assert np.array_equal(got[finite], want[finite])


# --------------------------------------------------------------------------
# exact statistic: the sum of |v| without rounding, then one rounding
# --------------------------------------------------------------------------
def _exact_abs_sum_ref(v):
    """Exact rational sum of |v| (each v flushed first), one binary32
    rounding by tests/_exact.py, +inf past the binary32 range."""
    v = np.asarray(v, np.float32).ravel()
    if np.isnan(v).any():
        return float("nan")
    if np.isinf(v).any():
        return float("inf")
    tot = sum((Fraction(abs(float(x))) for x in v if abs(float(x)) >= 2.0 ** -126), Fraction(0))
    r = X.op(tot)
    return float("inf") if r >= Fraction(2) ** 128 else float(r)


def _same(a, b):
    a, b = float(a), float(b)
    return (math.isnan(a) and math.isnan(b)) or bits(a) == bits(b)


def test_exact_abs_sum_directed(orc):
    """Ties to even, the sticky bit, carries, the range ends, specials."""
    big = float(np.finfo(np.float32).max)
    cases = [
        ([], 0.0),
        ([-3.0, 5.0], 8.0),
        ([2.0 ** 24, 1.0], 2.0 ** 24),                      # tie, even kept
        ([2.0 ** 24 + 2, 1.0], 2.0 ** 24 + 4),              # tie, odd rounds up
        ([2.0 ** 24, 1.0, 2.0 ** -20], 2.0 ** 24 + 2),      # just above the tie
        ([2.0 ** 24, 1.0, 2.0], 2.0 ** 24 + 4),
        ([1.0, 2.0 ** -24, 2.0 ** -24], 1.0 + 2.0 ** -23),  # a tree gives 1.0
        ([1.0] + [2.0 ** -30] * 1024, 1.0 + 2.0 ** -20),
        ([2.0 ** -126 * (1 + 2.0 ** -23), 2.0 ** -126], 2.0 ** -125),  # tie at the bottom
        ([2.0 ** -126], 2.0 ** -126),
        ([X.bits_to_float(0x00000007), 1.0], 1.0),          # subnormal input reads as 0
        ([X.bits_to_float(0x007FFFFF)], 0.0),
        ([X.bits_to_float(0x007FFFFF)] * 2, 0.0),           # would sum to a normal
        ([2.0 ** -126, X.bits_to_float(0x00400000)], 2.0 ** -126),
        ([big, big], float("inf")),
        ([big, 2.0 ** 103], float("inf")),                  # tie above FLT_MAX goes up
        ([big, 2.0 ** 102], big),
        ([float("inf"), 1.0], float("inf")),
        ([-float("inf")], float("inf")),
        ([float("nan"), float("inf")], float("nan")),
    ]
    for v, want in cases:
        got = orc.exact_abs_sum(np.array(v, np.float32))
        assert _same(got, want), (v, got, want)
        assert _same(_exact_abs_sum_ref(v), want), v


@pytest.mark.parametrize("seed", range(6))
def test_exact_abs_sum_random_vs_rationals(orc, seed):
    """Values whose exponents span the whole binary32 range (the sum of any
    such set needs far more than 64 bits), random lengths, random signs."""
    rng = np.random.default_rng(1000 + seed)
    for trial in range(40):
        n = int(rng.integers(1, 400))
        lo, hi = sorted(rng.integers(1, 255, size=2))
        e = rng.integers(lo, hi + 1, size=n).astype(np.uint32)
        u = (e << 23) | rng.integers(0, 1 << 23, size=n).astype(np.uint32)
        u |= (rng.integers(0, 2, size=n).astype(np.uint32) << 31)
        v = u.view(np.float32)
        got = orc.exact_abs_sum(v)
        assert _same(got, _exact_abs_sum_ref(v)), (seed, trial)
        # order-free: any permutation gives the same bits
        assert _same(orc.exact_abs_sum(v[rng.permutation(n)]), got)


def test_exact_abs_sum_gaussian_and_ties(orc, syn):
    """Layer-like data (N(0,1) bf16 activations), and sums built to land on
    exact ties of the final rounding."""
    x = syn.normal((8, 1024), 1.0, tag=95, bf16=True)
    v = (x.astype(np.uint32) << 16).view(np.float32)
    assert _same(orc.exact_abs_sum(v), _exact_abs_sum_ref(v))
    rng = np.random.default_rng(7)
    for _ in range(50):
        a = np.float32(rng.uniform(1.0, 2.0)) * np.float32(2.0 ** int(rng.integers(-40, 40)))
        ulp = float(np.spacing(a))
        for k in (0.5, 1.5, 0.25, 0.75):
            v = np.array([a, k * ulp], np.float32)
            assert _same(orc.exact_abs_sum(v), _exact_abs_sum_ref(v))


def test_lsq_exact_statistic_scale_and_codes(orc, syn):
    """The exact variant differs from the tree only in S: its step size is
    lsq_scale(exact S) and its codes the reciprocal-multiply codes of that
    step; per-row groups each take their own exact S; col_mul multiplies
    first."""
    x = syn.normal((64, 256), 1.0, tag=96)
    q, _, s, amax, fl = orc.quantize_lsq(x, exact=True)
    S = _exact_abs_sum_ref(x)
    assert fl == 0 and amax[0] == np.abs(x).max()
    s_want, r_want = orc.lsq_scale(S, x.size)
    assert bits(s[0]) == bits(s_want)
    exact = 2 * np.abs(x.astype(np.float64)).mean() / math.sqrt(127)
    assert abs(float(s[0]) - exact) <= 4 * np.spacing(np.float32(exact))
    prod = (x.astype(np.float64) * np.float64(r_want)).astype(np.float32)
    want = np.clip(np.rint(prod.astype(np.float64)), -127, 127).astype(np.int8)
    assert np.array_equal(q, want)
    w = syn.normal((16, 256), 0.02, tag=97)
    q, qt, s, amax, _ = orc.quantize_lsq(w, per_row=True, want_t=True, exact=True)
    assert np.array_equal(qt, q.T)
    for r in range(16):
        assert bits(s[r]) == bits(orc.lsq_scale(_exact_abs_sum_ref(w[r]), 256)[0])
    cm = syn.normal((256,), 0.01, mean=0.02, tag=98)
    a = orc.quantize_lsq(x, col_mul=cm, exact=True)
    prod = (x.astype(np.float64) * cm.astype(np.float64)[None, :]).astype(np.float32)
    b = orc.quantize_lsq(prod, exact=True)
    assert np.array_equal(a[0], b[0]) and a[2][0] == b[2][0]
    z = np.zeros((4, 64), np.float32)
    q, _, s, amax, fl = orc.quantize_lsq(z, exact=True)
    assert s[0] == 0 and not q.any() and fl == 0
    z[1, 3] = np.inf
    assert orc.quantize_lsq(z, exact=True)[4] == orc.FLAG_NONFINITE


# --------------------------------------------------------------------------
# rotated input-gradient GEMM (rotation along n)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("b", [1, 2, 8, 128])
def test_wht_rows_integer_inputs_exact(orc, b):
    """Integer-valued inputs stay exact: the row rotation must equal the
    Sylvester transform of each aligned block of b consecutive n."""
    H = scipy.linalg.hadamard(b).astype(np.int64)
    rng = np.random.default_rng(b + 11)
    M, N = 6, 2 * b if b >= 8 else 16
    d = rng.integers(-1000, 1001, size=(M, N))
    _, _, v, fl = orc.wht_fp_rows_quant(d.astype(np.float32), b, want_v=True)
    want = np.concatenate([d[:, i:i + b] @ H.T for i in range(0, N, b)], axis=1)
    assert fl == 0 and np.array_equal(v, want.astype(np.float32))


def test_wht_rows_random_within_bound_and_multiplier(orc, syn):
    """fp32 rows rotation of dy * s_w within the butterfly's rounding bound
    of the fp64 transform of the fp64 product."""
    b = 128
    H = scipy.linalg.hadamard(b).astype(np.float64)
    dy = syn.normal((8, 512), 1e-3, tag=310)
    sw = syn.normal((512,), 0.01, mean=0.02, tag=311)
    _, _, v, _ = orc.wht_fp_rows_quant(dy, b, s_w=sw, want_v=True)
    g = dy.astype(np.float64) * sw.astype(np.float64)[None, :]
    want = np.concatenate([g[:, i:i + b] @ H.T for i in range(0, 512, b)], axis=1)
    l1 = np.concatenate([np.abs(g[:, i:i + b]) @ np.abs(H.T) for i in range(0, 512, b)], axis=1)
    bound = (math.log2(b) + 1) * 2.0 ** -24 * l1 * 1.01
    assert np.all(np.abs(v - want) <= bound)


def test_wht_rows_b1_is_the_plain_quantiser(orc, syn):
    """b = 1 rotates nothing: the codes and step of g = dy * s_w are those of
    the unrotated path's quantiser."""
    dy = syn.normal((64, 256), 1e-3, tag=312)
    sw = syn.normal((256,), 0.01, mean=0.02, tag=313)
    q, s, _, _ = orc.wht_fp_rows_quant(dy, 1, s_w=sw)
    q0, _, s0, _, _ = orc.quantize_lsq(dy, col_mul=sw)
    assert np.array_equal(q, q0) and bits(s) == bits(s0[0])


@pytest.mark.parametrize("b", [16, 128])
def test_dx_wht_epilogue_closed_form(orc, syn, b):
    """dx = fl(fl(acc) * fl(fl(s_g * s_h) * 1/b)) with acc the exact int64
    product of the two rotated code tensors (numpy integer algebra)."""
    M, N, K = 64, 256, 96
    dy = syn.normal((M, N), 1e-3, tag=314)
    w = syn.normal((N, K), 0.02, tag=315)
    qw, _, sw, _, _ = orc.quantize_lsq(w, per_row=True)
    dx, s_g, s_h, fl = orc.qgemm_bwd_dx_wht(dy, sw, qw, b)
    q_g, s_g2, _, _ = orc.wht_fp_rows_quant(dy, b, s_w=sw)
    q_h, s_h2, _ = orc.wht_int_quant(qw, b)
    assert fl == 0 and bits(s_g) == bits(s_g2) and bits(s_h) == bits(s_h2)
    acc = q_g.astype(np.int64) @ q_h.astype(np.int64)
    c = np.float32(np.float32(s_g) * np.float32(s_h)) * np.float32(1.0 / b)
    want = (acc.astype(np.float32) * np.float32(c)).astype(np.float32)
    assert np.array_equal(dx, want)


def test_dx_wht_reduces_error_on_heavy_tails(orc, syn):
    """§3.2 "int8 computation": the rotation along the contraction flattens
    outliers.  On heavy-tailed gradients the rotated dX is closer to the
    fp64 product dY * W^ than the plain int8 dX; on Gaussian gradients both
    stay at the LSQ noise floor."""
    M, N, K = 512, 512, 256
    w = syn.normal((N, K), 0.02, tag=316)
    qw, _, sw, _, _ = orc.quantize_lsq(w, per_row=True)
    what = sw.astype(np.float64)[:, None] * qw.astype(np.float64)
    for tag, dy, heavy in ((317, syn.student_t3((M, N), 1e-3, tag=317), True),
                           (318, syn.normal((M, N), 1e-3, tag=318), False)):
        ref = dy.astype(np.float64) @ what
        q_g, _, s_g, _, _ = orc.quantize_lsq(dy, col_mul=sw)
        plain = orc.qgemm_bwd_dx(q_g, s_g, qw)
        rot, _, _, _ = orc.qgemm_bwd_dx_wht(dy, sw, qw, 128)
        e0 = np.linalg.norm(plain - ref) / np.linalg.norm(ref)
        e1 = np.linalg.norm(rot - ref) / np.linalg.norm(ref)
        if heavy:
            assert e1 < 0.7 * e0 and e1 < 0.07, (e0, e1)
        else:
            assert e0 < 0.06 and e1 < 0.07, (e0, e1)


# --------------------------------------------------------------------------
# attention forward with an int8 P.V product
# --------------------------------------------------------------------------
def _bf16(a):
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _wide(h):
    return (h.astype(np.uint32) << 16).view(np.float32)


def test_exp_f_within_bound(orc):
    """The softmax's binary32 exp: within 2 ulp of e^x over the normal
    range, exact at 0, 0 below the range, monotone."""
    xs = np.linspace(-87.0, 0.0, 40001).astype(np.float32)
    got = np.array([orc.exp_f(float(x)) for x in xs], np.float32)
    ref = np.exp(xs.astype(np.float64))
    assert np.all(np.abs(got - ref) <= 2 * np.spacing(ref.astype(np.float32)))
    assert np.all(np.diff(got) >= 0)
    assert orc.exp_f(0.0) == 1.0 and orc.exp_f(-np.inf) == 0.0 and orc.exp_f(-104.5) == 0.0
    for kk in (-1, -10, -60):  # near x = k ln 2 the reduction leaves r ~ 0
        x = np.float32(kk * math.log(2))
        assert abs(float(orc.exp_f(float(x))) / math.exp(float(x)) - 1) < 2 ** -23


@pytest.mark.parametrize("Hq,Hkv,T,d,window", [(4, 1, 256, 128, None), (2, 2, 192, 64, 64),
                                               (4, 2, 128, 128, 100)])
def test_attn_fp64_bound(orc, Hq, Hkv, T, d, window):
    """Against fp64 softmax attention on the same bf16 inputs: only the int8
    P.V product is coarse (codes of P in [0, 127], of V per 64-key block)."""
    rng = np.random.default_rng(Hq * 100 + T)
    q = _bf16(rng.standard_normal((Hq, T, d)))
    k = _bf16(rng.standard_normal((Hkv, T, d)))
    v = _bf16(rng.standard_normal((Hkv, T, d)))
    o, fl = orc.attn_fwd(q, k, v, window)
    Q, K, V = (_wide(a).astype(np.float64) for a in (q, k, v))
    w = T if window is None else window
    i, j = np.meshgrid(np.arange(T), np.arange(T), indexing="ij")
    vis = (j <= i) & (j > i - w)
    ref = np.empty_like(o, dtype=np.float64)
    for h in range(Hq):
        S = Q[h] @ K[h // (Hq // Hkv)].T / math.sqrt(d)
        S[~vis] = -np.inf
        P = np.exp(S - S.max(1, keepdims=True))
        ref[h] = (P / P.sum(1, keepdims=True)) @ V[h // (Hq // Hkv)]
    assert fl == 0
    assert np.linalg.norm(o - ref) / np.linalg.norm(ref) < 0.03


def test_attn_window_one_closed_form(orc):
    """window = 1: each query sees only its own key, p = 1, l = 1, so
    o = fl(fl(127 * qv) * fl(s_p * s_v)) with s_p = fl(1 * fl(1/127)) and the
    V block's own absmax step (numpy binary32 arithmetic)."""
    rng = np.random.default_rng(3)
    T, d = 128, 64
    q = _bf16(rng.standard_normal((1, T, d)))
    k = _bf16(rng.standard_normal((1, T, d)))
    v = _bf16(rng.standard_normal((1, T, d)))
    o, _ = orc.attn_fwd(q, k, v, 1)
    f = np.float32
    inv127 = f(1) / f(127)
    sp = f(1) * inv127
    V = _wide(v)[0]
    want = np.empty((T, d), np.float32)
    for b in range(T // 64):
        blk = V[64 * b:64 * b + 64]
        sv = f(np.abs(blk).max()) * inv127
        qv = np.clip(np.rint(blk * (f(1) / sv)), -127, 127)
        assert np.rint(f(1) * (f(1) / sp)) == 127
        want[64 * b:64 * b + 64] = (f(127) * qv.astype(np.float32)) * (sp * sv)
    assert np.array_equal(o[0], want)


def test_attn_uniform_closed_form(orc):
    """q = 0: every visible logit is 0, p = 1, the rescale factor is 1, and
    o is the running sum of each block's dequantised integer product over
    the visible keys divided by their count (numpy binary32, same order)."""
    rng = np.random.default_rng(4)
    T, d = 192, 64
    q = np.zeros((1, T, d), np.uint16)
    k = _bf16(rng.standard_normal((1, T, d)))
    v = _bf16(rng.integers(-3, 4, size=(1, T, d)).astype(np.float32))
    o, _ = orc.attn_fwd(q, k, v)
    f = np.float32
    inv127 = f(1) / f(127)
    sp = f(1) * inv127
    V = _wide(v)[0]
    want = np.empty((T, d), np.float32)
    for i in range(T):
        acc = np.zeros(d, np.float32)
        for b in range(i // 64 + 1):
            blk = V[64 * b:64 * b + 64]
            sv = f(np.abs(blk).max()) * inv127
            qv = np.clip(np.rint(blk * (f(1) / sv)), -127, 127).astype(np.int64)
            hi = min(64, i - 64 * b + 1)
            s32 = 127 * qv[:hi].sum(0)
            acc = acc * f(1) + s32.astype(np.float32) * (sp * sv)
        want[i] = acc * (f(1) / f(i + 1))
    assert np.array_equal(o[0], want)


def test_attn_gqa_mapping(orc):
    """Query head h reads key/value head h / (Hq / Hkv)."""
    rng = np.random.default_rng(5)
    Hq, Hkv, T, d = 4, 2, 128, 64
    q = _bf16(rng.standard_normal((Hq, T, d)))
    k = _bf16(rng.standard_normal((Hkv, T, d)))
    v = _bf16(rng.standard_normal((Hkv, T, d)))
    o, _ = orc.attn_fwd(q, k, v, 80)
    for h in range(Hq):
        g = h // 2
        o1, _ = orc.attn_fwd(q[h:h + 1], k[g:g + 1], v[g:g + 1], 80)
        assert np.array_equal(o[h], o1[0])
