"""Pins of the oracle's deterministic gradient exchange (Open-1B report,
App. A: A.1 TreeFold over replicas, A.2 the ascending-rank shard sum, A.3
averages as reciprocal multiplies) against values fixed outside it:
hand-derived vectors (tests/golden/exchange_vectors.txt), a message-passing
simulation of the cluster's recursive-doubling all-reduce in exact rational
arithmetic (tests/_exact.py), closed forms on powers of two and integer
inputs, and fp64 bounds.
"""
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

from tests import _exact as X

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(f):
    return struct.unpack("<I", struct.pack("<f", float(f)))[0]


def _val(tok):
    if tok.startswith("0x"):
        return X.bits_to_float(int(tok, 16))
    return float(tok)


def _golden():
    rows = []
    with open(os.path.join(GOLDEN, "exchange_vectors.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            kind, want, leaves, _why = (p.strip() for p in line.split(";", 3))
            rows.append((kind, _val(want), [_val(t) for t in leaves.split()]))
    return rows


def _cols(values):
    return [np.array([v], np.float32) for v in values]


@pytest.mark.parametrize("row", _golden(), ids=lambda r: f"{r[0]}-{len(r[2])}")
def test_exchange_golden(orc, row):
    kind, want, leaves = row
    if kind == "ascending":
        got = orc.ascending_sum(_cols(leaves))[0]
    elif kind == "treefold":
        got = orc.treefold(_cols(leaves))[0]
    elif kind == "average3":
        got = orc.average(np.array(leaves, np.float32), 3)[0]
    else:
        raise AssertionError(kind)
    assert _bits(got) == _bits(want), (kind, leaves, got, want)


# --------------------------------------------------------------------------
# TreeFold against a simulated recursive-doubling all-reduce
# --------------------------------------------------------------------------
def _recursive_doubling(vals):
    """The cluster's all-reduce as message passing between len(vals) ranks,
    in exact rationals rounded to binary32 after every add (App. A.1, §5):
    a power-of-two group runs log2 hops, at hop k rank r adds the value of
    rank r ^ 2^k with the lower rank's value on the left; a group that is
    not a power of two splits into its largest power-of-two block and the
    remainder, each reduced the same way, and the two are combined (block
    on the left) and broadcast.  Returns every rank's final value."""
    n = len(vals)
    if n & (n - 1) == 0:
        cur = list(vals)
        k = 1
        while k < n:
            nxt = []
            for r in range(n):
                p = r ^ k
                lo, hi = (cur[r], cur[p]) if r < p else (cur[p], cur[r])
                nxt.append(X.op(lo + hi))
            cur = nxt
            k *= 2
        return cur
    p = 1
    while p * 2 < n:
        p *= 2
    a = _recursive_doubling(vals[:p])
    b = _recursive_doubling(vals[p:])
    s = X.op(a[0] + b[0])
    return [s] * n


def _rand_binary32(rng, n):
    """Values with assorted exponents and signs, exact as binary32."""
    m = rng.integers(1, 2 ** 24, size=n)
    e = rng.integers(-30, 10, size=n)
    s = rng.choice([-1, 1], size=n)
    return [Fraction(int(s[i] * m[i])) * Fraction(2) ** int(e[i] - 23) for i in range(n)]


@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 6, 7, 8, 11, 16, 24, 31, 48, 64])
def test_treefold_equals_recursive_doubling(orc, R):
    rng = np.random.default_rng(1000 + R)
    for _ in range(20):
        vals = _rand_binary32(rng, R)
        ranks = _recursive_doubling(vals)
        assert all(v == ranks[0] for v in ranks), "ranks disagree"
        got = orc.treefold(_cols([float(v) for v in vals]))[0]
        assert _bits(got) == _bits(float(ranks[0])), (R, got, float(ranks[0]))


@pytest.mark.parametrize("R", [1, 2, 4, 8, 16, 32, 64])
def test_treefold_power_of_two_is_the_pairwise_tree(orc, R):
    """For a power-of-two replica count the binary-carry fold is the
    balanced pairwise tree (App. A.1: depth log2 dp_replicate), which the
    canonical tree routine computes by another coding."""
    rng = np.random.default_rng(R)
    v = (rng.standard_normal((R, 257)) * np.exp2(rng.integers(-20, 20, (R, 257)))).astype(np.float32)
    got = orc.treefold(list(v))
    want = np.array([orc.tree_sum(v[:, i]) for i in range(v.shape[1])], np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


# --------------------------------------------------------------------------
# reciprocal averages (App. A.3)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("k", [2, 3, 5, 6, 7, 8, 12, 48])
def test_average_is_reciprocal_multiply_within_one_ulp_of_quotient(orc, k):
    rng = np.random.default_rng(k)
    x = (rng.standard_normal(4096) * np.exp2(rng.integers(-40, 40, 4096))).astype(np.float32)
    got = orc.average(x, k)
    inv = X.op(Fraction(1, k))
    quot = (x / np.float32(k)).astype(np.float32)  # correctly rounded division
    diff = 0
    for i in range(0, 4096, 7):
        want = X.op(Fraction(float(x[i])) * inv)
        assert _bits(got[i]) == _bits(float(want)), (k, x[i])
        d = abs(int(got[i].view(np.int32)) - int(quot[i].view(np.int32)))
        assert d <= 1, "a reciprocal multiply is within one ulp of the quotient"
        diff += d
    if k & (k - 1) == 0:
        assert diff == 0 and np.array_equal(got, quot), "exact for powers of two"
    else:
        assert diff > 0, "the page's claim: some quotients differ"


# --------------------------------------------------------------------------
# the whole exchange
# --------------------------------------------------------------------------
def test_dp_reduce_mesh_order_is_replica_major(orc):
    # R=2, S=2: replica 0 holds parts 0,1; replica 1 parts 2,3 (App. A:
    # virtual ranks in replica-major, shard-minor order).  Replica sums 2 and
    # 2^24 give 2^24+2; a shard-major split would give (1+2^24 -> 2^24) +
    # (1+0) -> 2^24.
    out, fl = orc.dp_reduce(_cols([1, 1, 16777216, 0]), 2, 2, 1, average=False)
    assert out[0] == 16777218.0 and fl == 0


def test_dp_reduce_microbatches_innermost(orc):
    # R=1, S=2, A=2: shard 0's microbatches (2^24, 1) sum to 2^24, shard 1's
    # (1, 1) to 2; inner = 2^24 + 2.
    out, _ = orc.dp_reduce(_cols([16777216, 1, 1, 1]), 1, 2, 2, average=False)
    assert out[0] == 16777218.0


@pytest.mark.parametrize("R,S,A", [(1, 1, 1), (2, 4, 1), (4, 2, 2), (8, 8, 1), (2, 2, 16),
                                   (1, 64, 1), (64, 1, 1)])
def test_dp_reduce_integer_inputs_power_of_two_counts_exact(orc, R, S, A):
    """Integer inputs keep every partial sum exact, and reciprocals of
    powers of two are exact: the output is the exact mean."""
    rng = np.random.default_rng(R * 100 + S * 10 + A)
    parts = rng.integers(-1000, 1000, (R * S * A, 333)).astype(np.float32)
    out, fl = orc.dp_reduce(list(parts), R, S, A)
    want = parts.astype(np.float64).mean(axis=0)
    assert fl == 0 and np.array_equal(out.astype(np.float64), want)


@pytest.mark.parametrize("R,S,A", [(3, 5, 1), (6, 8, 1), (5, 3, 3), (7, 1, 1), (1, 7, 1),
                                   (1, 1, 7), (2, 3, 2)])
def test_dp_reduce_fp64_bound(orc, R, S, A):
    """Each output is within the rounding-error bound of the exact mean:
    (A - 1) + (S - 1) + ceil(log2 R) adds and three reciprocal multiplies,
    each off by at most one unit roundoff relative to its own magnitude."""
    rng = np.random.default_rng(R * 31 + S * 7 + A)
    parts = (rng.standard_normal((R * S * A, 2000)) * 1e-3).astype(np.float32)
    out, fl = orc.dp_reduce(list(parts), R, S, A)
    exact = parts.astype(np.float64).mean(axis=0)
    steps = (A - 1) + (S - 1) + math.ceil(math.log2(R)) + 6
    bound = steps * 2.0 ** -24 * np.abs(parts.astype(np.float64)).mean(axis=0) * 1.01
    assert fl == 0 and np.all(np.abs(out.astype(np.float64) - exact) <= bound)


def test_dp_reduce_exact_rational_emulation(orc):
    """The exchange in exact rationals, each add and multiply rounded once."""
    rng = np.random.default_rng(7)
    R, S, A = 5, 3, 2
    vals = [_rand_binary32(rng, 16) for _ in range(R * S * A)]
    parts = [np.array([float(v) for v in p], np.float32) for p in vals]
    out, _ = orc.dp_reduce(parts, R, S, A)
    inv = {k: X.op(Fraction(1, k)) for k in (A, S, R)}
    for i in range(16):
        reps = []
        for r in range(R):
            inner = None
            for s in range(S):
                acc = vals[(r * S + s) * A][i]
                for a in range(1, A):
                    acc = X.op(acc + vals[(r * S + s) * A + a][i])
                acc = X.op(acc * inv[A])
                inner = acc if inner is None else X.op(inner + acc)
            reps.append(X.op(inner * inv[S]))
        want = X.op(_recursive_doubling(reps)[0] * inv[R])
        assert _bits(out[i]) == _bits(float(want)), i


def test_dp_reduce_subnormal_inputs_and_flags(orc):
    tiny = X.bits_to_float(0x00000005)
    out, fl = orc.dp_reduce(_cols([tiny, -tiny, 1.0, 2.0]), 2, 2, 1, average=False)
    assert out[0] == 3.0 and fl == 0
    # a subnormal sum flushes: 2^-126 - 2^-126*(1-2^-23) is subnormal
    a, b = X.bits_to_float(0x00800001), X.bits_to_float(0x00800000)
    out, _ = orc.dp_reduce(_cols([a, -b]), 1, 2, 1, average=False)
    assert out[0] == 0.0
    out, fl = orc.dp_reduce(_cols([3e38, 3e38]), 2, 1, 1, average=False)
    assert math.isinf(out[0]) and fl == 1
    with pytest.raises(ValueError):
        orc.dp_reduce(_cols([1.0] * 65), 65, 1, 1)
