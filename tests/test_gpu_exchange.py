"""GPU parity of the deterministic gradient exchange (brq_dp_reduce) with the
oracle: the ascending-rank shard sum (App. A.2), TreeFold over replicas
(App. A.1) and the reciprocal averages (App. A.3), bit for bit, on ragged
lengths, order-sensitive vectors, the subnormal band, in place, and at one
rank's full share of the Open-1B gradient (sampled outputs)."""
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
N_RAGGED = 4096 * 5 + 1664 + 3


@pytest.fixture(scope="module")
def brq():
    import bitwise_reproducible_int8_amd as m
    m.lib()
    return m


def _dev(arrs):
    from tests.gpu_util import to_dev
    return [to_dev(a) for a in arrs]


def _run(brq, parts, R, S, A, average=True):
    flags = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    out = brq.dp_reduce(_dev(parts), R, S, A, average=average, flags=flags)
    torch.cuda.synchronize()
    return out, int(flags.item())


@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("S,A", [(1, 1), (2, 1), (3, 1), (8, 1), (3, 2), (1, 4)])
def test_dp_reduce_vs_oracle(brq, orc, syn, R, S, A):
    from tests.gpu_util import assert_bitwise
    parts = syn.exchange_parts(R * S * A, N_RAGGED)
    for average in (True, False):
        want, wfl = orc.dp_reduce(parts, R, S, A, average=average)
        got, gfl = _run(brq, parts, R, S, A, average)
        assert_bitwise(got, want, f"dp_reduce R={R} S={S} A={A} average={average}")
        assert gfl == wfl == 0


@pytest.mark.parametrize("R,S,A", [(64, 1, 1), (1, 64, 1), (1, 1, 64), (6, 8, 1), (4, 4, 4),
                                   (11, 5, 1), (31, 2, 1)])
def test_dp_reduce_large_counts(brq, orc, syn, R, S, A):
    from tests.gpu_util import assert_bitwise
    parts = syn.exchange_parts(R * S * A, 1027)
    want, _ = orc.dp_reduce(parts, R, S, A)
    got, _ = _run(brq, parts, R, S, A)
    assert_bitwise(got, want, f"dp_reduce R={R} S={S} A={A}")


def _golden():
    rows = []
    with open(os.path.join(GOLDEN, "exchange_vectors.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            kind, want, leaves, _ = (p.strip() for p in line.split(";", 3))
            if kind in ("ascending", "treefold"):
                rows.append((kind, float(want), [float(t) for t in leaves.split()]))
    return rows


@pytest.mark.parametrize("row", _golden(), ids=lambda r: f"{r[0]}-{len(r[2])}")
def test_dp_reduce_golden_vectors(brq, row):
    kind, want, leaves = row
    parts = [np.full(5, v, np.float32) for v in leaves]
    P = len(parts)
    R, S = (1, P) if kind == "ascending" else (P, 1)
    got, _ = _run(brq, parts, R, S, 1, average=False)
    g = got.cpu().numpy()
    assert np.all(g.view(np.uint32) == np.float32(want).view(np.uint32)), (kind, leaves, g)


def test_dp_reduce_subnormal_band_and_signed_zero(brq, orc, syn):
    from tests.gpu_util import assert_bitwise
    rng = np.random.default_rng(5)
    P = 12
    # magnitudes around 2^-126: inputs and sums fall in and out of the
    # subnormal range; some entries are exact negatives of each other
    parts = [(rng.standard_normal(N_RAGGED) * np.float32(2.0 ** -125)).astype(np.float32)
             for _ in range(P)]
    parts[3][:100] = -parts[2][:100]
    parts[0][100:200] = -0.0
    parts[5][200:300] = np.float32(2.0 ** -140)  # subnormal input reads as zero
    for R, S in ((3, 4), (12, 1), (1, 12), (2, 6)):
        for average in (True, False):
            want, _ = orc.dp_reduce(parts, R, S, 1, average=average)
            got, _ = _run(brq, parts, R, S, 1, average)
            assert_bitwise(got, want, f"subnormal band R={R} S={S} average={average}")
    zeros = [np.full(7, -0.0, np.float32) for _ in range(3)]
    got, _ = _run(brq, zeros, 3, 1, 1, average=False)
    assert np.all(got.cpu().numpy().view(np.uint32) == 0x80000000)


def test_dp_reduce_nonfinite_flag(brq, orc):
    parts = [np.ones(99, np.float32) for _ in range(4)]
    parts[2][17] = np.inf
    got, fl = _run(brq, parts, 2, 2, 1)
    want, wfl = orc.dp_reduce(parts, 2, 2, 1)
    assert fl == wfl == 1
    assert np.isinf(got.cpu().numpy()[17])


def test_dp_reduce_nan_inputs_flagged(brq, orc):
    """A NaN contribution (quiet or signalling) gives a NaN output and the
    non-finite flag on both sides, also where every count is one (no add
    and, with average, only multiplies by one); the payload bits of a NaN
    are not compared."""
    nan_bits = np.array([0x7FC00000, 0x7F800001, 0xFFC12345, 0x7FA00000], np.uint32)
    for R, S in ((1, 1), (1, 2), (2, 1), (3, 3)):
        parts = [np.full(37, 0.25 * (j + 1), np.float32) for j in range(R * S)]
        for k, b in enumerate(nan_bits):
            parts[k % (R * S)][5 + k] = b.view(np.float32)
        for average in (True, False):
            want, wfl = orc.dp_reduce(parts, R, S, 1, average=average)
            got, gfl = _run(brq, parts, R, S, 1, average)
            g = got.cpu().numpy()
            assert gfl == wfl == 1
            assert np.array_equal(np.isnan(g), np.isnan(want))
            finite = ~np.isnan(want)
            assert np.array_equal(g[finite].view(np.uint32), want[finite].view(np.uint32))


def test_dp_reduce_in_place_and_repeat(brq, orc, syn):
    from tests.gpu_util import assert_bitwise
    parts = syn.exchange_parts(6, N_RAGGED)
    want, _ = orc.dp_reduce(parts, 3, 2, 1)
    d = _dev(parts)
    for k in range(3):  # same bits on every call
        o = brq.dp_reduce(d, 3, 2, 1)
        torch.cuda.synchronize()
        assert_bitwise(o, want, f"repeat {k}")
    brq.dp_reduce(d, 3, 2, 1, out=d[0])  # out aliases the first contribution
    torch.cuda.synchronize()
    assert_bitwise(d[0], want, "in place")


def test_dp_reduce_argument_errors(brq):
    import ctypes as C
    L = brq.lib()
    x = torch.zeros(64, dtype=torch.float32, device="cuda:0")
    ptrs = (C.c_void_p * 65)(*([x.data_ptr()] * 65))
    assert L.brq_dp_reduce(ptrs, 65, 1, 1, 64, 1, x.data_ptr(), None, None) == -5
    assert L.brq_dp_reduce(ptrs, 0, 1, 1, 64, 1, x.data_ptr(), None, None) == -9
    assert L.brq_dp_reduce(ptrs, 2, 1, 1, -1, 1, x.data_ptr(), None, None) == -3
    assert L.brq_dp_reduce(None, 2, 1, 1, 64, 1, x.data_ptr(), None, None) == -1
    bad = (C.c_void_p * 2)(x.data_ptr(), x.data_ptr() + 4)
    assert L.brq_dp_reduce(bad, 2, 1, 1, 8, 1, x.data_ptr(), None, None) == -4
    # n == 0 launches nothing and succeeds
    assert L.brq_dp_reduce(ptrs, 2, 1, 1, 0, 1, x.data_ptr(), None, None) == 0


@pytest.fixture(scope="module")
def rank_share(syn):
    """One rank's share of the Open-1B gradient after the all-to-all: the
    grad-norm vector viewed as 8 contributions of 201.25e6 fp32 values."""
    v = syn.normal((syn.GRAD_NORM_N,), 1e-4, tag=syn.TAG_V)
    return v.reshape(8, -1)


def _sampled(rng, n):
    idx = np.concatenate([np.arange(4099), n - 4099 + np.arange(4099),
                          rng.integers(0, n, 65536)])
    return np.unique(idx)


@pytest.mark.parametrize("R,S,n", [(1, 8, 201_250_000), (6, 1, 201_250_000),
                                   (6, 8, 33_541_664)])
def test_dp_reduce_full_share_sampled(brq, orc, rank_share, R, S, n):
    """The bench's launches: the reduce-scatter's ascending sum over 8
    shards of 201.25e6 values, the replica fold over 6 of them, and the
    audit replay of 6 replicas x 8 shards over 33.5e6 values each; outputs
    at 73,000 sampled indices (both ends included) against the oracle."""
    flat = rank_share.reshape(-1)
    P = R * S
    host = [flat[j * n:(j + 1) * n] for j in range(P)]
    V = torch.from_numpy(flat[:P * n]).to("cuda:0")
    parts = [V[j * n:(j + 1) * n] for j in range(P)]
    out = brq.dp_reduce(parts, R, S, 1)
    torch.cuda.synchronize()
    idx = _sampled(np.random.default_rng(R * 10 + S), n)
    want, fl = orc.dp_reduce([h[idx] for h in host], R, S, 1)
    got = out[torch.from_numpy(idx).to("cuda:0")].cpu().numpy()
    assert fl == 0
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), \
        f"R={R} S={S}: {int((got.view(np.uint32) != want.view(np.uint32)).sum())} differ"
    del V, parts, out
    torch.cuda.empty_cache()
