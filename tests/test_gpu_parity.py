"""GPU parity, small and ragged shapes: every libbrq entry point through the
C ABI against the CPU oracle, bit for bit, across launch geometries.

Shapes span several tiles and leave ragged tails; tune settings sweep the
GEMM kernel (reference / three MFMA tilings), split-K, the reduction chunk
size and the RMSNorm backward block height.  Outputs must be identical for
every setting.
"""
import sys

import numpy as np
import pytest
import torch

import brq_synth as syn
import oracle as orc
from tests.gpu_util import DEV, assert_bitwise, codes, sha, to_dev, to_np

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


# --------------------------------------------------------------------------
# quantize_lsq
# --------------------------------------------------------------------------
QUANT_CASES = [
    ((64, 256), False, None),      # tiny activation, fp32
    ((100, 264), True, None),      # ragged rows, bf16
    ((257, 520), False, None),     # ragged everything, fp32
    ((300, 512), True, "cm"),      # bf16 with a per-column multiplier
    ((64, 256), False, "cm"),
]


@pytest.mark.parametrize("shape,bf16,cm", QUANT_CASES)
@pytest.mark.parametrize("chunk", [0, 10, 12, 15])
def test_quantize_per_tensor(shape, bf16, cm, chunk):
    say("quantize_per_tensor", shape, bf16, cm, chunk)
    x = syn.normal(shape, 1.0, tag=201, bf16=bf16)
    col = syn.normal((shape[1],), 0.01, mean=0.02, tag=202) if cm else None
    q, qt, s, amax, fl = orc.quantize_lsq(x, col_mul=col, want_t=(shape[0] % 16 == 0 and shape[1] % 16 == 0))
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    gq, gqt, gs, gamax = brq.quantize_lsq(to_dev(x), col_mul=None if col is None else to_dev(col),
                                          want_t=qt is not None, tune={"chunk_log2": chunk},
                                          flags=flags)
    assert_bitwise(gq, q, "q")
    assert_bitwise(gs, s, "scale")
    assert_bitwise(gamax, amax, "amax")
    if qt is not None:
        assert_bitwise(gqt, qt, "q_t")
    assert int(flags.item()) == fl == 0


@pytest.mark.parametrize("shape,bf16", [((256, 256), False), ((3072, 2048), True),
                                        ((48, 8192), True), ((16, 264), True), ((5, 16384), True),
                                        ((33, 100), False), ((64, 16384), True), ((32, 8192), False),
                                        ((16, 4096), True), ((8192, 2048), True), ((2048, 8192), True),
                                        ((512, 2048), True), ((48, 1024), False)])
def test_quantize_per_row(shape, bf16):
    say("quantize_per_row", shape, bf16)
    w = syn.normal(shape, 0.02, tag=203, bf16=bf16)
    want_t = shape[0] % 16 == 0 and shape[1] % 16 == 0
    q, qt, s, amax, fl = orc.quantize_lsq(w, per_row=True, want_t=want_t)
    gq, gqt, gs, gamax = brq.quantize_lsq(to_dev(w), per_row=True, want_t=want_t)
    assert_bitwise(gq, q, "q")
    assert_bitwise(gs, s, "scale")
    assert_bitwise(gamax, amax, "amax")
    if want_t:
        assert_bitwise(gqt, qt, "q_t")


def _rows_multi_check(shapes, tag):
    ws = []
    for k, (rows, cols, bf16) in enumerate(shapes):
        ws.append(syn.normal((rows, cols), 0.02, tag=tag + k, bf16=bf16))
    want_t = all(r % 16 == 0 and c % 16 == 0 for r, c, _ in shapes)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = brq.quantize_lsq_rows_multi([to_dev(w) for w in ws], want_t=want_t, flags=flags)
    for k, w in enumerate(ws):
        q, qt, s, amax, fl = orc.quantize_lsq(w, per_row=True, want_t=want_t)
        gq, gqt, gs, gamax = got[k]
        name = f"job {k} {shapes[k]}"
        assert_bitwise(gq, q, f"{name} q")
        assert_bitwise(gs, s, f"{name} scale")
        assert_bitwise(gamax, amax, f"{name} amax")
        if want_t:
            assert_bitwise(gqt, qt, f"{name} q_t")
    assert int(flags.item()) == 0


def test_quantize_rows_multi_layer_weights():
    """The seven Open-1B weights of a layer in one grouped call (two row
    width classes, one transpose launch) equal the per-row quantiser."""
    say("quantize_rows_multi layer weights")
    shapes = [(N, K, True) for _, K, N, _ in syn.LAYER_LINEARS]
    _rows_multi_check(shapes, 500)


@pytest.mark.parametrize("case", ["mixed", "many", "ragged"])
def test_quantize_rows_multi_edges(case):
    """Mixed element types and widths in one call, more tensors than one
    launch table holds, rows that are not a multiple of the 4 rows of a
    work-group, and an empty tensor among the jobs."""
    say("quantize_rows_multi", case)
    if case == "mixed":
        shapes = [(48, 1024, False), (32, 8192, True), (64, 272, True), (16, 16384, True),
                  (0, 512, True), (80, 2048, False), (16, 64, True)]
        _rows_multi_check(shapes, 540)
    elif case == "many":
        shapes = [(16 * (1 + k % 5), 64 * (1 + k % 7), k % 2 == 0) for k in range(37)]
        _rows_multi_check(shapes, 560)
    else:
        shapes = [(5, 64, True), (33, 136, True), (1, 8, True), (7, 1000, False), (3, 16384, True)]
        _rows_multi_check(shapes, 600)


def test_quantize_edge_cases():
    say("quantize_edge_cases")
    z = np.zeros((32, 64), np.float32)
    gq, _, gs, _ = brq.quantize_lsq(to_dev(z))
    assert not to_np(gq).any() and float(gs.item()) == 0.0
    gq, _, gs, _ = brq.quantize_lsq(to_dev(z), per_row=True)
    assert not to_np(gq).any() and not to_np(gs).any()
    # empty tensor: step size 0
    e = torch.empty((0, 64), dtype=torch.float32, device=DEV)
    _, _, gs, _ = brq.quantize_lsq(e)
    q, _, s, _, _ = orc.quantize_lsq(np.zeros((0, 64), np.float32))
    assert_bitwise(gs, s, "empty scale")
    # non-finite statistic raises the device flag, per-tensor and per-row
    bad = np.ones((16, 64), np.float32)
    bad[3, 5] = np.inf
    for per_row in (False, True):
        flags = torch.zeros(1, dtype=torch.int32, device=DEV)
        brq.quantize_lsq(to_dev(bad), per_row=per_row, flags=flags)
        assert int(flags.item()) == brq.FLAG_NONFINITE
    # subnormal inputs read as zero; +-0 keep sign semantics in codes
    sub = np.full((16, 64), 1.0, np.float32)
    sub[0, :16] = np.float32(1e-40)
    sub[1, :16] = -np.float32(1e-40)
    q, _, s, _, _ = orc.quantize_lsq(sub)
    gq, _, gs, _ = brq.quantize_lsq(to_dev(sub))
    assert_bitwise(gq, q, "q subnormal")
    assert_bitwise(gs, s, "s subnormal")


def _plant_ties(x, scale, per_row, cm, rng, pairs_per_group):
    """Turn level-1 leaf pairs (2i, 2i+1) of the |x| tree into (t, u) with
    fl(t * r) = k + 1/2 for a random k, and u = c - t exact where c is the
    pair's node fl(leaf_2i + leaf_2i+1): the node, and with it the tree sum
    and the step size, keep their bits, so the codes of the t values are
    exact ties.  Leaves are |x * cm[col]|; cm holds powers of two, so the
    leaf is |x| times cm exactly.  Returns the number of pairs changed."""
    rows, cols = x.shape
    mult = np.ones(cols, np.float32) if cm is None else cm
    planted = 0
    groups = range(rows) if per_row else [None]
    flat = x.reshape(-1)
    for g in groups:
        s = np.float32(scale[g if per_row else 0])
        r = np.float32(1) / s
        base = g * cols if per_row else 0
        n = cols if per_row else x.size
        for p in rng.choice(n // 2, size=min(pairs_per_group, n // 2), replace=False):
            i0 = base + 2 * p
            m0, m1 = mult[i0 % cols], mult[(i0 + 1) % cols]
            a, b = abs(flat[i0]) * m0, abs(flat[i0 + 1]) * m1
            c = np.float32(a + b)
            top = int(np.floor(float(c) * float(r) - 0.5))
            if top < 0:
                continue
            k = int(rng.integers(0, min(126, top) + 1))
            t0 = np.float32((k + 0.5) / float(r))
            found = None
            for d in range(-4, 5):
                t = t0
                for _ in range(abs(d)):
                    t = np.nextafter(t, np.float32(np.inf) if d > 0 else np.float32(-np.inf))
                if np.float32(t * r) == np.float32(k + 0.5) and t <= c:
                    u = np.float32(c - t)
                    if float(u) == float(c) - float(t) and np.float32(t + u) == c:
                        found = (t, u)
                        break
            if found is None:
                continue
            t, u = found
            sg = rng.choice([-1.0, 1.0], size=2).astype(np.float32)
            flat[i0] = sg[0] * t / m0
            flat[i0 + 1] = sg[1] * u / m1
            planted += 1
    return planted


def _count_ties(x, scale, per_row, cm):
    rows, cols = x.shape
    v = x * (np.ones(cols, np.float32) if cm is None else cm)[None, :]
    r = (np.float32(1) / np.asarray(scale, np.float32)).astype(np.float32)
    p = (v * (r[:, None] if per_row else r[0])).astype(np.float32)
    return int(np.sum(np.abs(p - np.trunc(p)) == np.float32(0.5)))


@pytest.mark.parametrize("mode", ["per_tensor", "per_row", "col_mul"])
def test_quantize_ties_and_clamps(mode):
    """Exact ties x*r = k + 1/2 (round half to even) that leave the step
    size's bits unchanged, plus clamps beyond +-127.5."""
    say("quantize_ties", mode)
    rng = np.random.default_rng(5)
    per_row = mode == "per_row"
    x = rng.standard_normal((64, 256)).astype(np.float32)
    x[10, :8] = np.float32(1000)  # clamps: in the tensor before its statistic
    x[11, 8:16] = np.float32(-1000)
    cm = np.exp2(rng.integers(-2, 3, 256)).astype(np.float32) if mode == "col_mul" else None
    _, _, s0, _, _ = orc.quantize_lsq(x, per_row=per_row, col_mul=cm)
    planted = _plant_ties(x, s0, per_row, cm, rng, 8 if per_row else 400)
    q, _, s, amax, fl = orc.quantize_lsq(x, per_row=per_row, col_mul=cm)
    assert np.array_equal(np.asarray(s).view(np.uint32), np.asarray(s0).view(np.uint32)), \
        "planting must keep the step size"
    ties = _count_ties(x, s, per_row, cm)
    assert planted >= 100 and ties >= 100, (planted, ties)
    assert np.any(np.abs(q) == 127)
    gq, _, gs, gamax = brq.quantize_lsq(to_dev(x), per_row=per_row,
                                        col_mul=None if cm is None else to_dev(cm))
    assert_bitwise(gq, q, f"q ties {mode}")
    assert_bitwise(gs, s, f"s ties {mode}")
    assert_bitwise(gamax, amax, f"amax ties {mode}")


# --------------------------------------------------------------------------
# GEMMs
# --------------------------------------------------------------------------
GEMM_TUNES = [dict(gemm_kernel=k, split_k=s) for k, s in
              [(1, 1), (2, 1), (3, 1), (4, 1), (2, 2), (2, 4), (3, 2), (4, 4),
               (5, 1), (6, 1), (7, 1), (8, 1), (7, 2), (5, 4), (0, 0),
               (9, 1), (10, 1), (11, 1), (12, 1), (10, 2), (12, 4), (10, 16), (0, 8),
               (13, 1), (13, 2), (13, 4), (14, 1), (14, 2), (14, 4)]]


@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (200, 300, 2048), (128, 512, 16),
                                   (333, 515, 1152), (1, 1, 64), (256, 512, 256),
                                   (1024, 2048, 128)])
def test_qgemm_fwd(M, N, K):
    say("qgemm_fwd", M, N, K)
    rng = np.random.default_rng(M * 7 + N)
    qx, qw = codes(rng, (M, K)), codes(rng, (N, K))
    sx = np.array([0.0173], np.float32)
    sw = (np.abs(rng.standard_normal(N)) * 1e-3 + 1e-4).astype(np.float32)
    want = orc.qgemm_fwd(qx, sx, qw, sw)
    want_pt = orc.qgemm_fwd(qx, sx, qw, sw[:1])
    dqx, dqw, dsx, dsw = to_dev(qx), to_dev(qw), to_dev(sx), to_dev(sw)
    for t in GEMM_TUNES:
        assert_bitwise(brq.qgemm_fwd(dqx, dsx, dqw, dsw, tune=t), want, f"y {t}")
    assert_bitwise(brq.qgemm_fwd(dqx, dsx, dqw, dsw[:1]), want_pt, "y per-tensor w")


@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (160, 336, 528), (256, 2048, 64)])
def test_qgemm_bwd_dx(M, N, K):
    say("qgemm_bwd_dx", M, N, K)
    rng = np.random.default_rng(N)
    qg, qw = codes(rng, (M, N)), codes(rng, (N, K))
    sg = np.array([3.1e-5], np.float32)
    want = orc.qgemm_bwd_dx(qg, sg, qw)
    dqg, dqwt, dsg = to_dev(qg), to_dev(np.ascontiguousarray(qw.T)), to_dev(sg)
    for t in GEMM_TUNES:
        assert_bitwise(brq.qgemm_bwd_dx(dqg, dsg, dqwt, tune=t), want, f"dx {t}")


@pytest.mark.parametrize("M,N,K,split", [(8200, 4000, 256, 1), (4100, 4001, 320, 1),
                                         (8200, 4000, 512, 2), (2304, 2560, 1024, 4),
                                         (8200, 4000, 192, 1), (8200, 4000, 1024, 1),
                                         (8200, 4001, 1088, 1)])
def test_qgemm_persistent_many_tiles(M, N, K, split):
    """The persistent kernel with more tiles than CUs: several tiles per
    work-group, the load pipeline crossing tile boundaries, column scales
    double-buffered per tile, ragged right and bottom edges; 4 contraction
    steps per tile is the kernel's minimum, 3 takes the one-tile-per-group
    kernel.  Sampled rows (every tile-row boundary and the ragged tail)
    against the oracle."""
    say("qgemm_persistent", M, N, K, split)
    rng = np.random.default_rng(M + N + K)
    qx, qw = codes(rng, (M, K)), codes(rng, (N, K))
    sx = np.array([0.0173], np.float32)
    sw = (np.abs(rng.standard_normal(N)) * 1e-3 + 1e-4).astype(np.float32)
    rows = sorted(set([0, 1, M - 1] + [r for b in range(256, M, 256) for r in (b - 1, b)]
                      + list(rng.integers(0, M, 24))))
    t = dict(gemm_kernel=13, split_k=split)
    dqx, dqw, dsx, dsw = to_dev(qx), to_dev(qw), to_dev(sx), to_dev(sw)
    y = to_np(brq.qgemm_fwd(dqx, dsx, dqw, dsw, tune=t))
    assert_bitwise(y[rows], orc.qgemm_fwd(qx[rows], sx, qw, sw), f"y rows {t}")
    y1 = to_np(brq.qgemm_fwd(dqx, dsx, dqw, dsw[:1], tune=t))
    assert_bitwise(y1[rows], orc.qgemm_fwd(qx[rows], sx, qw, sw[:1]), f"y per-tensor rows {t}")
    # the same codes as an input-gradient GEMM (uniform scale): q_g [M][K'],
    # q_w^T [N'][K'] with K' = K the contraction
    sg = np.array([3.1e-5], np.float32)
    dx = to_np(brq.qgemm_bwd_dx(dqx, to_dev(sg), dqw, tune=t))
    assert_bitwise(dx[rows], orc.qgemm_bwd_dx(qx[rows], sg, np.ascontiguousarray(qw.T)),
                   f"dx rows {t}")


BF16_TUNES = [dict(gemm_kernel=k, split_k=s) for k, s in
              [(0, 0), (1, 1), (2, 1), (2, 4), (7, 1), (10, 1), (10, 4), (12, 1), (13, 1), (13, 2)]]


@pytest.mark.parametrize("M,N,K", [(200, 300, 2048), (333, 515, 1152), (1024, 2048, 128),
                                   (256, 512, 256), (1, 1, 64)])
def test_qgemm_bf16_outputs(M, N, K):
    """bf16-output variant: each output is the fp32 result rounded once."""
    say("qgemm bf16 outputs", M, N, K)
    rng = np.random.default_rng(M + 3 * N + K)
    qx, qw = codes(rng, (M, K)), codes(rng, (N, K))
    sx = np.array([0.0173], np.float32)
    sw = (np.abs(rng.standard_normal(N)) * 1e-3 + 1e-4).astype(np.float32)
    sg = np.array([3.1e-5], np.float32)
    want_y = orc.to_bf16(orc.qgemm_fwd(qx, sx, qw, sw))
    want_dx = orc.to_bf16(orc.qgemm_bwd_dx(qx, sg, np.ascontiguousarray(qw.T)))
    dqx, dqw, dsx, dsw, dsg = to_dev(qx), to_dev(qw), to_dev(sx), to_dev(sw), to_dev(sg)
    for t in BF16_TUNES:
        assert_bitwise(brq.qgemm_fwd(dqx, dsx, dqw, dsw, tune=t, out_dtype=torch.bfloat16),
                       want_y, f"y bf16 {t}")
        assert_bitwise(brq.qgemm_bwd_dx(dqx, dsg, dqw, tune=t, out_dtype=torch.bfloat16),
                       want_dx, f"dx bf16 {t}")


def test_qgemm_bf16_outputs_many_tiles():
    M, N, K = 8200, 4001, 1088
    say("qgemm bf16 outputs many tiles", M, N, K)
    rng = np.random.default_rng(5)
    qx, qw = codes(rng, (M, K)), codes(rng, (N, K))
    sx = np.array([0.0173], np.float32)
    sw = (np.abs(rng.standard_normal(N)) * 1e-3 + 1e-4).astype(np.float32)
    rows = sorted(set([0, M - 1] + [r for b in range(256, M, 256) for r in (b - 1, b)]))
    for t in (dict(gemm_kernel=13, split_k=1), dict(gemm_kernel=10, split_k=1), None):
        y = to_np(brq.qgemm_fwd(to_dev(qx), to_dev(sx), to_dev(qw), to_dev(sw), tune=t,
                                out_dtype=torch.bfloat16))
        assert_bitwise(y[rows], orc.to_bf16(orc.qgemm_fwd(qx[rows], sx, qw, sw)), f"y rows {t}")


def test_gemm_extreme_accumulator():
    """Codes of magnitude 127 and 128 at the int32 bound of the contraction
    (128 * 128 * K < 2^31)."""
    say("gemm_extreme")
    K = 131056  # the largest multiple of 16 <= 131071
    qx = np.full((3, K), 127, np.int8)
    qx[1] = -127
    qx[2] = -128
    qw = np.full((3, K), 127, np.int8)
    qw[2] = -128
    one = np.ones(1, np.float32)
    want = orc.qgemm_fwd(qx, one, qw, np.ones(3, np.float32))
    for t in GEMM_TUNES:
        assert_bitwise(brq.qgemm_fwd(to_dev(qx), to_dev(one), to_dev(qw), to_dev(np.ones(3, np.float32)), tune=t),
                       want, f"extreme {t}")


# --------------------------------------------------------------------------
# Walsh-Hadamard stages and the dW GEMM
# --------------------------------------------------------------------------
@pytest.mark.parametrize("b", [1, 2, 16, 64, 128])
def test_wht_quant_x(b):
    say("wht_quant_x", b)
    rng = np.random.default_rng(b)
    M, K = 256, 192
    qx = codes(rng, (M, K))
    qu, su, _ = orc.wht_int_quant(qx, b)
    gqut, gsu = brq.wht_quant_x(to_dev(qx), b)
    assert_bitwise(gqut, np.ascontiguousarray(qu.T), "q_u^T")
    assert_bitwise(gsu, np.array([su], np.float32), "s_u")


@pytest.mark.parametrize("shape,b,bf16", [((256, 192), 1, True), ((256, 192), 16, False),
                                          ((384, 640), 64, True), ((256, 1088), 128, True),
                                          ((512, 2048), 128, False), ((128, 64), 128, True)])
def test_quantize_x_wht(shape, b, bf16):
    """The activation codes and their rotation in one call equal the oracle's
    per-tensor quantiser followed by its integer rotation, bit for bit
    (ragged 512-column tiles, both element types, every tile height)."""
    say("quantize_x_wht", shape, b, bf16)
    x = syn.normal(shape, 1.0, tag=610 + b, bf16=bf16)
    if bf16:
        x = x.copy()
        x.reshape(-1)[::97] = np.uint16(0x0005)  # bf16 subnormals read as zero
    q, _, s, amax, fl = orc.quantize_lsq(x)
    qu, su, _ = orc.wht_int_quant(q, b)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    gq, gs, gamax, gqut, gsu = brq.quantize_x_wht(to_dev(x), b, flags=flags)
    assert_bitwise(gq, q, "q_x")
    assert_bitwise(gs, np.array([s], np.float32).reshape(-1), "s_x")
    assert_bitwise(gamax, np.array([amax], np.float32).reshape(-1), "amax_x")
    assert_bitwise(gqut, np.ascontiguousarray(qu.T), "q_u^T")
    assert_bitwise(gsu, np.array([su], np.float32), "s_u")
    assert int(flags.item()) == fl == 0


def test_quantize_x_wht_empty_and_flags():
    """No tokens or no columns: both step sizes 0; a non-finite input raises
    the flag as the per-tensor quantiser does."""
    say("quantize_x_wht empty and flags")
    for shape in ((0, 64), (64, 0)):
        x = np.zeros(shape, np.float32)
        _, gs, _, _, gsu = brq.quantize_x_wht(to_dev(x), 64)
        assert float(gs.item()) == 0.0 and float(gsu.item()) == 0.0
    x = np.ones((64, 64), np.float32)
    x[5, 7] = np.inf
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    brq.quantize_x_wht(to_dev(x), 64, flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 1


def test_wht_quant_x_empty_and_wide():
    """No tokens or no columns: step size 0 as for any empty group; and a
    wide input (K = 8192; the first pass's partials are summed by every
    work-group of the second: 128 of them here; the layer's 32768 x 8192
    input, with 4096, is in the full-size layer test)."""
    say("wht_quant_x empty and wide")
    for shape in ((0, 64), (64, 0)):
        qx = np.zeros(shape, np.int8)
        _, su, _ = orc.wht_int_quant(qx, 64)
        _, gsu = brq.wht_quant_x(to_dev(qx), 64)
        assert_bitwise(gsu, np.array([su], np.float32), f"s_u {shape}")
    rng = np.random.default_rng(77)
    qx = codes(rng, (1024, 8192))
    qu, su, _ = orc.wht_int_quant(qx, 128)
    gqut, gsu = brq.wht_quant_x(to_dev(qx), 128)
    assert_bitwise(gqut, np.ascontiguousarray(qu.T), "q_u^T wide")
    assert_bitwise(gsu, np.array([su], np.float32), "s_u wide")


@pytest.mark.parametrize("b", [1, 16, 64, 128])
@pytest.mark.parametrize("bf16", [False, True])
def test_wht_quant_dy(b, bf16):
    say("wht_quant_dy", b, bf16)
    M, N = 384, 320
    dy = syn.student_t3((M, N), 1e-3, tag=204, bf16=bf16)
    qv, sv, _, fl = orc.wht_fp_quant(dy, b)
    for chunk in (0, 10):
        flags = torch.zeros(1, dtype=torch.int32, device=DEV)
        gqvt, gsv = brq.wht_quant_dy(to_dev(dy), b, tune={"chunk_log2": chunk}, flags=flags)
        assert_bitwise(gqvt, np.ascontiguousarray(qv.T), f"q_v^T chunk {chunk}")
        assert_bitwise(gsv, np.array([sv], np.float32), "s_v")
        assert int(flags.item()) == fl == 0


@pytest.mark.parametrize("M,N,K,b", [(64, 256, 256, 64), (512, 192, 320, 128), (384, 64, 64, 16)])
def test_qgemm_bwd_dw_wht(M, N, K, b):
    say("qgemm_bwd_dw_wht", M, N, K, b)
    x = syn.normal((M, K), 1.0, tag=205)
    dy = syn.student_t3((M, N), 1e-3, tag=206, bf16=True)
    qx, _, sx, _, _ = orc.quantize_lsq(x)
    want, su, sv, _ = orc.qgemm_bwd_dw_wht(qx, sx, dy, b)
    dqx, dsx, ddy = to_dev(qx), to_dev(sx), to_dev(dy)
    for t in GEMM_TUNES[:6]:
        dw, gsu, gsv = brq.qgemm_bwd_dw_wht(dqx, dsx, ddy, b, tune=t)
        assert_bitwise(dw, want, f"dw {t}")
        assert_bitwise(gsu, np.array([su], np.float32), "s_u")
        assert_bitwise(gsv, np.array([sv], np.float32), "s_v")


@pytest.mark.parametrize("M,N,b,bf16", [(384, 320, 128, True), (256, 512, 64, True),
                                        (128, 64, 16, True), (1024, 2048, 128, True),
                                        (64, 256, 64, False), (192, 256, 64, True),
                                        (512, 768, 1, True), (256, 128, 32, True)])
def test_quantize_dy_bwd(M, N, b, bf16):
    """Both dY codes in one call equal quantize_lsq(col_mul) and the rotated
    LSQ of the oracle (two-pass form and its fallbacks)."""
    say("quantize_dy_bwd", M, N, b, bf16)
    dy = syn.student_t3((M, N), 1e-3, tag=230, bf16=bf16)
    sw = syn.normal((N,), 0.01, mean=0.02, tag=231)
    qg, _, sg, ag, fl = orc.quantize_lsq(dy, col_mul=sw)
    qv, sv, _, fl2 = orc.wht_fp_quant(dy, b)
    for chunk in (0, 10):
        flags = torch.zeros(1, dtype=torch.int32, device=DEV)
        gqg, gsg, gag, gqvt, gsv = brq.quantize_dy_bwd(to_dev(dy), to_dev(sw), b,
                                                       tune={"chunk_log2": chunk}, flags=flags)
        assert_bitwise(gqg, qg, f"q_g chunk {chunk}")
        assert_bitwise(gsg, sg, "s_g")
        assert_bitwise(gag, ag, "amax_g")
        assert_bitwise(gqvt, np.ascontiguousarray(qv.T), "q_v^T")
        assert_bitwise(gsv, np.array([sv], np.float32), "s_v")
        assert int(flags.item()) == fl == fl2 == 0


@pytest.mark.parametrize("M,N,b", [(256, 256, 128), (128, 320, 64), (256, 128, 32)])
def test_quantize_dy_bwd_tiny(M, N, b):
    """dY near the bottom of the binary32 range, with bf16 subnormals: the
    tiles take the flushing forms of the products and the butterflies."""
    say("quantize_dy_bwd tiny", M, N, b)
    dy = syn.student_t3((M, N), 1e-36, tag=232, bf16=True)
    syn.bf16_subnormals(dy, 50, tag=233)
    sw = syn.normal((N,), 0.01, mean=0.02, tag=234)
    qg, _, sg, ag, fl = orc.quantize_lsq(dy, col_mul=sw)
    qv, sv, _, fl2 = orc.wht_fp_quant(dy, b)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    gqg, gsg, gag, gqvt, gsv = brq.quantize_dy_bwd(to_dev(dy), to_dev(sw), b, flags=flags)
    assert_bitwise(gqg, qg, "q_g")
    assert_bitwise(gsg, sg, "s_g")
    assert_bitwise(gag, ag, "amax_g")
    assert_bitwise(gqvt, np.ascontiguousarray(qv.T), "q_v^T")
    assert_bitwise(gsv, np.array([sv], np.float32), "s_v")
    assert int(flags.item()) == (fl | fl2)


def test_quantize_dy_bwd_edges():
    say("quantize_dy_bwd_edges")
    M, N = 256, 128
    z = np.zeros((M, N), np.uint16)
    sw = np.full(N, 0.5, np.float32)
    gqg, gsg, _, gqvt, gsv = brq.quantize_dy_bwd(to_dev(z), to_dev(sw), 128)
    assert not to_np(gqg).any() and not to_np(gqvt).any()
    assert float(gsg.item()) == 0.0 and float(gsv.item()) == 0.0
    bad = syn.normal((M, N), 1e-3, tag=232, bf16=True)
    bad[7, 9] = 0x7f80  # +inf in bf16
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    brq.quantize_dy_bwd(to_dev(bad), to_dev(sw), 128, flags=flags)
    assert int(flags.item()) == brq.FLAG_NONFINITE


def test_qgemm_dw_stage_alone():
    say("qgemm_dw")
    rng = np.random.default_rng(17)
    M, N, K, b = 256, 128, 192, 64
    qv, qu = codes(rng, (M, N)), codes(rng, (M, K))
    want = orc.dw_gemm(qv, qu, 0.0123, 0.5, 3e-4, b)
    f = lambda v: to_dev(np.array([v], np.float32))
    got = brq.qgemm_dw(to_dev(np.ascontiguousarray(qv.T)), to_dev(np.ascontiguousarray(qu.T)),
                       f(0.0123), f(0.5), f(3e-4), b)
    assert_bitwise(got, want, "dw stage")


# --------------------------------------------------------------------------
# the whole tiny layer (64 tokens x 256 -> 256), fp32 inputs
# --------------------------------------------------------------------------
def test_tiny_layer_chain():
    say("tiny_layer_chain")
    d = syn.tiny()
    x, w, dy, b = d["x"], d["w"], d["dy"], d["block"]
    X, W, DY = to_dev(x), to_dev(w), to_dev(dy)
    oqx, _, osx, oax, _ = orc.quantize_lsq(x)
    oqw, oqwt, osw, oaw, _ = orc.quantize_lsq(w, per_row=True, want_t=True)
    oy = orc.qgemm_fwd(oqx, osx, oqw, osw)
    oqg, _, osg, _, _ = orc.quantize_lsq(dy, col_mul=osw)
    odx = orc.qgemm_bwd_dx(oqg, osg, oqw)
    odw, osu, osv, _ = orc.qgemm_bwd_dw_wht(oqx, osx, dy, b)
    qx, _, sx, ax = brq.quantize_lsq(X)
    qw, qwt, sw, aw = brq.quantize_lsq(W, per_row=True, want_t=True)
    y = brq.qgemm_fwd(qx, sx, qw, sw)
    qg, _, sg, _ = brq.quantize_lsq(DY, col_mul=sw)
    dx = brq.qgemm_bwd_dx(qg, sg, qwt)
    dw, su, sv, qut, qvt = brq.qgemm_bwd_dw_wht(qx, sx, DY, b, return_codes=True)
    for name, g, o in [("q_x", qx, oqx), ("s_x", sx, osx), ("amax_x", ax, oax), ("q_w", qw, oqw),
                       ("q_wt", qwt, oqwt), ("s_w", sw, osw), ("y", y, oy), ("q_g", qg, oqg),
                       ("s_g", sg, osg), ("dx", dx, odx), ("dw", dw, odw)]:
        assert_bitwise(g, o, name)
    qu, _, _ = orc.wht_int_quant(oqx, b)
    qv, _, _, _ = orc.wht_fp_quant(dy, b)
    assert_bitwise(qut, np.ascontiguousarray(qu.T), "q_u^T")
    assert_bitwise(qvt, np.ascontiguousarray(qv.T), "q_v^T")
    # on-device state hash of the outputs equals the oracle's
    ts = [("y", y), ("dx", dx), ("dw", dw)]
    want = orc.hash_state([(n, to_np(t)) for n, t in ts])
    assert bytes(to_np(brq.hash_state(ts))) == want


# --------------------------------------------------------------------------
# RMSNorm and grad-norm
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T,D,bf16", [(100, 2048, True), (64, 264, True), (33, 512, False),
                                      (17, 4096, True), (8, 8192, True)])
def test_rmsnorm_fwd(T, D, bf16):
    say("rmsnorm_fwd", T, D, bf16)
    x = syn.normal((T, D), 1.0, tag=207, bf16=bf16)
    if bf16:
        syn.bf16_subnormals(x, 100, tag=208)
    g = syn.normal((D,), 0.1, mean=1.0, tag=209, bf16=bf16)
    y, rstd, fl = orc.rmsnorm_fwd(x, g, 1e-6)
    gy, grstd = brq.rmsnorm_fixed_fwd(to_dev(x), to_dev(g), 1e-6)
    assert_bitwise(gy, y, "y")
    assert_bitwise(grstd, rstd, "rstd")


@pytest.mark.parametrize("T,D,xstd,gstd,gmean", [(64, 2048, 2.0 ** -63, 0.1, 1.0),
                                                 (48, 512, 1e-30, 0.1, 1.0),
                                                 (64, 2048, 1.0, 1e-37, 0.0),
                                                 (40, 264, 1e-19, 1e-30, 0.0)])
def test_rmsnorm_fwd_subnormal_band(T, D, xstd, gstd, gmean):
    """bf16 rows whose squares or products land at or below 2^-126: the
    unflushed evaluation of the squares (exponent bound on x) and of
    x * rstd * g (bounds on x, rstd and g) must fall back to the flushed one
    wherever a bound fails."""
    say("rmsnorm_fwd subnormal band", T, D, xstd, gstd)
    x = syn.normal((T, D), xstd, tag=218, bf16=True)
    syn.bf16_subnormals(x, 50, tag=219)
    # every other row at full scale, so waves of both kinds meet
    x[::2] = syn.normal((T, D), 1.0, tag=220, bf16=True)[::2]
    g = syn.normal((D,), gstd, mean=gmean, tag=221, bf16=True)
    y, rstd, fl = orc.rmsnorm_fwd(x, g, 1e-6)
    gy, grstd = brq.rmsnorm_fixed_fwd(to_dev(x), to_dev(g), 1e-6)
    assert_bitwise(gy, y, "y")
    assert_bitwise(grstd, rstd, "rstd")


def test_rmsnorm_fwd_subnormal_eps():
    """A subnormal eps reads as zero (DAZ on every input): rows whose mean
    square sits just above 2^-126, where an unflushed eps of 1e-40 would
    move rstd."""
    say("rmsnorm_fwd_subnormal_eps")
    rng = np.random.default_rng(11)
    T, D = 40, 512
    x = (rng.standard_normal((T, D)) * 2.0 ** -62).astype(np.float32)
    x[0] = np.float32(2.0 ** -63)  # ms = 2^-126 exactly
    x[1] = np.float32(-(2.0 ** -62))
    g = syn.normal((D,), 0.1, mean=1.0, tag=209)
    for eps in (1e-40, -1e-40, 0.0, 1e-6):
        y, rstd, fl = orc.rmsnorm_fwd(x, g, eps)
        gy, grstd = brq.rmsnorm_fixed_fwd(to_dev(x), to_dev(g), eps)
        assert_bitwise(grstd, rstd, f"rstd eps={eps}")
        assert_bitwise(gy, y, f"y eps={eps}")
    _, r0, _ = orc.rmsnorm_fwd(x, g, 0.0)
    _, r1, _ = orc.rmsnorm_fwd(x, g, 1e-40)
    assert np.array_equal(r0, r1)


@pytest.mark.parametrize("T,D,bf16", [(100, 2048, True), (64, 264, True), (33, 512, False),
                                      (70, 4096, True), (1025, 264, True)])
@pytest.mark.parametrize("rows", [0, 1, 4])
def test_rmsnorm_bwd(T, D, bf16, rows):
    """dg's block nodes folded 32 at a time over one to three levels (1025
    single-row blocks: 1025 -> 33 -> 2 -> 1)."""
    say("rmsnorm_bwd", T, D, bf16, rows)
    x = syn.normal((T, D), 1.0, tag=210, bf16=bf16)
    if bf16:
        syn.bf16_subnormals(x, 100, tag=211)
    g = syn.normal((D,), 0.1, mean=1.0, tag=212, bf16=bf16)
    dy = syn.normal((T, D), 1e-3, tag=213, bf16=bf16)
    _, rstd, _ = orc.rmsnorm_fwd(x, g, 1e-6)
    dx, dg = orc.rmsnorm_bwd(x, g, rstd, dy)
    gdx, gdg = brq.rmsnorm_fixed_bwd(to_dev(x), to_dev(g), to_dev(rstd), to_dev(dy),
                                     tune={"rows_per_block": rows})
    assert_bitwise(gdx, dx, "dx")
    assert_bitwise(gdg, dg, "dg")


@pytest.mark.parametrize("T,D,xstd,dystd", [(64, 2048, 1.0, 1e-36), (40, 264, 1e-19, 1e-19),
                                             (96, 2048, 1.0, 1e-3)])
def test_rmsnorm_bwd_subnormal_band(T, D, xstd, dystd):
    """Gradients in or near the subnormal band: products and sums of the
    backward land below 2^-126, so the unflushed row evaluation must fall
    back to the flushed one (and does not, for the last, ordinary case)."""
    say("rmsnorm_bwd subnormal band", T, D, xstd, dystd)
    x = syn.normal((T, D), xstd, tag=214, bf16=True)
    syn.bf16_subnormals(x, 100, tag=215)
    g = syn.normal((D,), 0.1, mean=1.0, tag=216, bf16=True)
    dy = syn.normal((T, D), dystd, tag=217, bf16=True)
    _, rstd, _ = orc.rmsnorm_fwd(x, g, 1e-6)
    dx, dg = orc.rmsnorm_bwd(x, g, rstd, dy)
    gdx, gdg = brq.rmsnorm_fixed_bwd(to_dev(x), to_dev(g), to_dev(rstd), to_dev(dy))
    assert_bitwise(gdx, dx, "dx")
    assert_bitwise(gdg, dg, "dg")


@pytest.mark.parametrize("n", [1, 1000, 4096 * 5 + 1664, (1 << 20) + 3])
@pytest.mark.parametrize("chunk", [0, 10, 14])
def test_grad_norm(n, chunk):
    say("grad_norm", n, chunk)
    v = syn.normal((n,), 1e-4, tag=214)
    ss, nrm, fl = orc.grad_norm(v)
    gs, gn = brq.grad_norm(to_dev(v), tune={"chunk_log2": chunk})
    assert_bitwise(gs, np.array(ss, np.float32), "sumsq")
    assert_bitwise(gn, np.array(nrm, np.float32), "norm")


def test_grad_norm_order_sensitive_vector():
    """The hand-derived tree vectors, as squares: leaves 4096^2 = 2^24 and
    ones.  Different reduction orders give different sums here."""
    say("grad_norm_order")
    for leaves in ([4096.0, 1, 1, 1], [4096.0, 1, 1], [4096.0, 1, 1, 1, 1, 1, 1]):
        v = np.array(leaves, np.float32)
        ss, _, _ = orc.grad_norm(v)
        gs, _ = brq.grad_norm(to_dev(v))
        assert_bitwise(gs, np.array(ss, np.float32), f"sumsq {leaves}")


# --------------------------------------------------------------------------
# hash
# --------------------------------------------------------------------------
def test_hash_state_vs_oracle():
    say("hash_state")
    rng = np.random.default_rng(19)
    ts = [("y", rng.standard_normal((33, 70)).astype(np.float32)),
          ("dw", rng.standard_normal((5, 4096 * 3 + 1)).astype(np.float32)),
          ("x", rng.integers(0, 65535, size=(7, 9), dtype=np.uint16)),
          ("big", rng.integers(0, 255, size=(4096 * 130 + 77,), dtype=np.uint8)),
          ("q", np.zeros((0, 4), np.int8))]
    want = orc.hash_state(ts)
    dts = []
    for n, a in ts:
        t = to_dev(a) if a.dtype != np.uint16 else to_dev(a)
        dts.append((n, t))
    got = bytes(to_np(brq.hash_state(dts)))
    assert got == want
    ts[1][1].view(np.uint8).reshape(-1)[4097] ^= 1
    assert bytes(to_np(brq.hash_state([(n, to_dev(a)) for n, a in ts]))) != want


def test_hash_split_equals_state():
    """Tensor digests in groups (and on another stream), then the combine,
    equal hash_state over the same list and the oracle."""
    say("hash_split")
    rng = np.random.default_rng(23)
    ts = [("a", rng.standard_normal((40, 4096 + 8)).astype(np.float32)),
          ("b", rng.integers(0, 65535, size=(9, 17), dtype=np.uint16)),
          ("c", rng.integers(-128, 127, size=(4096 * 129,), dtype=np.int8)),
          ("d", np.zeros((0, 4), np.float32))]
    want = orc.hash_state(ts)
    dts = [(n, to_dev(a)) for n, a in ts]
    assert bytes(to_np(brq.hash_state(dts))) == want
    dig = torch.zeros(32 * len(dts), dtype=torch.uint8, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        brq.hash_tensor_digests(dts[:2], dig[:64])
        brq.hash_tensor_digests(dts[2:], dig[64:])
    torch.cuda.current_stream().wait_stream(side)
    assert bytes(to_np(brq.hash_combine(dig))) == want
    for i, (n, a) in enumerate(ts):
        assert bytes(to_np(dig[32 * i:32 * i + 32])) == orc.tensor_digest(n, a)
    # the two stages: leaves on this stream, the rest on another once the
    # leaves are done -- after the tensors themselves have been overwritten
    ws = torch.zeros(brq.hash_digests_workspace_size(dts), dtype=torch.uint8, device=DEV)
    brq.hash_tensor_leaves(dts, ws)
    for _, t in dts:
        t.zero_()
    dig2 = torch.zeros_like(dig)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        brq.hash_tensor_finish(dts, dig2, ws)
    torch.cuda.current_stream().wait_stream(side)
    assert bytes(to_np(dig2)) == bytes(to_np(dig))


# --------------------------------------------------------------------------
# determinism: repeated calls and concurrent streams
# --------------------------------------------------------------------------
def test_repeat_and_streams():
    say("repeat_and_streams")
    x = to_dev(syn.normal((1024, 2048), 1.0, tag=215, bf16=True))
    w = to_dev(syn.normal((768, 2048), 0.02, tag=216, bf16=True))
    def run():
        qx, _, sx, _ = brq.quantize_lsq(x, ws=torch.zeros(1 << 22, dtype=torch.uint8, device=DEV))
        qw, _, sw, _ = brq.quantize_lsq(w, per_row=True)
        return brq.qgemm_fwd(qx, sx, qw, sw)
    ref = sha(run())
    for _ in range(3):
        assert sha(run()) == ref
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for s in (s1, s2):
        with torch.cuda.stream(s):
            outs.append(run())
    torch.cuda.synchronize()
    assert all(sha(o) == ref for o in outs)
