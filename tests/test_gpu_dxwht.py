"""GPU parity of the rotated input-gradient GEMM (brq_qgemm_bwd_dx_wht)
and its rows-rotation stage (brq_wht_quant_dy_rows) against the oracle, bit
for bit: Hadamard blocks 1..128, fp32 and bf16 gradients, several tiles
and every GEMM plan, and the layer's gate shape at full size (codes in full,
sampled rows of dX).
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


def weights(N, K, tag):
    w = syn.normal((N, K), 0.02, tag=tag)
    qw, _, sw, _, _ = orc.quantize_lsq(w, per_row=True)
    return qw, sw


@pytest.mark.parametrize("M,N,b,bf16", [(64, 256, 128, True), (48, 512, 64, False),
                                        (16, 64, 1, True), (32, 128, 2, False),
                                        (80, 384, 16, True), (64, 1024, 128, False),
                                        (128, 192, 32, True)])
def test_wht_quant_dy_rows(M, N, b, bf16):
    say("wht_quant_dy_rows", M, N, b, bf16)
    dy = syn.normal((M, N), 1e-3, tag=321, bf16=bf16)
    sw = syn.normal((N,), 0.01, mean=0.02, tag=322)
    q, s, _, fl = orc.wht_fp_rows_quant(dy, b, s_w=sw)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    gq, gs = brq.wht_quant_dy_rows(to_dev(dy), to_dev(sw), b, flags=flags)
    assert_bitwise(gs, np.array([s], np.float32), "s_g")
    assert_bitwise(gq, q, "q_g")
    assert int(flags.item()) == fl == 0


@pytest.mark.parametrize("M,N,K,b,bf16", [(64, 256, 128, 128, True), (320, 512, 192, 64, False),
                                          (48, 128, 64, 8, True), (256, 2048, 512, 128, True),
                                          (1024, 512, 2048, 128, True), (16, 64, 64, 1, False)])
def test_qgemm_bwd_dx_wht(M, N, K, b, bf16):
    say("qgemm_bwd_dx_wht", M, N, K, b, bf16)
    dy = syn.student_t3((M, N), 1e-3, tag=323, bf16=bf16)
    qw, sw = weights(N, K, 324)
    dx, s_g, s_h, fl = orc.qgemm_bwd_dx_wht(dy, sw, qw, b)
    q_g, _, _, _ = orc.wht_fp_rows_quant(dy, b, s_w=sw)
    q_h, _, _ = orc.wht_int_quant(qw, b)
    gdx, gsg, gsh, gqht, gqg = brq.qgemm_bwd_dx_wht(to_dev(dy), to_dev(sw), to_dev(qw), b,
                                                    return_codes=True)
    assert_bitwise(gsg, np.array([s_g], np.float32), "s_g")
    assert_bitwise(gsh, np.array([s_h], np.float32), "s_h")
    assert_bitwise(gqg, q_g, "q_g")
    assert_bitwise(gqht, np.ascontiguousarray(q_h.T), "q_h^T")
    assert_bitwise(gdx, dx, "dx")
    assert fl == 0


@pytest.mark.parametrize("tune", [dict(gemm_kernel=1), dict(gemm_kernel=2), dict(gemm_kernel=10),
                                  dict(gemm_kernel=10, split_k=4), dict(gemm_kernel=13),
                                  dict(chunk_log2=10)])
def test_qgemm_bwd_dx_wht_plans(tune):
    """Every GEMM plan and reduction chunk gives the same bits."""
    say("qgemm_bwd_dx_wht_plans", tune)
    M, N, K, b = 512, 1024, 512, 128
    dy = syn.normal((M, N), 1e-3, tag=325, bf16=True)
    qw, sw = weights(N, K, 326)
    dx, _, _, _ = orc.qgemm_bwd_dx_wht(dy, sw, qw, b)
    gdx, _, _ = brq.qgemm_bwd_dx_wht(to_dev(dy), to_dev(sw), to_dev(qw), b, tune=tune)
    assert_bitwise(gdx, dx, f"dx {tune}")


@pytest.mark.parametrize("bf16", [False, True])
def test_wht_rows_subnormal_band(bf16):
    """Values near the bottom of the binary32 range: products dY * s_w and
    butterfly sums land on subnormals (flushed to signed zeros) in some
    waves and not in others, so both evaluation forms run."""
    say("wht_rows_subnormal_band", bf16)
    M, N, b = 64, 512, 128
    dy = syn.normal((M, N), 1e-36, tag=328)
    dy[::3] *= np.float32(1e30)  # every third row well inside the normal range
    sw = syn.normal((N,), 0.01, mean=0.02, tag=329)
    sw[::17] = np.float32(3e-39)  # subnormal steps read as zero
    if bf16:
        dy = orc.to_bf16(dy)
    q, s, _, _ = orc.wht_fp_rows_quant(dy, b, s_w=sw)
    gq, gs = brq.wht_quant_dy_rows(to_dev(dy), to_dev(sw), b)
    assert_bitwise(gs, np.array([s], np.float32), "s_g")
    assert_bitwise(gq, q, "q_g")
    # only tiny rows: the statistic itself is near the bottom of the range
    tiny = np.ascontiguousarray(dy[1::3][:16])
    q, s, _, _ = orc.wht_fp_rows_quant(tiny, b, s_w=sw)
    gq, gs = brq.wht_quant_dy_rows(to_dev(tiny), to_dev(sw), b)
    assert_bitwise(gs, np.array([s], np.float32), "s_g tiny")
    assert_bitwise(gq, q, "q_g tiny")


def test_qgemm_bwd_dx_wht_edges():
    say("qgemm_bwd_dx_wht_edges")
    qw, sw = weights(256, 64, 327)
    # a zero gradient: codes 0, steps 0, dX = +0
    dy = np.zeros((32, 256), np.float32)
    gdx, gsg, _ = brq.qgemm_bwd_dx_wht(to_dev(dy), to_dev(sw), to_dev(qw), 64)
    assert float(gsg.item()) == 0.0 and not to_np(gdx).view(np.uint32).any()
    # non-finite statistic raises the flag
    dy[3, 7] = np.inf
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    brq.qgemm_bwd_dx_wht(to_dev(dy), to_dev(sw), to_dev(qw), 64, flags=flags)
    assert int(flags.item()) == brq.FLAG_NONFINITE
    # shapes outside the supported set are refused before any launch
    with pytest.raises(brq.BrqError):
        brq.qgemm_bwd_dx_wht(to_dev(np.zeros((32, 96), np.float32)), to_dev(sw[:96]),
                             to_dev(qw[:96]), 64)
    with pytest.raises(brq.BrqError):
        brq.qgemm_bwd_dx_wht(to_dev(np.zeros((8, 256), np.float32)), to_dev(sw), to_dev(qw), 64)
    # empty token count: nothing computed, nothing fails
    e = torch.empty((0, 256), dtype=torch.float32, device=DEV)
    gdx, _, _ = brq.qgemm_bwd_dx_wht(e, to_dev(sw), to_dev(qw), 64)
    assert gdx.shape == (0, 64)


def test_qgemm_bwd_dx_wht_gate_full():
    """The layer's gate linear at full size (32768 tokens, N = 8192 output
    channels, K = 2048): both rotated codes and scales in full, dX rows
    sampled across the tensor from the oracle's codes."""
    say("qgemm_bwd_dx_wht_gate_full")
    i = [n for n, *_ in syn.LAYER_LINEARS].index("gate")
    dy = syn.layer_dy(i)
    w = syn.layer_weight(i)
    qw, _, sw, _, _ = orc.quantize_lsq(w, per_row=True)
    b = 128
    q_g, s_g, _, fl = orc.wht_fp_rows_quant(dy, b, s_w=sw)
    q_h, s_h, _ = orc.wht_int_quant(qw, b)
    gdx, gsg, gsh, gqht, gqg = brq.qgemm_bwd_dx_wht(to_dev(dy), to_dev(sw), to_dev(qw), b,
                                                    return_codes=True)
    assert_bitwise(gsg, np.array([s_g], np.float32), "s_g")
    assert_bitwise(gsh, np.array([s_h], np.float32), "s_h")
    assert_bitwise(gqg, q_g, "q_g")
    assert_bitwise(gqht, np.ascontiguousarray(q_h.T), "q_h^T")
    rows = np.array([0, 1, 4095, 4096, 17000, 32767])
    acc = q_g[rows].astype(np.int64) @ q_h.astype(np.int64)
    c = np.float32(np.float32(s_g) * np.float32(s_h)) * np.float32(1.0 / b)
    want = (acc.astype(np.float32) * np.float32(c)).astype(np.float32)
    assert_bitwise(to_np(gdx)[rows], want, "dx sampled rows")
    assert fl == 0
