"""GPU parity of the per-tensor weight-scale variant (one LSQ step size per
weight tensor instead of one per output channel), composed from the
library's entry points exactly as a linear layer uses them: the weight
codes and their transpose, the forward GEMM with a scalar weight step, the
gradient codes of dY * s_w (the scalar broadcast to every column), and the
input-gradient GEMM.  Small shapes in full; the layer's k linear at full
size on sampled rows.
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


def linear_per_tensor_w(x, w, dy):
    """GPU: the linear's codes and products with a per-tensor weight step."""
    gx, _, gsx, _ = brq.quantize_lsq(to_dev(x))
    gqw, gqwt, gsw, _ = brq.quantize_lsq(to_dev(w), want_t=True)
    gy = brq.qgemm_fwd(gx, gsx, gqw, gsw)
    col = gsw.expand(w.shape[0]).contiguous()  # the scalar step of every output channel
    gqg, _, gsg, _ = brq.quantize_lsq(to_dev(dy), col_mul=col)
    gdx = brq.qgemm_bwd_dx(gqg, gsg, gqwt)
    return gx, gsx, gqw, gqwt, gsw, gy, gqg, gsg, gdx


@pytest.mark.parametrize("M,K,N,bf16", [(64, 256, 128, True), (200, 512, 320, False),
                                        (512, 1024, 512, True)])
def test_per_tensor_w_scales_linear(M, K, N, bf16):
    say("per_tensor_w_scales", M, K, N, bf16)
    x = syn.normal((M, K), 1.0, tag=331, bf16=bf16)
    w = syn.normal((N, K), 0.02, tag=332, bf16=bf16)
    dy = syn.normal((M, N), 1e-3, tag=333, bf16=bf16)
    qx, _, sx, _, _ = orc.quantize_lsq(x)
    qw, qwt, sw, _, _ = orc.quantize_lsq(w, want_t=True)
    y = orc.qgemm_fwd(qx, sx, qw, sw)
    qg, _, sg, _, _ = orc.quantize_lsq(dy, col_mul=np.full(N, sw[0], np.float32))
    dx = orc.qgemm_bwd_dx(qg, sg, qw)
    gx, gsx, gqw, gqwt, gsw, gy, gqg, gsg, gdx = linear_per_tensor_w(x, w, dy)
    assert_bitwise(gsw, sw, "s_w")
    assert_bitwise(gqw, qw, "q_w")
    assert_bitwise(gqwt, qwt, "q_w^T")
    assert_bitwise(gy, y, "y")
    assert_bitwise(gsg, sg, "s_g")
    assert_bitwise(gqg, qg, "q_g")
    assert_bitwise(gdx, dx, "dx")


def test_per_tensor_w_scales_k_linear_full():
    """The layer's k linear (32768 x 2048 -> 512) at full size: codes and
    scales in full, y and dX on sampled rows from the oracle's codes."""
    say("per_tensor_w_scales_k_full")
    i = [n for n, *_ in syn.LAYER_LINEARS].index("k")
    _, K, N, xin = syn.LAYER_LINEARS[i]
    x, w, dy = syn.layer_input(xin), syn.layer_weight(i), syn.layer_dy(i)
    qx, _, sx, _, _ = orc.quantize_lsq(x)
    qw, qwt, sw, _, _ = orc.quantize_lsq(w, want_t=True)
    qg, _, sg, _, _ = orc.quantize_lsq(dy, col_mul=np.full(N, sw[0], np.float32))
    gx, gsx, gqw, gqwt, gsw, gy, gqg, gsg, gdx = linear_per_tensor_w(x, w, dy)
    for g, want, name in ((gx, qx, "q_x"), (gsx, sx, "s_x"), (gqw, qw, "q_w"), (gqwt, qwt, "q_w^T"),
                          (gsw, sw, "s_w"), (gqg, qg, "q_g"), (gsg, sg, "s_g")):
        assert_bitwise(g, want, name)
    rows = np.array([0, 3, 8191, 8192, 20000, 32767])
    assert_bitwise(to_np(gy)[rows], orc.qgemm_fwd(qx[rows], sx, qw, sw), "y rows")
    assert_bitwise(to_np(gdx)[rows], orc.qgemm_bwd_dx(qg[rows], sg, qw), "dx rows")
