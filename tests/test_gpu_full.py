"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (default tune) and, for the MLP and layer workloads, under
two other launch configurations (GEMM kernel, split-K, reduction chunk and
RMSNorm backward rows per block): every output's SHA-256 against the digests
the CPU oracle wrote (tests/golden/config_digests.txt, produced by
tests/golden/make_digests.py from oracle/ alone), plus outputs the oracle
recomputes here row by row, so a mismatch names where it is.

Workloads (seeded synthetic inputs, brq_synth):
  qkv    4096 tokens x 2048 -> 3072 forward, per-channel and per-tensor W
  mlp    16384 tokens x 2048 -> 8192 forward + backward, Hadamard block 128
  norm   RMSNorm 32768 x 2048 forward + backward; grad-norm over 1.61e9
  layer  one decoder layer's step over 32768 tokens (the benchmark step)
"""
import hashlib
import os
import sys

import numpy as np
import pytest
import torch

import brq_synth as syn
import oracle as orc
from tests.gpu_util import DEV, assert_bitwise, to_dev, to_np

pytestmark = pytest.mark.gpu

DIGESTS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "config_digests.txt")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def stored(cfg):
    out = {}
    if os.path.exists(DIGESTS):
        for line in open(DIGESTS):
            f = line.split()
            if len(f) >= 3 and f[0] == cfg:
                out[f[1]] = f[2]
    if not out:
        pytest.skip(f"no oracle digests for {cfg}: run tests/golden/make_digests.py {cfg}")
    return out


def sha_dev(t: torch.Tensor) -> str:
    return hashlib.sha256(to_np(t).tobytes()).hexdigest()


def check_digests(cfg, got):
    want = stored(cfg)
    bad = [n for n, t in got.items() if n in want and sha_dev(t) != want[n]]
    missing = [n for n in got if n not in want]
    assert not missing, f"{cfg}: no stored digest for {missing}"
    assert not bad, f"{cfg}: outputs differ from the oracle: {bad}"


def sample_rows(M, k=6):
    return sorted(set([0, 1, M // 2 - 1, M // 2, M - 2, M - 1][:k]))


@pytest.fixture(scope="module")
def brq():
    import bitwise_reproducible_int8_amd as m
    m.lib()
    return m


@pytest.mark.timeout(600)
def test_qkv_full(brq):
    say("full qkv 4096x2048->3072")
    d = syn.qkv()
    X, W = to_dev(d["x"]), to_dev(d["w"])
    qx, _, sx, ax = brq.quantize_lsq(X)
    qw, _, sw, aw = brq.quantize_lsq(W, per_row=True)
    y = brq.qgemm_fwd(qx, sx, qw, sw)
    qp, _, sp, ap = brq.quantize_lsq(W)
    ypt = brq.qgemm_fwd(qx, sx, qp, sp)
    # the oracle, row by row on sampled tokens
    oqx, _, osx, _, _ = orc.quantize_lsq(d["x"])
    oqw, _, osw, _, _ = orc.quantize_lsq(d["w"], per_row=True)
    rows = sample_rows(4096)
    assert_bitwise(to_np(y)[rows], orc.qgemm_fwd(oqx[rows], osx, oqw, osw), "y sampled rows")
    check_digests("qkv", {"q_x": qx, "s_x": sx, "amax_x": ax, "q_w": qw, "s_w": sw, "amax_w": aw,
                          "y": y, "q_w_pt": qp, "s_w_pt": sp, "amax_w_pt": ap, "y_pt": ypt})


# Launch configurations the full-size workloads also run under: the
# benchmark's default plan, the 8-wave direct-to-LDS GEMM with the
# contraction split in two (exact int32 partials) and the smallest
# reduction chunk, and the persistent GEMM split in two with the largest
# chunk; RMSNorm backward at 4 and 32 rows per block (the default is 8).
FULL_TUNES = [None,
              dict(gemm_kernel=10, split_k=2, chunk_log2=10, rows_per_block=4),
              dict(gemm_kernel=13, split_k=2, chunk_log2=16, rows_per_block=32)]


def _tid(t):
    return "default" if t is None else "k{gemm_kernel}-s{split_k}-c{chunk_log2}-r{rows_per_block}".format(**t)


@pytest.fixture(scope="module")
def mlp_data():
    d = syn.mlp()
    return d, to_dev(d["x"]), to_dev(d["w"]), to_dev(d["dy"])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("tune", FULL_TUNES, ids=_tid)
def test_mlp_full(brq, mlp_data, tune):
    say("full mlp 16384x2048->8192 fwd+bwd", tune)
    d, X, W, DY = mlp_data
    b = d["block"]
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    qx, _, sx, ax = brq.quantize_lsq(X, flags=flags, tune=tune)
    qw, qwt, sw, aw = brq.quantize_lsq(W, per_row=True, want_t=True, flags=flags, tune=tune)
    y = brq.qgemm_fwd(qx, sx, qw, sw, tune=tune)
    qg, _, sg, ag = brq.quantize_lsq(DY, col_mul=sw, flags=flags, tune=tune)
    dx = brq.qgemm_bwd_dx(qg, sg, qwt, tune=tune)
    dw, su, sv, qut, qvt = brq.qgemm_bwd_dw_wht(qx, sx, DY, b, flags=flags, return_codes=True,
                                                tune=tune)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    got = {"q_x": qx, "s_x": sx, "amax_x": ax, "q_w": qw, "q_wt": qwt, "s_w": sw, "amax_w": aw,
           "y": y, "q_g": qg, "s_g": sg, "amax_g": ag, "dx": dx, "q_ut": qut, "s_u": su,
           "q_vt": qvt, "s_v": sv, "dw": dw}
    # oracle recomputation of sampled rows of every GEMM output
    oqx, _, osx, _, _ = orc.quantize_lsq(d["x"])
    oqw, _, osw, _, _ = orc.quantize_lsq(d["w"], per_row=True)
    rows = sample_rows(16384)
    assert_bitwise(to_np(y)[rows], orc.qgemm_fwd(oqx[rows], osx, oqw, osw), "y sampled rows")
    oqg, _, osg, _, _ = orc.quantize_lsq(d["dy"], col_mul=osw)
    assert_bitwise(to_np(dx)[rows], orc.qgemm_bwd_dx(oqg[rows], osg, oqw), "dx sampled rows")
    oqu, osu, _ = orc.wht_int_quant(oqx, b)
    oqv, osv, _, _ = orc.wht_fp_quant(d["dy"], b)
    n_lo, n_hi = 8192 - 4, 8192
    odw = orc.dw_gemm(oqv, oqu, osx[0], osu, osv, b, n_lo, n_hi)
    assert_bitwise(to_np(dw)[n_lo:n_hi], odw[n_lo:n_hi], "dw sampled rows")
    check_digests("mlp", got)
    ts = [("y", y), ("dx", dx), ("dw", dw)]
    assert bytes(to_np(brq.hash_state(ts))).hex() == stored("mlp")["state"]


@pytest.mark.timeout(900)
def test_norm_full(brq):
    say("full norm 32768x2048 + grad-norm 1.61e9")
    d = syn.norm(n_grad=0)
    X, G, DY = to_dev(d["x"]), to_dev(d["g"]), to_dev(d["dy"])
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    y, rstd = brq.rmsnorm_fixed_fwd(X, G, 1e-6, flags=flags)
    dx, dg = brq.rmsnorm_fixed_bwd(X, G, rstd, DY)
    rows = sample_rows(32768)
    oy, orstd, _ = orc.rmsnorm_fwd(d["x"][rows], d["g"], 1e-6)
    assert_bitwise(to_np(y)[rows], oy, "y sampled rows")
    assert_bitwise(to_np(rstd)[rows], orstd, "rstd sampled rows")
    odx, _ = orc.rmsnorm_bwd(d["x"][rows], d["g"], orstd, d["dy"][rows])
    assert_bitwise(to_np(dx)[rows], odx, "dx sampled rows")
    got = {"y": y, "rstd": rstd, "dx": dx, "dg": dg}
    del X, DY, d
    v = syn.normal((syn.GRAD_NORM_N,), 1e-4, tag=syn.TAG_V)
    V = torch.from_numpy(v).to(DEV)
    del v
    ss, nrm = brq.grad_norm(V, flags=flags)
    got["grad_norm"] = torch.stack([ss, nrm])
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    check_digests("norm", got)


@pytest.fixture(scope="module")
def layer_data():
    M = 32768
    x = {name: to_dev(syn.layer_input(name, M)) for name, _ in syn.LAYER_INPUTS}
    w = [to_dev(syn.layer_weight(i)) for i in range(len(syn.LAYER_LINEARS))]
    dy = [to_dev(syn.layer_dy(i, M)) for i in range(len(syn.LAYER_LINEARS))]
    norms = [(n,) + tuple(to_dev(a) for a in syn.layer_norm_inputs(j, M))
             for j, (n, _) in enumerate(syn.LAYER_NORMS)]
    return M, x, w, dy, norms


@pytest.mark.timeout(900)
@pytest.mark.parametrize("tune", FULL_TUNES, ids=_tid)
def test_layer_full(brq, layer_data, tune):
    """The benchmark's step: digests of every output, gradient and scale,
    and the on-device state hash."""
    say("full layer 32768 tokens (the benchmark step)", tune)
    from bitwise_reproducible_int8_amd.layer import LayerStep
    M, x, w, dy, norms = layer_data
    step = LayerStep(syn.LAYER_LINEARS, x, w, dy, norms, block=128, tune=tune)
    step.run()
    torch.cuda.synchronize()
    assert int(step.flags.item()) == 0
    got = {}
    for name in x:
        got.update({f"{name}.q_x": step.q_x[name], f"{name}.s_x": step.s_x[name],
                    f"{name}.amax_x": step.amax_x[name], f"{name}.q_ut": step.q_ut[name],
                    f"{name}.s_u": step.s_u[name]})
    for i, (ln, _, _, _) in enumerate(syn.LAYER_LINEARS):
        got.update({f"{ln}.q_w": step.q_w[i], f"{ln}.q_wt": step.q_wt[i], f"{ln}.s_w": step.s_w[i],
                    f"{ln}.y": step.y[i], f"{ln}.q_g": step.q_g[i], f"{ln}.s_g": step.s_g[i],
                    f"{ln}.dx": step.dx[i], f"{ln}.q_vt": step.q_vt[i], f"{ln}.s_v": step.s_v[i],
                    f"{ln}.dw": step.dw[i]})
    for j, (nn, _) in enumerate(syn.LAYER_NORMS):
        got.update({f"{nn}.y": step.ny[j], f"{nn}.rstd": step.nrstd[j], f"{nn}.dx": step.ndx[j],
                    f"{nn}.dg": step.ndg[j]})
    got["grad_norm"] = step.gn
    # oracle on sampled tokens of the widest-contraction linear (down, K=8192)
    i = [n for n, _, _, _ in syn.LAYER_LINEARS].index("down")
    xin = syn.LAYER_LINEARS[i][3]
    xd = syn.layer_input(xin, M)
    oqx, _, osx, _, _ = orc.quantize_lsq(xd)
    oqw, _, osw, _, _ = orc.quantize_lsq(syn.layer_weight(i), per_row=True)
    rows = sample_rows(M, 4)
    assert_bitwise(to_np(step.y[i])[rows], orc.qgemm_fwd(oqx[rows], osx, oqw, osw),
                   "down.y sampled rows")
    check_digests("layer", got)
    assert bytes(to_np(step.digest)).hex() == stored("layer")["state"]
    # a second step on the same inputs reproduces the digest
    step.run()
    assert bytes(to_np(step.digest)).hex() == stored("layer")["state"]


@pytest.mark.timeout(900)
def test_layer_full_overlapped_hash(brq, layer_data):
    """The benchmark's timed loop: steps back to back with each step's hash
    above its leaf level on a second stream, overlapping the next step.
    Every step's state digest (each into its own buffer) equals the
    oracle's, and a step without the overlap after them still does."""
    say("full layer 32768 tokens, overlapped hash, 4 steps")
    from bitwise_reproducible_int8_amd.layer import LayerStep
    M, x, w, dy, norms = layer_data
    step = LayerStep(syn.LAYER_LINEARS, x, w, dy, norms, block=128)
    outs = [torch.zeros(32, dtype=torch.uint8, device=DEV) for _ in range(4)]
    for d in outs:
        step.run(overlap_hash=True, digest_out=d)
    step.finish()
    torch.cuda.synchronize()
    want = stored("layer")["state"]
    for k, d in enumerate(outs):
        assert bytes(to_np(d)).hex() == want, f"step {k}"
    step.run()
    torch.cuda.synchronize()
    assert bytes(to_np(step.digest)).hex() == want


@pytest.mark.parametrize("grad_std,expect", [(1e-4, "keep"), (3e-4, "clip"), (1e-3, "skip")])
def test_optimizer_full(brq, grad_std, expect):
    """The optimizer step over a layer-sized parameter set (the seven
    linears' 60.8 M bf16 weights with weight decay, the two norm gains
    without), clipped by the global norm of the same gradients: unclipped,
    clipped and skipped steps, against the oracle, every element."""
    n_lin = sum(N * K for _, K, N, _ in syn.LAYER_LINEARS)
    n_nrm = sum(D for _, D in syn.LAYER_NORMS)
    say("full optimizer", n_lin, n_nrm, grad_std, expect)
    p1, g1, m1, v1 = syn.optimizer_group(n_lin, grad_std=grad_std, group=0)
    p2, g2, m2, v2 = syn.optimizer_group(n_nrm, grad_std=grad_std, group=1)
    g = np.concatenate([g1, g2])
    t, lr = 5, 3e-4
    _, onorm, _ = orc.grad_norm(g)
    ap, cl, ost, _ = orc.adamw_decide(onorm, 0)
    kind = "skip" if ap == 0 else ("clip" if cl != 1.0 else "keep")
    assert kind == expect, (float(onorm), kind)
    bc = orc.adamw_bias_corrections(t)
    dp = to_dev(np.concatenate([p1, p2]))
    dg = to_dev(g)
    dm = to_dev(np.concatenate([m1, m2]))
    dv = to_dev(np.concatenate([v1, v2]))
    gn = torch.empty(2, dtype=torch.float32, device=DEV)
    brq.grad_norm(dg, out=gn)
    skip = torch.zeros(1, dtype=torch.int32, device=DEV)
    ctl = brq.adamw_decide(gn[1:2], skip)
    bcd = brq.adamw_bias_corrections(t)
    brq.adamw_step(dp[:n_lin], dg[:n_lin], dm[:n_lin], dv[:n_lin], ctl, lr, bcd, weight_decay=0.1)
    brq.adamw_step(dp[n_lin:], dg[n_lin:], dm[n_lin:], dv[n_lin:], ctl, lr, bcd, weight_decay=0.0)
    torch.cuda.synchronize()
    assert_bitwise(gn[1:2], np.array([onorm], np.float32), "norm")
    assert_bitwise(ctl, np.array([ap, cl], np.float32), "ctl")
    assert int(skip.item()) == ost
    del g, dg
    for lo, hi, (p, gg, m, v), wd in ((0, n_lin, (p1, g1, m1, v1), 0.1),
                                      (n_lin, n_lin + n_nrm, (p2, g2, m2, v2), 0.0)):
        wp, wm, wv = orc.adamw_step(p, gg, m, v, lr, bc[0], bc[1], ap, cl, wd=wd)
        assert_bitwise(dp[lo:hi], wp, f"param [{lo}, {hi})")
        assert_bitwise(dm[lo:hi], wm, f"m [{lo}, {hi})")
        assert_bitwise(dv[lo:hi], wv, f"v [{lo}, {hi})")
