"""Seeded synthetic inputs for the W8A8 QAT linear layer and its reductions.

This module makes input tensors only: it holds none of the method's
arithmetic.  Both the CPU oracle and the GPU library consume what it writes.
Every value is a pure function of (seed, tensor tag, flat index) through
Philox4x32-10 (see ``philox.c``), so inputs do not depend on thread counts.

bfloat16 tensors are returned as ``numpy.uint16`` bit patterns.

Workload recipes (shapes and distributions of the Open-1B report's layer:
d_model 2048, GQA 16/4 heads of 128, 4096-token windows, 16,384-token
micro-batches; §3.1 Table 3, §3.2 "Batch size"):

  tiny   X fp32 [64,256] N(0,1); W fp32 [256,256] N(0,0.02);
         dY fp32 [64,256] N(0,1e-3); Hadamard block 64
  qkv    X bf16 [4096,2048] N(0,1) with 2 outlier input channels x20;
         W bf16 [3072,2048] N(0,0.02); forward only
  mlp    X bf16 [16384,2048] N(0,1); W bf16 [8192,2048] N(0,0.02);
         dY bf16 [16384,8192] 1e-3 * Student-t(3); Hadamard block 128
  norm   x bf16 [32768,2048] N(0,1) with 1% bf16 subnormals; g bf16 [2048]
         1+N(0,0.1); dy bf16 [32768,2048] N(0,1e-3); grad vector fp32
         [1.61e9] N(0,1e-4)
  layer  seven linears of one decoder layer over 32768 tokens (8 windows of
         4096): inputs bf16 N(0,1), weights bf16 N(0,0.02), dY per linear bf16
         N(0,1e-3); plus the layer's two RMSNorms at the norm recipe's
         distributions (h with 1% bf16 subnormals, g 1+N(0,0.1), dy N(0,1e-3))
  exchange  fp32 gradient contributions N(0,1e-4), one Philox tag each; at
         full size one rank's share of the Open-1B gradient (1.61e9 values)
         reduce-scattered over 8 shards: the grad-norm vector (the norm
         recipe's v) viewed as 8 contributions of 201.25e6 values
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbrq_synth.so")
SEED = 42

# tensor tags (the Philox key's second word)
TAG_X, TAG_W, TAG_DY, TAG_OUTLIER, TAG_G, TAG_V, TAG_SUBN = 1, 2, 3, 4, 5, 6, 7
TAG_P, TAG_M, TAG_S = 8, 9, 10

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(LIB_PATH)
        vp, i64, u32, i32, f64 = C.c_void_p, C.c_int64, C.c_uint32, C.c_int, C.c_double
        L.syn_philox4x32_10.restype = None
        L.syn_philox4x32_10.argtypes = [vp, vp, vp]
        L.syn_normal.restype = None
        L.syn_normal.argtypes = [u32, u32, i64, f64, f64, i32, vp]
        L.syn_student_t3.restype = None
        L.syn_student_t3.argtypes = [u32, u32, i64, f64, i32, vp]
        L.syn_pick_distinct.restype = None
        L.syn_pick_distinct.argtypes = [u32, u32, i64, i32, vp]
        L.syn_scale_columns.restype = None
        L.syn_scale_columns.argtypes = [vp, i32, i64, i64, vp, i32, f64]
        L.syn_bf16_subnormals.restype = None
        L.syn_bf16_subnormals.argtypes = [u32, u32, i64, u32, vp]
        L.syn_num_threads.restype = i32
        L.syn_num_threads.argtypes = []
        _lib = L
    return _lib


def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(np.asarray(ctr, np.uint32))
    k = np.ascontiguousarray(np.asarray(key, np.uint32))
    out = np.zeros(4, np.uint32)
    lib().syn_philox4x32_10(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def normal(shape, std=1.0, mean=0.0, tag=TAG_X, bf16=False, seed=SEED, out=None):
    n = int(np.prod(shape))
    a = out if out is not None else np.empty(shape, np.uint16 if bf16 else np.float32)
    lib().syn_normal(seed, tag, n, mean, std, int(bf16), a.ctypes.data)
    return a


def student_t3(shape, scale, tag=TAG_DY, bf16=False, seed=SEED):
    n = int(np.prod(shape))
    a = np.empty(shape, np.uint16 if bf16 else np.float32)
    lib().syn_student_t3(seed, tag, n, scale, int(bf16), a.ctypes.data)
    return a


def pick_distinct(range_, count, tag=TAG_OUTLIER, seed=SEED):
    out = np.zeros(count, np.int64)
    lib().syn_pick_distinct(seed, tag, range_, count, out.ctypes.data)
    return out


def scale_columns(a, which, mul):
    which = np.ascontiguousarray(which, np.int64)
    rows, cols = a.shape
    lib().syn_scale_columns(a.ctypes.data, int(a.dtype == np.uint16), rows, cols,
                            which.ctypes.data, which.size, float(mul))
    return a


def bf16_subnormals(a, every=100, tag=TAG_SUBN, seed=SEED):
    assert a.dtype == np.uint16
    lib().syn_bf16_subnormals(seed, tag, a.size, every, a.ctypes.data)
    return a


def num_threads():
    return lib().syn_num_threads()


def tag_for(layer: int, role: int) -> int:
    """Distinct tag per (linear index, tensor role) for multi-linear workloads."""
    return 1000 * (layer + 1) + role


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
def tiny(M=64, K=256, N=256, seed=SEED):
    return dict(
        x=normal((M, K), 1.0, tag=TAG_X, seed=seed),
        w=normal((N, K), 0.02, tag=TAG_W, seed=seed),
        dy=normal((M, N), 1e-3, tag=TAG_DY, seed=seed),
        block=64,
    )


def qkv(M=4096, K=2048, N=3072, seed=SEED):
    x = normal((M, K), 1.0, tag=TAG_X, bf16=True, seed=seed)
    n_out = max(1, int(round(0.001 * K)))
    cols = pick_distinct(K, n_out, tag=TAG_OUTLIER, seed=seed)
    scale_columns(x, cols, 20.0)
    return dict(x=x, w=normal((N, K), 0.02, tag=TAG_W, bf16=True, seed=seed), outlier_cols=cols)


def mlp(M=16384, K=2048, N=8192, seed=SEED):
    return dict(
        x=normal((M, K), 1.0, tag=TAG_X, bf16=True, seed=seed),
        w=normal((N, K), 0.02, tag=TAG_W, bf16=True, seed=seed),
        dy=student_t3((M, N), 1e-3, tag=TAG_DY, bf16=True, seed=seed),
        block=128,
    )


GRAD_NORM_N = 1_610_000_000


def norm(T=32768, D=2048, n_grad=GRAD_NORM_N, seed=SEED):
    x = normal((T, D), 1.0, tag=TAG_X, bf16=True, seed=seed)
    bf16_subnormals(x, 100, tag=TAG_SUBN, seed=seed)
    out = dict(
        x=x,
        g=normal((D,), 0.1, mean=1.0, tag=TAG_G, bf16=True, seed=seed),
        dy=normal((T, D), 1e-3, tag=TAG_DY, bf16=True, seed=seed),
    )
    if n_grad:
        out["v"] = normal((n_grad,), 1e-4, tag=TAG_V, seed=seed)
    return out


# one decoder layer: (name, in_features, out_features, input tensor name)
LAYER_LINEARS = [
    ("q", 2048, 2048, "x_attn"),
    ("k", 2048, 512, "x_attn"),
    ("v", 2048, 512, "x_attn"),
    ("o", 2048, 2048, "x_o"),
    ("gate", 2048, 8192, "x_mlp"),
    ("up", 2048, 8192, "x_mlp"),
    ("down", 8192, 2048, "x_down"),
]
LAYER_INPUTS = [("x_attn", 2048), ("x_o", 2048), ("x_mlp", 2048), ("x_down", 8192)]


def layer_input(name, M=32768, seed=SEED):
    idx = [n for n, _ in LAYER_INPUTS].index(name)
    K = LAYER_INPUTS[idx][1]
    return normal((M, K), 1.0, tag=tag_for(idx, TAG_X), bf16=True, seed=seed)


def layer_weight(i, seed=SEED):
    _, K, N, _ = LAYER_LINEARS[i]
    return normal((N, K), 0.02, tag=tag_for(i, TAG_W), bf16=True, seed=seed)


def layer_dy(i, M=32768, seed=SEED):
    _, _, N, _ = LAYER_LINEARS[i]
    return normal((M, N), 1e-3, tag=tag_for(i, TAG_DY), bf16=True, seed=seed)


# the layer's two pre-norm RMSNorms: (name, width)
LAYER_NORMS = [("attn_norm", 2048), ("mlp_norm", 2048)]


def layer_norm_inputs(j, M=32768, seed=SEED):
    """(h, g, dy) of norm j: h bf16 N(0,1) with 1% bf16 subnormals, g bf16
    1+N(0,0.1), dy bf16 N(0,1e-3)."""
    D = LAYER_NORMS[j][1]
    base = 20 + j
    h = normal((M, D), 1.0, tag=tag_for(base, TAG_X), bf16=True, seed=seed)
    bf16_subnormals(h, 100, tag=tag_for(base, TAG_SUBN), seed=seed)
    g = normal((D,), 0.1, mean=1.0, tag=tag_for(base, TAG_G), bf16=True, seed=seed)
    dy = normal((M, D), 1e-3, tag=tag_for(base, TAG_DY), bf16=True, seed=seed)
    return h, g, dy


def optimizer_group(n, grad_std=1e-4, param_bf16=True, grad_bf16=False, group=0, seed=SEED):
    """One synthetic parameter group for the optimizer step: parameters
    N(0, 0.02) (bf16 or fp32), gradients N(0, grad_std), first moments
    N(0, grad_std / 10), second moments |N(0, grad_std^2)| (fp32).  A Philox
    mask replaces 1% of the gradients with bf16 subnormals (read as zeros)."""
    base = 40 + group
    p = normal((n,), 0.02, tag=tag_for(base, TAG_P), bf16=param_bf16, seed=seed)
    g = normal((n,), grad_std, tag=tag_for(base, TAG_DY), bf16=grad_bf16, seed=seed)
    if grad_bf16:
        bf16_subnormals(g, 100, tag=tag_for(base, TAG_SUBN), seed=seed)
    m = normal((n,), grad_std / 10, tag=tag_for(base, TAG_M), seed=seed)
    v = np.abs(normal((n,), grad_std * grad_std, tag=tag_for(base, TAG_S), seed=seed))
    return p, g, m, v


def exchange_parts(count, n, std=1e-4, seed=SEED):
    """count fp32 gradient contributions of n values, N(0, std), tag per
    contribution."""
    return [normal((n,), std, tag=tag_for(60 + j, TAG_V), seed=seed) for j in range(count)]
