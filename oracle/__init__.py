"""ctypes binding of the plain sequential C oracle (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The product path (``libbrq``) never
touches it.  All arrays are host numpy arrays; bfloat16 tensors are carried
as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("BRQ_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")

F32, BF16, I8, I32, U8 = 0, 1, 2, 3, 4
PER_TENSOR, PER_ROW = 0, 1
FLAG_NONFINITE = 1

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(LIB_PATH)
        vp, i64, f32, i32 = C.c_void_p, C.c_int64, C.c_float, C.c_int
        L.orc_num_threads.restype = i32
        L.orc_num_threads.argtypes = []
        L.orc_set_num_threads.restype = None
        L.orc_set_num_threads.argtypes = [i32]
        L.orc_flush.restype = f32
        L.orc_flush.argtypes = [f32]
        L.orc_bf16_to_f32.restype = f32
        L.orc_bf16_to_f32.argtypes = [C.c_uint16]
        L.orc_f32_to_bf16.restype = C.c_uint16
        L.orc_f32_to_bf16.argtypes = [f32]
        L.orc_f32_to_bf16_array.restype = None
        L.orc_f32_to_bf16_array.argtypes = [vp, i64, vp]
        L.orc_lsq_k2.restype = f32
        L.orc_lsq_k2.argtypes = []
        L.orc_tree_sum.restype = f32
        L.orc_tree_sum.argtypes = [vp, i64]
        L.orc_tree_sum_recursive.restype = f32
        L.orc_tree_sum_recursive.argtypes = [vp, i64]
        L.orc_lsq_scale.restype = None
        L.orc_lsq_scale.argtypes = [f32, i64, vp, vp]
        L.orc_quant1.restype = C.c_int8
        L.orc_quant1.argtypes = [f32, f32]
        L.orc_quantize_lsq.restype = i32
        L.orc_quantize_lsq.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp, vp, vp]
        L.orc_quantize_lsq_exact.restype = i32
        L.orc_quantize_lsq_exact.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp, vp, vp]
        L.orc_exact_abs_sum.restype = f32
        L.orc_exact_abs_sum.argtypes = [vp, i64]
        L.orc_qgemm_fwd.restype = None
        L.orc_qgemm_fwd.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, vp]
        L.orc_qgemm_bwd_dx.restype = None
        L.orc_qgemm_bwd_dx.argtypes = [vp, vp, vp, i64, i64, i64, vp]
        L.orc_wht_int.restype = None
        L.orc_wht_int.argtypes = [vp, i64, i64, i32, vp]
        L.orc_wht_int_quant.restype = None
        L.orc_wht_int_quant.argtypes = [vp, i64, i64, i32, vp, vp, vp]
        L.orc_wht_fp_quant.restype = i32
        L.orc_wht_fp_quant.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp]
        L.orc_dw_gemm.restype = None
        L.orc_dw_gemm.argtypes = [vp, vp, i64, i64, i64, f32, f32, f32, i32, i64, i64, vp]
        L.orc_qgemm_bwd_dw_wht.restype = i32
        L.orc_wht_fp_rows_quant.restype = i32
        L.orc_wht_fp_rows_quant.argtypes = [vp, i32, i64, i64, vp, i32, vp, vp, vp]
        L.orc_qgemm_bwd_dx_wht.restype = i32
        L.orc_exp_f.restype = f32
        L.orc_exp_f.argtypes = [f32]
        L.orc_attn_fwd.restype = i32
        L.orc_attn_fwd.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, vp]
        L.orc_qgemm_bwd_dx_wht.argtypes = [vp, i32, vp, vp, i64, i64, i64, i32, vp, vp, vp]
        L.orc_qgemm_bwd_dw_wht.argtypes = [vp, vp, vp, i32, i64, i64, i64, i32, vp, vp, vp]
        L.orc_rmsnorm_fwd.restype = i32
        L.orc_rmsnorm_fwd.argtypes = [vp, vp, i32, i64, i64, f32, vp, vp]
        L.orc_rmsnorm_bwd.restype = None
        L.orc_rmsnorm_bwd.argtypes = [vp, vp, vp, vp, i32, i64, i64, vp, vp]
        L.orc_grad_norm.restype = i32
        L.orc_grad_norm.argtypes = [vp, i64, vp, vp]
        L.orc_adamw_bias_corrections.restype = None
        L.orc_adamw_bias_corrections.argtypes = [i64, f32, f32, vp, vp]
        L.orc_adamw_decide.restype = i32
        L.orc_adamw_decide.argtypes = [f32, f32, f32, i32, vp, vp, vp]
        L.orc_adamw_step.restype = None
        L.orc_adamw_step.argtypes = [vp, i32, vp, i32, vp, vp, i64] + [f32] * 9
        L.orc_ascending_sum.restype = None
        L.orc_ascending_sum.argtypes = [vp, i32, i64, vp]
        L.orc_average.restype = None
        L.orc_average.argtypes = [vp, i64, i64, vp]
        L.orc_treefold.restype = None
        L.orc_treefold.argtypes = [vp, i32, i64, vp]
        L.orc_dp_reduce.restype = i32
        L.orc_dp_reduce.argtypes = [vp, i32, i32, i32, i64, i32, vp]
        L.orc_prim_sweep.restype = None
        L.orc_prim_sweep.argtypes = [i32, C.c_uint32, i64, vp]
        L.orc_sha256.restype = None
        L.orc_sha256.argtypes = [vp, C.c_uint64, vp]
        L.orc_merkle_root.restype = None
        L.orc_merkle_root.argtypes = [vp, C.c_uint64, vp]
        L.orc_tensor_digest.restype = None
        L.orc_tensor_digest.argtypes = [vp, C.c_uint64, i32, i32, vp, C.c_char_p, vp]
        L.orc_hash_state.restype = None
        L.orc_hash_state.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"unsupported dtype {a.dtype}")


def _c(a, dt=None):
    a = np.ascontiguousarray(a if dt is None else a.astype(dt, copy=False))
    return a


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    lib().orc_set_num_threads(int(n))


def flush(v: float) -> float:
    return lib().orc_flush(v)


def bf16_to_f32(h: int) -> float:
    return lib().orc_bf16_to_f32(h)


def f32_to_bf16(f: float) -> int:
    return lib().orc_f32_to_bf16(f)


def to_bf16(a):
    """fp32 array -> bf16 bit patterns (uint16), nearest even (the bf16
    output variant of the GEMMs)."""
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().orc_f32_to_bf16_array(_p(a), a.size, _p(out))
    return out


def lsq_k2() -> float:
    return lib().orc_lsq_k2()


def tree_sum(leaves, recursive: bool = False) -> np.float32:
    a = _c(leaves, np.float32)
    f = lib().orc_tree_sum_recursive if recursive else lib().orc_tree_sum
    return np.float32(f(_p(a), a.size))


def lsq_scale(S: float, n: int):
    s = np.zeros(1, np.float32)
    r = np.zeros(1, np.float32)
    lib().orc_lsq_scale(S, n, _p(s), _p(r))
    return s[0], r[0]


def quant1(x: float, r: float) -> int:
    return int(lib().orc_quant1(x, r))


def exact_abs_sum(v) -> np.float32:
    """Sum of |v| taken exactly, rounded once to binary32 (nearest even)."""
    a = _c(v, np.float32)
    return np.float32(lib().orc_exact_abs_sum(_p(a), a.size))


def quantize_lsq(x: np.ndarray, per_row: bool = False, col_mul=None, want_t: bool = False,
                 exact: bool = False):
    """Returns (q, q_t or None, scale, amax, flags).  exact=True takes the
    statistic as the exact sum of |v| rounded once instead of the tree."""
    x = _c(x)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.int8)
    q_t = np.empty((cols, rows), np.int8) if want_t else None
    ns = rows if per_row else 1
    scale = np.empty(ns, np.float32)
    amax = np.empty(ns, np.float32)
    cm = None if col_mul is None else _c(col_mul, np.float32)
    f = lib().orc_quantize_lsq_exact if exact else lib().orc_quantize_lsq
    flags = f(_p(x), _dtype_code(x), rows, cols, PER_ROW if per_row else PER_TENSOR,
              _p(cm), _p(q), _p(q_t), _p(scale), _p(amax))
    return q, q_t, scale, amax, flags


def qgemm_fwd(q_x, s_x, q_w, s_w):
    q_x, q_w = _c(q_x, np.int8), _c(q_w, np.int8)
    M, K = q_x.shape
    N = q_w.shape[0]
    s_x = _c(np.atleast_1d(s_x), np.float32)
    s_w = _c(np.atleast_1d(s_w), np.float32)
    y = np.empty((M, N), np.float32)
    lib().orc_qgemm_fwd(_p(q_x), _p(s_x), _p(q_w), _p(s_w), int(s_w.size > 1),
                        M, N, K, _p(y))
    return y


def qgemm_bwd_dx(q_g, s_g, q_w):
    q_g, q_w = _c(q_g, np.int8), _c(q_w, np.int8)
    M, N = q_g.shape
    K = q_w.shape[1]
    s_g = _c(np.atleast_1d(s_g), np.float32)
    dx = np.empty((M, K), np.float32)
    lib().orc_qgemm_bwd_dx(_p(q_g), _p(s_g), _p(q_w), M, N, K, _p(dx))
    return dx


def _block(length: int, b: int, what: str) -> None:
    """The rotation runs over aligned blocks of b along one dimension: b must
    be a power of two dividing that dimension (the C loops index whole
    blocks and would run past a ragged end)."""
    if b < 1 or b & (b - 1) or length % b:
        raise ValueError(f"rotation block {b}: needs a power of two dividing {what} = {length}")


def wht_int(q_x, b: int):
    q_x = _c(q_x, np.int8)
    M, K = q_x.shape
    _block(M, b, "tokens")
    u = np.empty((M, K), np.int32)
    lib().orc_wht_int(_p(q_x), M, K, b, _p(u))
    return u


def wht_int_quant(q_x, b: int):
    q_x = _c(q_x, np.int8)
    M, K = q_x.shape
    _block(M, b, "tokens")
    q_u = np.empty((M, K), np.int8)
    s_u = np.zeros(1, np.float32)
    S = np.zeros(1, np.int64)
    lib().orc_wht_int_quant(_p(q_x), M, K, b, _p(q_u), _p(s_u), _p(S))
    return q_u, s_u[0], int(S[0])


def wht_fp_quant(dy, b: int, want_v: bool = False):
    dy = _c(dy)
    M, N = dy.shape
    _block(M, b, "tokens")
    q_v = np.empty((M, N), np.int8)
    s_v = np.zeros(1, np.float32)
    v = np.empty((M, N), np.float32) if want_v else None
    flags = lib().orc_wht_fp_quant(_p(dy), _dtype_code(dy), M, N, b, _p(q_v), _p(s_v), _p(v))
    return q_v, s_v[0], v, flags


def dw_gemm(q_v, q_u, s_x, s_u, s_v, b: int, n_lo: int = 0, n_hi=None):
    q_v, q_u = _c(q_v, np.int8), _c(q_u, np.int8)
    M, N = q_v.shape
    K = q_u.shape[1]
    n_hi = N if n_hi is None else n_hi
    dw = np.zeros((N, K), np.float32)
    lib().orc_dw_gemm(_p(q_v), _p(q_u), M, N, K, float(s_x), float(s_u), float(s_v), b,
                      n_lo, n_hi, _p(dw))
    return dw


def qgemm_bwd_dw_wht(q_x, s_x, dy, b: int):
    q_x = _c(q_x, np.int8)
    dy = _c(dy)
    M, K = q_x.shape
    N = dy.shape[1]
    if dy.shape[0] != M:
        raise ValueError("dy: token count differs from q_x")
    _block(M, b, "tokens")
    s_x = _c(np.atleast_1d(s_x), np.float32)
    dw = np.empty((N, K), np.float32)
    su = np.zeros(1, np.float32)
    sv = np.zeros(1, np.float32)
    flags = lib().orc_qgemm_bwd_dw_wht(_p(q_x), _p(s_x), _p(dy), _dtype_code(dy), M, N, K, b,
                                       _p(dw), _p(su), _p(sv))
    return dw, su[0], sv[0], flags


def wht_fp_rows_quant(dy, b: int, s_w=None, want_v: bool = False):
    """g = dy * s_w[n] rotated along each row in blocks of b, per-tensor
    LSQ.  Returns (q, s, rotated values or None, flags)."""
    dy = _c(dy)
    M, N = dy.shape
    _block(N, b, "columns")
    q = np.empty((M, N), np.int8)
    s = np.zeros(1, np.float32)
    v = np.empty((M, N), np.float32) if want_v else None
    sw = None if s_w is None else _c(s_w, np.float32)
    flags = lib().orc_wht_fp_rows_quant(_p(dy), _dtype_code(dy), M, N, _p(sw), b, _p(q), _p(s),
                                        _p(v))
    return q, s[0], v, flags


def qgemm_bwd_dx_wht(dy, s_w, q_w, b: int):
    """Rotated input-gradient GEMM.  Returns (dx, s_g, s_h, flags)."""
    dy = _c(dy)
    q_w = _c(q_w, np.int8)
    M, N = dy.shape
    K = q_w.shape[1]
    _block(N, b, "columns")
    sw = _c(s_w, np.float32)
    dx = np.empty((M, K), np.float32)
    sg = np.zeros(1, np.float32)
    sh = np.zeros(1, np.float32)
    flags = lib().orc_qgemm_bwd_dx_wht(_p(dy), _dtype_code(dy), _p(sw), _p(q_w), M, N, K, b,
                                       _p(dx), _p(sg), _p(sh))
    return dx, sg[0], sh[0], flags


def exp_f(x: float) -> np.float32:
    """The attention softmax's binary32 exp (x <= 0)."""
    return np.float32(lib().orc_exp_f(x))


def attn_fwd(q, k, v, window=None):
    """Attention forward with an int8 P.V product.  q [Hq][T][d], k, v
    [Hkv][T][d] bf16 bit patterns (uint16); window None = plain causal.
    Returns (o [Hq][T][d] fp32, flags)."""
    q, k, v = _c(q, np.uint16), _c(k, np.uint16), _c(v, np.uint16)
    Hq, T, d = q.shape
    Hkv = k.shape[0]
    o = np.empty((Hq, T, d), np.float32)
    w = T if window is None else int(window)
    flags = lib().orc_attn_fwd(_p(q), _p(k), _p(v), Hq, Hkv, T, d, w, _p(o))
    if flags < 0:
        raise ValueError("attn_fwd: unsupported shape")
    return o, flags


def rmsnorm_fwd(x, g, eps: float = 1e-6):
    x, g = _c(x), _c(g)
    T, D = x.shape
    y = np.empty_like(x)
    rstd = np.empty(T, np.float32)
    flags = lib().orc_rmsnorm_fwd(_p(x), _p(g), _dtype_code(x), T, D, eps, _p(y), _p(rstd))
    return y, rstd, flags


def rmsnorm_bwd(x, g, rstd, dy):
    x, g, dy = _c(x), _c(g), _c(dy)
    rstd = _c(rstd, np.float32)
    T, D = x.shape
    dx = np.empty_like(x)
    dg = np.empty(D, np.float32)
    lib().orc_rmsnorm_bwd(_p(x), _p(g), _p(rstd), _p(dy), _dtype_code(x), T, D, _p(dx), _p(dg))
    return dx, dg


def grad_norm(v):
    v = _c(v, np.float32).reshape(-1)
    ss = np.zeros(1, np.float32)
    nrm = np.zeros(1, np.float32)
    flags = lib().orc_grad_norm(_p(v), v.size, _p(ss), _p(nrm))
    return ss[0], nrm[0], flags


# AdamW defaults of the pages (report §3.2 "Optimizer").
ADAMW_BETA1, ADAMW_BETA2, ADAMW_EPS, ADAMW_WD = 0.9, 0.95, 1e-8, 0.1
CLIP_MAX_NORM, SPIKE_THRESHOLD, SPIKE_SKIP_STEPS = 1.0, 5.0, 5


def adamw_bias_corrections(t: int, beta1: float = ADAMW_BETA1, beta2: float = ADAMW_BETA2):
    b1, b2 = C.c_float(), C.c_float()
    lib().orc_adamw_bias_corrections(t, beta1, beta2, C.byref(b1), C.byref(b2))
    return np.float32(b1.value), np.float32(b2.value)


def adamw_decide(norm: float, skip_state: int, max_norm: float = CLIP_MAX_NORM,
                 spike_threshold: float = SPIKE_THRESHOLD, skip_steps: int = SPIKE_SKIP_STEPS):
    """Returns (apply, clip, new_skip_state, flags)."""
    st = C.c_int32(skip_state)
    ap, cl = C.c_float(), C.c_float()
    fl = lib().orc_adamw_decide(norm, max_norm, spike_threshold, skip_steps, C.byref(st),
                                C.byref(ap), C.byref(cl))
    return np.float32(ap.value), np.float32(cl.value), int(st.value), int(fl)


def adamw_step(param, grad, m, v, lr: float, bc1: float, bc2: float, apply: float = 1.0,
               clip: float = 1.0, beta1: float = ADAMW_BETA1, beta2: float = ADAMW_BETA2,
               eps: float = ADAMW_EPS, wd: float = ADAMW_WD):
    """Returns updated copies (param, m, v); param bf16 (uint16) or fp32."""
    p = _c(param).copy()
    g = _c(grad)
    m2, v2 = _c(m, np.float32).copy(), _c(v, np.float32).copy()
    assert p.size == g.size == m2.size == v2.size
    lib().orc_adamw_step(_p(p), _dtype_code(p), _p(g), _dtype_code(g), _p(m2), _p(v2), p.size,
                         lr, beta1, beta2, eps, wd, bc1, bc2, apply, clip)
    return p, m2, v2


def _part_ptrs(parts):
    """Contiguous fp32 copies of the contributions and a C array of their
    addresses (the arrays are returned too, to keep them alive)."""
    arrs = [_c(p, np.float32).reshape(-1) for p in parts]
    n = arrs[0].size if arrs else 0
    if any(a.size != n for a in arrs):
        raise ValueError("contributions differ in length")
    ptrs = (C.c_void_p * max(len(arrs), 1))(*[a.ctypes.data for a in arrs])
    return arrs, ptrs, n


def ascending_sum(parts):
    """Running sum of the contributions in index order (App. A.2)."""
    arrs, ptrs, n = _part_ptrs(parts)
    out = np.zeros(n, np.float32)
    lib().orc_ascending_sum(ptrs, len(arrs), n, _p(out))
    return out


def average(x, k: int):
    """x * fl(1/k) (App. A.3)."""
    x = _c(x, np.float32).reshape(-1)
    out = np.zeros(x.size, np.float32)
    lib().orc_average(_p(x), x.size, int(k), _p(out))
    return out


def treefold(parts):
    """TreeFold over replica partials in replica order (App. A.1)."""
    arrs, ptrs, n = _part_ptrs(parts)
    if not 1 <= len(arrs) <= 64:
        raise ValueError("1..64 replicas")
    out = np.zeros(n, np.float32)
    lib().orc_treefold(ptrs, len(arrs), n, _p(out))
    return out


def dp_reduce(parts, replicas: int, shards: int, accum: int = 1, average: bool = True):
    """The whole exchange of one step (App. A): parts holds replicas*shards*
    accum contributions in mesh order (replica-major, then shard, then
    microbatch).  Returns (out, flags)."""
    arrs, ptrs, n = _part_ptrs(parts)
    if len(arrs) != replicas * shards * accum:
        raise ValueError("parts must hold replicas * shards * accum arrays")
    out = np.zeros(n, np.float32)
    fl = lib().orc_dp_reduce(ptrs, replicas, shards, accum, n, int(bool(average)), _p(out))
    if fl < 0:
        raise ValueError("dp_reduce: counts outside 1..64 contributions")
    return out, int(fl)


def prim_sweep(prim: int, first: int, count: int, out=None):
    """The model's primitive ``prim`` on the bit patterns first + i (uint32
    results; see orc_prim_sweep)."""
    o = np.empty(count, np.uint32) if out is None else out
    lib().orc_prim_sweep(prim, first & 0xFFFFFFFF, count, _p(o))
    return o


def sha256(data: bytes) -> bytes:
    buf = np.frombuffer(data, np.uint8) if len(data) else np.zeros(1, np.uint8)
    out = np.zeros(32, np.uint8)
    lib().orc_sha256(_p(buf), len(data), _p(out))
    return out.tobytes()


def merkle_root(a: np.ndarray) -> bytes:
    b = np.ascontiguousarray(a).view(np.uint8).reshape(-1)
    buf = b if b.size else np.zeros(1, np.uint8)
    out = np.zeros(32, np.uint8)
    lib().orc_merkle_root(_p(buf), b.size, _p(out))
    return out.tobytes()


_DT = {np.dtype(np.float32): F32, np.dtype(np.uint16): BF16, np.dtype(np.int8): I8,
       np.dtype(np.int32): I32, np.dtype(np.uint8): U8}


def tensor_digest(name: str, a: np.ndarray, code=None) -> bytes:
    """Digest of one tensor: SHA-256 over the typed header and the Merkle
    root of its raw bytes (the per-tensor part of hash_state)."""
    a = np.ascontiguousarray(a)
    code = _DT[a.dtype] if code is None else code
    buf = a.view(np.uint8).reshape(-1) if a.size else np.zeros(1, np.uint8)
    dims = np.array(a.shape if a.ndim else [0], np.int64)
    out = np.zeros(32, np.uint8)
    lib().orc_tensor_digest(_p(buf), a.nbytes, code, a.ndim, _p(dims), name.encode(), _p(out))
    return out.tobytes()


def hash_state(tensors):
    """tensors: list of (name, numpy array[, dtype code]).  bf16 arrays are
    uint16 and hash with the bf16 dtype code unless one is given."""
    n = len(tensors)
    arrs, names, dtypes, ndims, dims, nbytes = [], [], [], [], [], []
    for t in tensors:
        name, a = t[0], np.ascontiguousarray(t[1])
        code = t[2] if len(t) > 2 else _DT[a.dtype]
        arrs.append(a if a.size else np.zeros(1, a.dtype))
        names.append(name.encode())
        dtypes.append(code)
        ndims.append(a.ndim)
        dims.extend(a.shape)
        nbytes.append(a.nbytes)
    ptrs = (C.c_void_p * max(n, 1))(*[x.ctypes.data for x in arrs])
    nb = np.array(nbytes, np.uint64)
    dt = np.array(dtypes, np.int32)
    nd = np.array(ndims, np.int32)
    dm = np.array(dims if dims else [0], np.int64)
    nm = (C.c_char_p * max(n, 1))(*names)
    out = np.zeros(32, np.uint8)
    lib().orc_hash_state(n, ptrs, _p(nb), _p(dt), _p(nd), _p(dm), nm, _p(out))
    return out.tobytes()
