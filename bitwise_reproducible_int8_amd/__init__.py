"""Python binding of libbrq (argument marshalling only).

Every step of the path runs in libbrq's HIP kernels; this module checks
tensors, allocates outputs and workspaces with torch (device memory and
streams are all torch is used for), and calls the C ABI declared in
include/brq.h on torch's current stream.  There is no fallback: if the
shared library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbrq.so")

F32, BF16, I8, I32, U8 = 0, 1, 2, 3, 4
PER_TENSOR, PER_ROW = 0, 1
FLAG_NONFINITE = 1
OP_QUANTIZE, OP_QGEMM, OP_DW_WHT, OP_RMSNORM_BWD, OP_GRAD_NORM, OP_DY_BWD = 1, 2, 3, 4, 5, 6
OP_QUANTIZE_EXACT, OP_DX_WHT, OP_DY_ROWS_WHT, OP_QUANTIZE_X_WHT = 7, 8, 9, 10
MAX_CONTRACTION = 131071
DP_MAX_PARTS = 64
STATIC_SCRATCH_BYTES = 4 << 20
E_SCRATCH = -10
PRIM_SQRT, PRIM_RCP, PRIM_RSQRT, PRIM_BF16_CVT, PRIM_BF16_INT = 0, 1, 2, 3, 4

SYMBOLS = [
    "brq_workspace_size", "brq_quantize_lsq", "brq_quantize_lsq_exact", "brq_quantize_lsq_static",
    "brq_quantize_lsq_rows_multi", "brq_quantize_x_wht", "brq_qgemm_fwd", "brq_qgemm_bwd_dx",
    "brq_qgemm_bwd_dw_wht", "brq_wht_quant_x", "brq_wht_quant_dy", "brq_qgemm_dw",
    "brq_qgemm_fwd_ex", "brq_qgemm_bwd_dx_ex",
    "brq_quantize_dy_bwd", "brq_qgemm_bwd_dx_wht", "brq_wht_quant_dy_rows", "brq_attn_fwd",
    "brq_rmsnorm_fixed_fwd", "brq_rmsnorm_fixed_bwd", "brq_grad_norm",
    "brq_hash_workspace_size", "brq_hash_state", "brq_hash_digests_workspace_size",
    "brq_hash_tensor_digests", "brq_hash_combine", "brq_hash_tensor_leaves",
    "brq_hash_tensor_finish", "brq_adamw_bias_corrections",
    "brq_adamw_decide", "brq_adamw_step", "brq_dp_reduce", "brq_fp32_primitive", "brq_status_string",
    "brq_last_hip_error", "brq_spec_version",
]


class BrqError(RuntimeError):
    pass


class AdamWHparams(C.Structure):
    _fields_ = [("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float), ("eps", C.c_float),
                ("weight_decay", C.c_float), ("bias_correction1", C.c_float),
                ("bias_correction2", C.c_float)]


# AdamW, clipping and spike-protocol defaults of the report (§3.2 "Optimizer",
# §3.4.2)
ADAMW_BETA1, ADAMW_BETA2, ADAMW_EPS, ADAMW_WD = 0.9, 0.95, 1e-8, 0.1
CLIP_MAX_NORM, SPIKE_THRESHOLD, SPIKE_SKIP_STEPS = 1.0, 5.0, 5


class RowsJob(C.Structure):
    """One tensor of brq_quantize_lsq_rows_multi (struct brq_rows_job)."""
    _fields_ = [("x", C.c_void_p), ("x_dtype", C.c_int), ("rows", C.c_int64), ("cols", C.c_int64),
                ("q", C.c_void_p), ("q_t", C.c_void_p), ("scale", C.c_void_p),
                ("amax", C.c_void_p)]


class Tune(C.Structure):
    _fields_ = [("gemm_kernel", C.c_int), ("split_k", C.c_int), ("chunk_log2", C.c_int),
                ("rows_per_block", C.c_int)]


class TensorRef(C.Structure):
    _fields_ = [("data", C.c_void_p), ("dtype", C.c_int), ("ndim", C.c_int),
                ("dims", C.c_int64 * 8), ("name", C.c_char_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise BrqError(f"{LIB_PATH} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = C.CDLL(LIB_PATH)
        vp, i64, i32, sz, f32 = C.c_void_p, C.c_int64, C.c_int, C.c_size_t, C.c_float
        L.brq_workspace_size.restype = sz
        L.brq_workspace_size.argtypes = [i32, i64, i64, i64, i32, vp]
        L.brq_quantize_lsq.restype = i32
        L.brq_quantize_lsq.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
        L.brq_quantize_lsq_exact.restype = i32
        L.brq_quantize_lsq_exact.argtypes = L.brq_quantize_lsq.argtypes
        L.brq_quantize_lsq_static.restype = i32
        L.brq_quantize_lsq_static.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp]
        L.brq_quantize_lsq_rows_multi.restype = i32
        L.brq_quantize_lsq_rows_multi.argtypes = [vp, i32, vp, vp]
        L.brq_quantize_x_wht.restype = i32
        L.brq_quantize_x_wht.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp, vp, vp, vp, sz, vp, vp,
                                         vp]
        L.brq_qgemm_fwd.restype = i32
        L.brq_qgemm_fwd.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, vp, vp, sz, vp, vp]
        L.brq_qgemm_bwd_dx.restype = i32
        L.brq_qgemm_bwd_dx.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, sz, vp, vp]
        L.brq_qgemm_fwd_ex.restype = i32
        L.brq_qgemm_fwd_ex.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, vp, i32, vp, sz, vp, vp]
        L.brq_qgemm_bwd_dx_ex.restype = i32
        L.brq_qgemm_bwd_dx_ex.argtypes = [vp, vp, vp, i64, i64, i64, vp, i32, vp, sz, vp, vp]
        L.brq_qgemm_bwd_dw_wht.restype = i32
        L.brq_qgemm_bwd_dx_wht.restype = i32
        L.brq_qgemm_bwd_dx_wht.argtypes = [vp, i32, vp, vp, i64, i64, i64, i32, vp, vp, vp, vp,
                                           sz, vp, vp, vp]
        L.brq_attn_fwd.restype = i32
        L.brq_attn_fwd.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp, vp]
        L.brq_wht_quant_dy_rows.restype = i32
        L.brq_wht_quant_dy_rows.argtypes = [vp, i32, i64, i64, vp, i32, vp, vp, vp, sz, vp, vp,
                                            vp]
        L.brq_qgemm_bwd_dw_wht.argtypes = [vp, vp, vp, i32, i64, i64, i64, i32, vp, vp, vp, vp,
                                           sz, vp, vp, vp]
        L.brq_wht_quant_x.restype = i32
        L.brq_wht_quant_x.argtypes = [vp, i64, i64, i32, vp, vp, vp, sz, vp, vp]
        L.brq_wht_quant_dy.restype = i32
        L.brq_wht_quant_dy.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp, sz, vp, vp, vp]
        L.brq_qgemm_dw.restype = i32
        L.brq_qgemm_dw.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, vp, sz, vp, vp]
        L.brq_quantize_dy_bwd.restype = i32
        L.brq_quantize_dy_bwd.argtypes = [vp, i32, i64, i64, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp,
                                          vp, vp]
        L.brq_rmsnorm_fixed_fwd.restype = i32
        L.brq_rmsnorm_fixed_fwd.argtypes = [vp, vp, i32, i64, i64, f32, vp, vp, vp, vp, vp]
        L.brq_rmsnorm_fixed_bwd.restype = i32
        L.brq_rmsnorm_fixed_bwd.argtypes = [vp, vp, vp, vp, i32, i64, i64, vp, vp, vp, sz, vp, vp]
        L.brq_grad_norm.restype = i32
        L.brq_grad_norm.argtypes = [vp, i64, vp, vp, vp, sz, vp, vp, vp]
        L.brq_hash_workspace_size.restype = sz
        L.brq_hash_workspace_size.argtypes = [vp, i32]
        L.brq_hash_state.restype = i32
        L.brq_hash_state.argtypes = [vp, i32, vp, vp, sz, vp]
        L.brq_hash_digests_workspace_size.restype = sz
        L.brq_hash_digests_workspace_size.argtypes = [vp, i32]
        L.brq_hash_tensor_digests.restype = i32
        L.brq_hash_tensor_digests.argtypes = [vp, i32, vp, vp, sz, vp]
        L.brq_hash_combine.restype = i32
        L.brq_hash_combine.argtypes = [vp, i32, vp, vp]
        L.brq_hash_tensor_leaves.restype = i32
        L.brq_hash_tensor_leaves.argtypes = [vp, i32, vp, sz, vp]
        L.brq_hash_tensor_finish.restype = i32
        L.brq_hash_tensor_finish.argtypes = [vp, i32, vp, vp, sz, vp]
        L.brq_adamw_bias_corrections.restype = i32
        L.brq_adamw_bias_corrections.argtypes = [i64, C.c_float, C.c_float, vp, vp]
        L.brq_adamw_decide.restype = i32
        L.brq_adamw_decide.argtypes = [vp, C.c_float, C.c_float, i32, vp, vp, vp, vp]
        L.brq_adamw_step.restype = i32
        L.brq_adamw_step.argtypes = [vp, i32, vp, i32, vp, vp, i64, vp, vp, vp]
        L.brq_dp_reduce.restype = i32
        L.brq_dp_reduce.argtypes = [vp, i32, i32, i32, i64, i32, vp, vp, vp]
        L.brq_fp32_primitive.restype = i32
        L.brq_fp32_primitive.argtypes = [i32, C.c_uint32, i64, vp, vp]
        L.brq_status_string.restype = C.c_char_p
        L.brq_status_string.argtypes = [i32]
        L.brq_last_hip_error.restype = i32
        L.brq_last_hip_error.argtypes = []
        L.brq_spec_version.restype = i32
        L.brq_spec_version.argtypes = []
        _lib = L
    return _lib


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------
def _check(status: int, what: str):
    if status != 0:
        msg = lib().brq_status_string(status).decode()
        extra = f" (hipError {lib().brq_last_hip_error()})" if status == -8 else ""
        raise BrqError(f"{what}: {msg}{extra}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _tune(t):
    if t is None:
        return None
    if isinstance(t, Tune):
        return C.byref(t)
    return C.byref(Tune(**t))


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise BrqError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise BrqError(f"{name} must be contiguous")


def _out(t, shape, dtype, name):
    """Check a caller-provided output tensor: device, contiguous, exact shape
    and dtype (a wrong shape would let a kernel write past its end)."""
    _dev(t, name)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise BrqError(f"{name}: expected {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    return t


def _fp_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise BrqError(f"unsupported dtype {t.dtype}")


_HASH_CODES = {torch.float32: F32, torch.bfloat16: BF16, torch.int8: I8, torch.int32: I32,
               torch.uint8: U8}


class Workspace:
    """Growable device byte buffers, one per (device, stream): calls on one
    stream are ordered and may share a buffer; calls on different streams
    get different buffers, so they may overlap (a caller that orders calls
    across streams itself may pass ``ws=`` instead).  A buffer is allocated
    on the stream it serves, and growing it frees the old one on that
    stream, after the calls already issued there."""

    def __init__(self):
        self.buf = {}

    def get(self, nbytes: int, device) -> torch.Tensor:
        dev = torch.device(device)
        key = (dev, torch.cuda.current_stream(dev).cuda_stream)
        b = self.buf.get(key)
        if b is None or b.numel() < nbytes:
            b = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
            self.buf[key] = b
        return b


_WS = Workspace()


def workspace_size(op: int, a: int, b: int = 0, c: int = 0, block: int = 0, tune=None) -> int:
    return int(lib().brq_workspace_size(op, a, b, c, block, _tune(tune)))


def _ws(nbytes, device, ws):
    if ws is not None:
        if ws.numel() < nbytes:
            raise BrqError(f"workspace too small: {ws.numel()} < {nbytes}")
        return ws
    return _WS.get(nbytes, device)


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def quantize_lsq(x, per_row=False, col_mul=None, want_t=False, tune=None, ws=None, flags=None,
                 out=None, exact=False):
    """LSQ int8 quantisation.  Returns (q, q_t or None, scale, amax).
    ``out`` may hold preallocated (q, q_t, scale, amax); a None entry is
    allocated here (q_t only when want_t).  ``exact`` selects
    brq_quantize_lsq_exact (the statistic summed exactly, rounded once)."""
    _dev(x, "x")
    rows, cols = x.shape
    ns = rows if per_row else 1
    q, q_t, scale, amax = out if out is not None else (None, None, None, None)
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    if q_t is None and want_t:
        q_t = torch.empty((cols, rows), dtype=torch.int8, device=x.device)
    if scale is None:
        scale = torch.empty(ns, dtype=torch.float32, device=x.device)
    if amax is None:
        amax = torch.empty(ns, dtype=torch.float32, device=x.device)
    for t, shape, dt, name in ((q, (rows, cols), torch.int8, "q"), (scale, (ns,), torch.float32, "scale"),
                               (amax, (ns,), torch.float32, "amax")):
        _dev(t, name)
        if tuple(t.shape) != shape or t.dtype != dt:
            raise BrqError(f"{name}: expected {dt} {shape}, got {t.dtype} {tuple(t.shape)}")
    if q_t is not None:
        _dev(q_t, "q_t")
        if tuple(q_t.shape) != (cols, rows) or q_t.dtype != torch.int8:
            raise BrqError("q_t: expected int8 (cols, rows)")
    if col_mul is not None:
        _dev(col_mul, "col_mul")
    need = workspace_size(OP_QUANTIZE_EXACT if exact else OP_QUANTIZE, rows, cols, tune=tune)
    w = _ws(need, x.device, ws)
    fn = lib().brq_quantize_lsq_exact if exact else lib().brq_quantize_lsq
    _check(fn(_ptr(x), _fp_code(x), rows, cols, PER_ROW if per_row else PER_TENSOR,
              _ptr(col_mul), _ptr(q), _ptr(q_t), _ptr(scale), _ptr(amax),
              _ptr(w), w.numel(), _ptr(flags), _tune(tune), _stream()),
           "quantize_lsq_exact" if exact else "quantize_lsq")
    return q, q_t, scale, amax


def quantize_lsq_rows_multi(xs, want_t=True, flags=None, outs=None):
    """Per-row LSQ quantisation of several tensors in one call
    (brq_quantize_lsq_rows_multi).  Returns a list of (q, q_t or None,
    scale, amax), each equal to quantize_lsq(x, per_row=True, want_t=...);
    ``outs`` may hold such tuples preallocated (None entries allocated)."""
    res = []
    jobs = (RowsJob * max(len(xs), 1))()
    for k, x in enumerate(xs):
        _dev(x, f"xs[{k}]")
        rows, cols = x.shape
        q, q_t, scale, amax = outs[k] if outs is not None else (None, None, None, None)
        if q is None:
            q = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
        if q_t is None and want_t:
            q_t = torch.empty((cols, rows), dtype=torch.int8, device=x.device)
        if scale is None:
            scale = torch.empty(rows, dtype=torch.float32, device=x.device)
        if amax is None:
            amax = torch.empty(rows, dtype=torch.float32, device=x.device)
        for t, shape, dt, name in ((q, (rows, cols), torch.int8, "q"),
                                   (scale, (rows,), torch.float32, "scale"),
                                   (amax, (rows,), torch.float32, "amax")):
            _dev(t, name)
            if tuple(t.shape) != shape or t.dtype != dt:
                raise BrqError(f"{name}[{k}]: expected {dt} {shape}, got {t.dtype} {tuple(t.shape)}")
        if q_t is not None:
            _dev(q_t, "q_t")
            if tuple(q_t.shape) != (cols, rows) or q_t.dtype != torch.int8:
                raise BrqError(f"q_t[{k}]: expected int8 (cols, rows)")
        jobs[k] = RowsJob(_ptr(x), _fp_code(x), rows, cols, _ptr(q), _ptr(q_t), _ptr(scale),
                          _ptr(amax))
        res.append((q, q_t, scale, amax))
    _check(lib().brq_quantize_lsq_rows_multi(jobs, len(xs), _ptr(flags), _stream()),
           "quantize_lsq_rows_multi")
    return res


def quantize_x_wht(x, block, tune=None, ws=None, flags=None, out=None):
    """Per-tensor LSQ codes of x and the integer rotation of those codes along
    tokens (brq_quantize_x_wht).  Returns (q_x, s_x, amax_x, q_ut, s_u), the
    results of quantize_lsq(x) then wht_quant_x(q_x, block); ``out`` may hold
    them preallocated (None entries allocated)."""
    _dev(x, "x")
    M, K = x.shape
    q_x, s_x, amax_x, q_ut, s_u = out if out is not None else (None,) * 5
    dev = x.device
    q_x = torch.empty((M, K), dtype=torch.int8, device=dev) if q_x is None else q_x
    q_ut = torch.empty((K, M), dtype=torch.int8, device=dev) if q_ut is None else q_ut
    s_x = torch.empty(1, dtype=torch.float32, device=dev) if s_x is None else s_x
    amax_x = torch.empty(1, dtype=torch.float32, device=dev) if amax_x is None else amax_x
    s_u = torch.empty(1, dtype=torch.float32, device=dev) if s_u is None else s_u
    for t, shape, dt, name in ((q_x, (M, K), torch.int8, "q_x"), (q_ut, (K, M), torch.int8, "q_ut"),
                               (s_x, (1,), torch.float32, "s_x"), (amax_x, (1,), torch.float32, "amax_x"),
                               (s_u, (1,), torch.float32, "s_u")):
        _dev(t, name)
        if tuple(t.shape) != shape or t.dtype != dt:
            raise BrqError(f"{name}: expected {dt} {shape}, got {t.dtype} {tuple(t.shape)}")
    need = workspace_size(OP_QUANTIZE_X_WHT, M, K, 0, block, tune=tune)
    w = _ws(need, dev, ws)
    _check(lib().brq_quantize_x_wht(_ptr(x), _fp_code(x), M, K, block, _ptr(q_x), _ptr(s_x),
                                    _ptr(amax_x), _ptr(q_ut), _ptr(s_u), _ptr(w), w.numel(),
                                    _ptr(flags), _tune(tune), _stream()), "quantize_x_wht")
    return q_x, s_x, amax_x, q_ut, s_u


def qgemm_fwd(q_x, s_x, q_w, s_w, tune=None, out=None, ws=None, out_dtype=torch.float32):
    """y = dequant(q_x q_w^T); out_dtype torch.float32 (the definition) or
    torch.bfloat16 (each value rounded once to bf16)."""
    _dev(q_x, "q_x"); _dev(q_w, "q_w")
    M, K = q_x.shape
    N = q_w.shape[0]
    if q_w.shape[1] != K:
        raise BrqError("q_w: contraction length differs from q_x")
    y = _out(out, (M, N), out_dtype, "y") if out is not None else \
        torch.empty((M, N), dtype=out_dtype, device=q_x.device)
    need = workspace_size(OP_QGEMM, M, N, K, tune=tune)
    w = _ws(need, q_x.device, ws) if need else None
    if out_dtype == torch.float32:
        st = lib().brq_qgemm_fwd(_ptr(q_x), _ptr(s_x), _ptr(q_w), _ptr(s_w), int(s_w.numel() > 1),
                                 M, N, K, _ptr(y), _ptr(w), 0 if w is None else w.numel(),
                                 _tune(tune), _stream())
    else:
        st = lib().brq_qgemm_fwd_ex(_ptr(q_x), _ptr(s_x), _ptr(q_w), _ptr(s_w),
                                    int(s_w.numel() > 1), M, N, K, _ptr(y), _fp_code(y), _ptr(w),
                                    0 if w is None else w.numel(), _tune(tune), _stream())
    _check(st, "qgemm_fwd")
    return y


def qgemm_bwd_dx(q_g, s_g, q_wt, tune=None, out=None, ws=None, out_dtype=torch.float32):
    """dx = dequant(q_g q_wt^T); out_dtype as qgemm_fwd."""
    _dev(q_g, "q_g"); _dev(q_wt, "q_wt")
    M, N = q_g.shape
    K = q_wt.shape[0]
    if q_wt.shape[1] != N:
        raise BrqError("q_wt: contraction length differs from q_g")
    dx = _out(out, (M, K), out_dtype, "dx") if out is not None else \
        torch.empty((M, K), dtype=out_dtype, device=q_g.device)
    need = workspace_size(OP_QGEMM, M, K, N, tune=tune)
    w = _ws(need, q_g.device, ws) if need else None
    if out_dtype == torch.float32:
        st = lib().brq_qgemm_bwd_dx(_ptr(q_g), _ptr(s_g), _ptr(q_wt), M, N, K, _ptr(dx), _ptr(w),
                                    0 if w is None else w.numel(), _tune(tune), _stream())
    else:
        st = lib().brq_qgemm_bwd_dx_ex(_ptr(q_g), _ptr(s_g), _ptr(q_wt), M, N, K, _ptr(dx),
                                       _fp_code(dx), _ptr(w), 0 if w is None else w.numel(),
                                       _tune(tune), _stream())
    _check(st, "qgemm_bwd_dx")
    return dx


def qgemm_bwd_dw_wht(q_x, s_x, dy, block, tune=None, out=None, ws=None, flags=None,
                     return_codes=False):
    """Returns (dw, s_u, s_v) and, with return_codes, also (q_ut, q_vt): the
    rotated codes the call left at the start of its workspace."""
    _dev(q_x, "q_x"); _dev(dy, "dy")
    M, K = q_x.shape
    N = dy.shape[1]
    if dy.shape[0] != M:
        raise BrqError("dy: token count differs from q_x")
    dw = _out(out, (N, K), torch.float32, "dw") if out is not None else \
        torch.empty((N, K), dtype=torch.float32, device=q_x.device)
    s_u = torch.empty(1, dtype=torch.float32, device=q_x.device)
    s_v = torch.empty(1, dtype=torch.float32, device=q_x.device)
    need = workspace_size(OP_DW_WHT, M, N, K, block, tune=tune)
    w = _ws(need, q_x.device, ws)
    _check(lib().brq_qgemm_bwd_dw_wht(_ptr(q_x), _ptr(s_x), _ptr(dy), _fp_code(dy), M, N, K, block,
                                      _ptr(dw), _ptr(s_u), _ptr(s_v), _ptr(w), w.numel(),
                                      _ptr(flags), _tune(tune), _stream()), "qgemm_bwd_dw_wht")
    if not return_codes:
        return dw, s_u, s_v
    off = (K * M + 255) // 256 * 256
    q_ut = w[:K * M].view(torch.int8).view(K, M).clone()
    q_vt = w[off:off + N * M].view(torch.int8).view(N, M).clone()
    return dw, s_u, s_v, q_ut, q_vt


def qgemm_bwd_dx_wht(dy, s_w, q_w, block, tune=None, out=None, ws=None, flags=None,
                     return_codes=False):
    """Input-gradient GEMM with the rotation along n.  Returns (dx, s_g, s_h)
    and, with return_codes, also (q_ht [K][N], q_g [M][N]): the rotated codes
    the call left at the start of its workspace."""
    _dev(dy, "dy"); _dev(s_w, "s_w"); _dev(q_w, "q_w")
    M, N = dy.shape
    K = q_w.shape[1]
    if q_w.shape[0] != N or s_w.numel() != N:
        raise BrqError("q_w / s_w: output-channel count differs from dy")
    dx = _out(out, (M, K), torch.float32, "dx") if out is not None else \
        torch.empty((M, K), dtype=torch.float32, device=dy.device)
    s_g = torch.empty(1, dtype=torch.float32, device=dy.device)
    s_h = torch.empty(1, dtype=torch.float32, device=dy.device)
    need = workspace_size(OP_DX_WHT, M, N, K, block, tune=tune)
    w = _ws(need, dy.device, ws)
    _check(lib().brq_qgemm_bwd_dx_wht(_ptr(dy), _fp_code(dy), _ptr(s_w), _ptr(q_w), M, N, K,
                                      block, _ptr(dx), _ptr(s_g), _ptr(s_h), _ptr(w), w.numel(),
                                      _ptr(flags), _tune(tune), _stream()), "qgemm_bwd_dx_wht")
    if not return_codes:
        return dx, s_g, s_h
    off = (K * N + 255) // 256 * 256
    q_ht = w[:K * N].view(torch.int8).view(K, N).clone()
    q_g = w[off:off + M * N].view(torch.int8).view(M, N).clone()
    return dx, s_g, s_h, q_ht, q_g


def attn_fwd(q, k, v, window=None, out=None, flags=None):
    """Attention forward with an int8 P.V product.  q [Hq][T][d], k, v
    [Hkv][T][d] bf16; window None = plain causal.  Returns o [Hq][T][d] fp32."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
        if t.dtype != torch.bfloat16 or t.dim() != 3:
            raise BrqError(f"{n}: expected bf16 [heads][T][d]")
    Hq, T, d = q.shape
    Hkv = k.shape[0]
    if tuple(k.shape) != (Hkv, T, d) or tuple(v.shape) != (Hkv, T, d):
        raise BrqError("k / v: expected [Hkv][T][d] like q")
    o = _out(out, (Hq, T, d), torch.float32, "o") if out is not None else \
        torch.empty((Hq, T, d), dtype=torch.float32, device=q.device)
    w = max(T, 1) if window is None else int(window)
    _check(lib().brq_attn_fwd(_ptr(q), _ptr(k), _ptr(v), Hq, Hkv, T, d, w, _ptr(o), _ptr(flags),
                              None, _stream()), "attn_fwd")
    return o


def wht_quant_dy_rows(dy, s_w, block, tune=None, ws=None, flags=None, out=None):
    """Rows rotation of dy * s_w and its per-tensor codes: (q_g [M][N], s_g)."""
    _dev(dy, "dy"); _dev(s_w, "s_w")
    M, N = dy.shape
    q_g, s_g = out if out is not None else (None, None)
    if q_g is None:
        q_g = torch.empty((M, N), dtype=torch.int8, device=dy.device)
    if s_g is None:
        s_g = torch.empty(1, dtype=torch.float32, device=dy.device)
    need = workspace_size(OP_DY_ROWS_WHT, M, N, tune=tune)
    w = _ws(need, dy.device, ws)
    _check(lib().brq_wht_quant_dy_rows(_ptr(dy), _fp_code(dy), M, N, _ptr(s_w), block, _ptr(q_g),
                                       _ptr(s_g), _ptr(w), w.numel(), _ptr(flags), _tune(tune),
                                       _stream()), "wht_quant_dy_rows")
    return q_g, s_g


def wht_quant_x(q_x, block, tune=None, ws=None, out=None):
    """Returns (q_ut [K][M], s_u); ``out`` may hold preallocated (q_ut, s_u)."""
    _dev(q_x, "q_x")
    M, K = q_x.shape
    q_ut, s_u = out if out is not None else (None, None)
    q_ut = torch.empty((K, M), dtype=torch.int8, device=q_x.device) if q_ut is None else q_ut
    s_u = torch.empty(1, dtype=torch.float32, device=q_x.device) if s_u is None else s_u
    _dev(q_ut, "q_ut")
    if tuple(q_ut.shape) != (K, M) or q_ut.dtype != torch.int8:
        raise BrqError("q_ut: expected int8 (K, M)")
    need = workspace_size(OP_DW_WHT, M, 64, K, block, tune=tune)
    w = _ws(need, q_x.device, ws)
    _check(lib().brq_wht_quant_x(_ptr(q_x), M, K, block, _ptr(q_ut), _ptr(s_u), _ptr(w), w.numel(),
                                 _tune(tune), _stream()), "wht_quant_x")
    return q_ut, s_u


def wht_quant_dy(dy, block, tune=None, ws=None, flags=None, out=None):
    """Returns (q_vt [N][M], s_v); ``out`` may hold preallocated (q_vt, s_v)."""
    _dev(dy, "dy")
    M, N = dy.shape
    q_vt, s_v = out if out is not None else (None, None)
    q_vt = torch.empty((N, M), dtype=torch.int8, device=dy.device) if q_vt is None else q_vt
    s_v = torch.empty(1, dtype=torch.float32, device=dy.device) if s_v is None else s_v
    _dev(q_vt, "q_vt")
    if tuple(q_vt.shape) != (N, M) or q_vt.dtype != torch.int8:
        raise BrqError("q_vt: expected int8 (N, M)")
    need = workspace_size(OP_DW_WHT, M, N, 64, block, tune=tune)
    w = _ws(need, dy.device, ws)
    _check(lib().brq_wht_quant_dy(_ptr(dy), _fp_code(dy), M, N, block, _ptr(q_vt), _ptr(s_v),
                                  _ptr(w), w.numel(), _ptr(flags), _tune(tune), _stream()),
           "wht_quant_dy")
    return q_vt, s_v


def quantize_dy_bwd(dy, s_w, block, tune=None, ws=None, flags=None, out=None):
    """Both backward codes of dY: returns (q_g [M][N], s_g, amax_g, q_vt [N][M],
    s_v).  ``out`` may hold preallocated tensors in that order (None entries
    are allocated here)."""
    _dev(dy, "dy"); _dev(s_w, "s_w")
    M, N = dy.shape
    if s_w.numel() != N or s_w.dtype != torch.float32:
        raise BrqError("s_w: expected fp32 [N]")
    o = list(out) if out is not None else [None] * 5
    shapes = [((M, N), torch.int8), ((1,), torch.float32), ((1,), torch.float32),
              ((N, M), torch.int8), ((1,), torch.float32)]
    names = ["q_g", "s_g", "amax_g", "q_vt", "s_v"]
    for i, ((shp, dt), nm) in enumerate(zip(shapes, names)):
        o[i] = torch.empty(shp, dtype=dt, device=dy.device) if o[i] is None else _out(o[i], shp, dt, nm)
    need = workspace_size(OP_DY_BWD, M, N, 0, block, tune=tune)
    w = _ws(need, dy.device, ws)
    _check(lib().brq_quantize_dy_bwd(_ptr(dy), _fp_code(dy), M, N, _ptr(s_w), block, _ptr(o[0]),
                                     _ptr(o[1]), _ptr(o[2]), _ptr(o[3]), _ptr(o[4]), _ptr(w),
                                     w.numel(), _ptr(flags), _tune(tune), _stream()),
           "quantize_dy_bwd")
    return tuple(o)


def qgemm_dw(q_vt, q_ut, s_x, s_u, s_v, block, tune=None, out=None, ws=None):
    _dev(q_vt, "q_vt"); _dev(q_ut, "q_ut")
    N, M = q_vt.shape
    K = q_ut.shape[0]
    if q_ut.shape[1] != M:
        raise BrqError("q_ut: token count differs from q_vt")
    dw = _out(out, (N, K), torch.float32, "dw") if out is not None else \
        torch.empty((N, K), dtype=torch.float32, device=q_vt.device)
    need = workspace_size(OP_QGEMM, N, K, M, tune=tune)
    w = _ws(need, q_vt.device, ws) if need else None
    _check(lib().brq_qgemm_dw(_ptr(q_vt), _ptr(q_ut), _ptr(s_x), _ptr(s_u), _ptr(s_v), M, N, K,
                              block, _ptr(dw), _ptr(w), 0 if w is None else w.numel(),
                              _tune(tune), _stream()), "qgemm_dw")
    return dw


def rmsnorm_fixed_fwd(x, g, eps=1e-6, flags=None, tune=None, out=None):
    """Returns (y, rstd); ``out`` may hold preallocated (y, rstd)."""
    _dev(x, "x"); _dev(g, "g")
    T, D = x.shape
    y, rstd = out if out is not None else (None, None)
    y = torch.empty_like(x) if y is None else y
    rstd = torch.empty(T, dtype=torch.float32, device=x.device) if rstd is None else rstd
    _dev(y, "y"); _dev(rstd, "rstd")
    if y.shape != x.shape or y.dtype != x.dtype or rstd.numel() != T:
        raise BrqError("rmsnorm_fixed_fwd: output shapes")
    _check(lib().brq_rmsnorm_fixed_fwd(_ptr(x), _ptr(g), _fp_code(x), T, D, eps, _ptr(y),
                                       _ptr(rstd), _ptr(flags), _tune(tune), _stream()),
           "rmsnorm_fixed_fwd")
    return y, rstd


def rmsnorm_fixed_bwd(x, g, rstd, dy, tune=None, ws=None, out=None):
    """Returns (dx, dg); ``out`` may hold preallocated (dx, dg)."""
    _dev(x, "x"); _dev(g, "g"); _dev(rstd, "rstd"); _dev(dy, "dy")
    T, D = x.shape
    dx, dg = out if out is not None else (None, None)
    dx = torch.empty_like(x) if dx is None else dx
    dg = torch.empty(D, dtype=torch.float32, device=x.device) if dg is None else dg
    _dev(dx, "dx"); _dev(dg, "dg")
    if dx.shape != x.shape or dx.dtype != x.dtype or dg.numel() != D or dg.dtype != torch.float32:
        raise BrqError("rmsnorm_fixed_bwd: output shapes")
    need = workspace_size(OP_RMSNORM_BWD, T, D, tune=tune)
    w = _ws(need, x.device, ws)
    _check(lib().brq_rmsnorm_fixed_bwd(_ptr(x), _ptr(g), _ptr(rstd), _ptr(dy), _fp_code(x), T, D,
                                       _ptr(dx), _ptr(dg), _ptr(w), w.numel(), _tune(tune),
                                       _stream()), "rmsnorm_fixed_bwd")
    return dx, dg


def grad_norm(v, flags=None, tune=None, ws=None, out=None):
    _dev(v, "v")
    if v.dtype != torch.float32:
        raise BrqError("grad_norm takes fp32 gradients")
    n = v.numel()
    res = out if out is not None else torch.empty(2, dtype=torch.float32, device=v.device)
    need = workspace_size(OP_GRAD_NORM, n, tune=tune)
    w = _ws(need, v.device, ws)
    _check(lib().brq_grad_norm(_ptr(v), n, res.data_ptr(), res.data_ptr() + 4, _ptr(w), w.numel(),
                               _ptr(flags), _tune(tune), _stream()), "grad_norm")
    return res[0], res[1]


def _refs(tensors):
    refs = (TensorRef * max(len(tensors), 1))()
    names = []
    for i, t in enumerate(tensors):
        name, a = t[0], t[1]
        _dev(a, name)
        code = t[2] if len(t) > 2 else _HASH_CODES[a.dtype]
        if a.dim() > 8:
            raise BrqError("at most 8 dims")
        nb = name.encode()
        names.append(nb)
        refs[i].data = a.data_ptr() if a.numel() else None
        refs[i].dtype = code
        refs[i].ndim = a.dim()
        for d in range(a.dim()):
            refs[i].dims[d] = a.shape[d]
        refs[i].name = nb
    return refs, names


def hash_state_workspace_size(tensors) -> int:
    refs, _ = _refs(tensors)
    return int(lib().brq_hash_workspace_size(refs, len(tensors)))


def hash_state(tensors, ws=None, out=None):
    """tensors: list of (name, device tensor[, dtype code]).  Returns the
    32-byte state digest as a device uint8 tensor."""
    refs, _keep = _refs(tensors)
    dev = tensors[0][1].device if tensors else torch.device("cuda")
    need = int(lib().brq_hash_workspace_size(refs, len(tensors)))
    w = _ws(need, dev, ws)
    digest = out if out is not None else torch.empty(32, dtype=torch.uint8, device=dev)
    _check(lib().brq_hash_state(refs, len(tensors), _ptr(digest), _ptr(w), w.numel(), _stream()),
           "hash_state")
    return digest


def hash_digests_workspace_size(tensors) -> int:
    refs, _ = _refs(tensors)
    return int(lib().brq_hash_digests_workspace_size(refs, len(tensors)))


def hash_tensor_digests(tensors, out, ws=None):
    """Tensor digests of ``tensors`` (list of (name, device tensor[, dtype
    code])) into ``out``, a device uint8 tensor of 32 * len(tensors) bytes."""
    refs, _keep = _refs(tensors)
    _dev(out, "out")
    if out.dtype != torch.uint8 or out.numel() != 32 * len(tensors):
        raise BrqError("out: expected uint8 [32 * n]")
    need = int(lib().brq_hash_digests_workspace_size(refs, len(tensors)))
    w = _ws(need, out.device, ws)
    _check(lib().brq_hash_tensor_digests(refs, len(tensors), _ptr(out), _ptr(w), w.numel(),
                                         _stream()), "hash_tensor_digests")
    return out


def hash_tensor_leaves(tensors, ws):
    """First stage of hash_tensor_digests: the leaf digests of ``tensors``
    into ``ws`` (a device workspace of hash_digests_workspace_size bytes),
    on the current stream.  The only stage that reads the tensors."""
    refs, _keep = _refs(tensors)
    _dev(ws, "ws")
    need = int(lib().brq_hash_digests_workspace_size(refs, len(tensors)))
    w = _ws(need, ws.device, ws)
    _check(lib().brq_hash_tensor_leaves(refs, len(tensors), _ptr(w), w.numel(), _stream()),
           "hash_tensor_leaves")


def hash_tensor_finish(tensors, out, ws):
    """Second stage: every level above the leaves and the tensor digests
    into ``out`` (uint8 [32 * n]), on the current stream, reading only
    ``ws`` as the first stage left it."""
    refs, _keep = _refs(tensors)
    _dev(out, "out"); _dev(ws, "ws")
    if out.dtype != torch.uint8 or out.numel() != 32 * len(tensors):
        raise BrqError("out: expected uint8 [32 * n]")
    need = int(lib().brq_hash_digests_workspace_size(refs, len(tensors)))
    w = _ws(need, ws.device, ws)
    _check(lib().brq_hash_tensor_finish(refs, len(tensors), _ptr(out), _ptr(w), w.numel(),
                                        _stream()), "hash_tensor_finish")
    return out


def hash_combine(digests, out=None):
    """State digest: SHA-256 of the concatenated 32-byte tensor digests."""
    _dev(digests, "digests")
    if digests.dtype != torch.uint8 or digests.numel() % 32:
        raise BrqError("digests: expected uint8 [32 * n]")
    d = out if out is not None else torch.empty(32, dtype=torch.uint8, device=digests.device)
    _out(d, (32,), torch.uint8, "out")
    _check(lib().brq_hash_combine(_ptr(digests), digests.numel() // 32, _ptr(d), _stream()),
           "hash_combine")
    return d


# --------------------------------------------------------------------------
# optimizer step
# --------------------------------------------------------------------------
def adamw_bias_corrections(t: int, beta1: float = ADAMW_BETA1, beta2: float = ADAMW_BETA2):
    """(1 - beta1^t, 1 - beta2^t) as binary32, computed by libbrq on the host."""
    b1, b2 = C.c_float(), C.c_float()
    _check(lib().brq_adamw_bias_corrections(int(t), beta1, beta2, C.byref(b1), C.byref(b2)),
           "adamw_bias_corrections")
    return b1.value, b2.value


def adamw_decide(norm, skip_state, out=None, max_norm: float = CLIP_MAX_NORM,
                 spike_threshold: float = SPIKE_THRESHOLD, skip_steps: int = SPIKE_SKIP_STEPS,
                 flags=None):
    """Step decision on the device: norm is a device fp32 tensor holding the
    pre-clip global norm (first element); skip_state a device int32 [1].
    Returns ctl, a device fp32 [2] = (apply, clip)."""
    _dev(norm, "norm")
    if norm.dtype != torch.float32 or norm.numel() < 1:
        raise BrqError("norm: expected a device fp32 tensor")
    _out(skip_state, (1,), torch.int32, "skip_state")
    ctl = _out(out, (2,), torch.float32, "ctl") if out is not None else \
        torch.empty(2, dtype=torch.float32, device=norm.device)
    _check(lib().brq_adamw_decide(norm.data_ptr(), max_norm, spike_threshold, skip_steps,
                                  skip_state.data_ptr(), ctl.data_ptr(), _ptr(flags), _stream()),
           "adamw_decide")
    return ctl


def adamw_step(param, grad, m, v, ctl, lr: float, bias_corrections, beta1: float = ADAMW_BETA1,
               beta2: float = ADAMW_BETA2, eps: float = ADAMW_EPS,
               weight_decay: float = ADAMW_WD):
    """In-place AdamW update of param (bf16 or fp32) and the fp32 moments m, v
    from grad (fp32 or bf16), under the decision ctl of adamw_decide."""
    for t, nm in ((param, "param"), (grad, "grad"), (m, "m"), (v, "v"), (ctl, "ctl")):
        _dev(t, nm)
    n = param.numel()
    if grad.numel() != n or m.numel() != n or v.numel() != n:
        raise BrqError("adamw_step: param, grad, m, v must have the same size")
    if m.dtype != torch.float32 or v.dtype != torch.float32 or ctl.dtype != torch.float32 \
            or ctl.numel() != 2:
        raise BrqError("adamw_step: m, v fp32 and ctl fp32 [2]")
    bc1, bc2 = bias_corrections
    hp = AdamWHparams(lr, beta1, beta2, eps, weight_decay, bc1, bc2)
    _check(lib().brq_adamw_step(param.data_ptr(), _fp_code(param), grad.data_ptr(), _fp_code(grad),
                                m.data_ptr(), v.data_ptr(), n, C.byref(hp), ctl.data_ptr(),
                                _stream()), "adamw_step")


# --------------------------------------------------------------------------
# deterministic gradient exchange
# --------------------------------------------------------------------------
def dp_reduce(parts, replicas: int, shards: int, accum: int = 1, average: bool = True,
              out=None, flags=None):
    """The exchange of one step over contributions resident on this device
    (brq_dp_reduce): parts is a list of replicas*shards*accum fp32 device
    tensors of equal size in mesh order (replica-major, then shard, then
    microbatch).  Returns out (fp32, the parts' shape); ``out`` may be one of
    the parts."""
    P = replicas * shards * accum
    if len(parts) != P or P < 1:
        raise BrqError("parts must hold replicas * shards * accum tensors")
    for j, t in enumerate(parts):
        _dev(t, f"parts[{j}]")
        if t.dtype != torch.float32 or t.shape != parts[0].shape or t.device != parts[0].device:
            raise BrqError("parts: fp32 tensors of one shape on one device")
    o = _out(out, tuple(parts[0].shape), torch.float32, "out") if out is not None else \
        torch.empty_like(parts[0])
    ptrs = (C.c_void_p * P)(*[t.data_ptr() for t in parts])
    _check(lib().brq_dp_reduce(ptrs, replicas, shards, accum, parts[0].numel(), int(bool(average)),
                               _ptr(o), _ptr(flags), _stream()), "dp_reduce")
    return o


def fp32_primitive(prim: int, first: int, count: int, out=None, device="cuda"):
    """The device's binary32 primitive ``prim`` (PRIM_*) on the bit patterns
    first, first + 1, ... (mod 2^32): returns a device uint32 tensor of the
    result bits (brq_fp32_primitive)."""
    o = _out(out, (count,), torch.int32, "out") if out is not None else \
        torch.empty(count, dtype=torch.int32, device=device)
    _check(lib().brq_fp32_primitive(prim, first & 0xFFFFFFFF, count, _ptr(o), _stream()),
           "fp32_primitive")
    return o
