"""One decoder layer's data-parallel hot path as a fixed sequence of libbrq
calls on preallocated device buffers (composition and marshalling only:
every step runs in libbrq's HIP kernels).

The layer is the Open-1B block shape (report §3.1 "Architecture", Table 3:
d_model 2048, GQA 16 query / 4 KV heads of 128, SwiGLU): seven W8A8 linears
(§3.2 "int8 computation") and the two pre-norm RMSNorms, over one rank's
micro-batch of tokens.  One call of :meth:`LayerStep.run` enqueues, on
torch's current stream:

  1. RMSNorm forward of each norm input                       (rmsnorm_fixed)
  2. per-tensor LSQ codes of each distinct linear input, and
     the Walsh-Hadamard rotation + requantisation of those
     codes along tokens for the weight-gradient GEMM            (quantize_x_wht)
  3. per-output-channel LSQ codes of every weight, plus the
     transposed copies for the input-gradient GEMM, in one
     call, then each forward GEMM + dequantisation             (quantize_lsq_rows_multi,
                                                                qgemm_fwd)
  4. both backward codes of each dY in two passes over it: dY
     scaled by the weight step sizes and quantised, and dY
     rotated along tokens and quantised                       (quantize_dy_bwd)
     then the input-gradient GEMM                              (qgemm_bwd_dx)
  5. the weight-gradient GEMM of each linear into the
     gradient arena                                            (qgemm_dw: the
                                                                stages of
                                                                qgemm_bwd_dw_wht)
  6. RMSNorm backward of each norm into the arena              (rmsnorm_fixed)
  7. global l2 norm over the gradient arena                     (grad_norm)
  8. SHA-256 state hash of every output and gradient          (hash_state)

The hash runs last, in one batched call on the same stream, or (with
overlap_hash) with only its leaf level there and the levels above it on a
second stream, where they overlap the next step: those levels are a few
long SHA chains on a few hundred lanes, about 0.6 ms of latency with the
GPU otherwise idle.  (Hashing each tensor's leaves on a second stream as
soon as it is written measured slower on MI355X: the integer-ALU hash and
the GEMMs then share CUs and both slow down.)

The rotated code of an activation depends on that activation alone, so
linears that share an input (Q/K/V, gate/up) share one rotation, made with
the activation's own codes (one read of the activation gives the codes and
the rotation's statistic); the results are the same bits as the one-call
qgemm_bwd_dw_wht per linear.

Gradient arena: one fp32 buffer holding, in order, dW of every linear
([N][K] row-major each) and then dg of every norm; grad_norm reduces it as
one vector in that order.

State hash tensors, in order: for each linear "<name>.y", "<name>.dx",
"<name>.dw"; for each norm "<name>.y", "<name>.dx", "<name>.dg"; then
"grad_norm" = [sum of squares, norm] (fp32).
"""
from __future__ import annotations

import torch

from . import (ADAMW_WD, SPIKE_THRESHOLD, BrqError, OP_DW_WHT, OP_DY_BWD, OP_GRAD_NORM, OP_QGEMM,
               OP_QUANTIZE, OP_QUANTIZE_X_WHT,
               OP_RMSNORM_BWD, adamw_bias_corrections, adamw_decide, adamw_step, grad_norm,
               hash_combine, hash_digests_workspace_size, hash_state, hash_state_workspace_size,
               hash_tensor_finish, hash_tensor_leaves, qgemm_bwd_dx, qgemm_dw, qgemm_fwd,
               quantize_dy_bwd, quantize_lsq_rows_multi, quantize_x_wht, rmsnorm_fixed_bwd,
               rmsnorm_fixed_fwd, workspace_size)


class _NoTimer:
    def begin(self, kind):
        pass

    def end(self, kind):
        pass


class LayerStep:
    """Buffers and call sequence of one layer step.

    linears: list of (name, in_features K, out_features N, input name)
    x:       dict input name -> bf16/fp32 device tensor [M][K]
    w:       list of device tensors [N][K] (nn.Linear layout), one per linear
    dy:      list of device tensors [M][N], one per linear
    norms:   list of (name, h [M][D], g [D], dy [M][D]) device tensors
    """

    def __init__(self, linears, x, w, dy, norms=(), block=128, eps=1e-6, tune=None):
        self.linears = list(linears)
        self.x, self.w, self.dy = x, list(w), list(dy)
        self.norms = list(norms)
        self.block, self.eps, self.tune = block, eps, tune
        first = next(iter(x.values()))
        dev = first.device
        self.device = dev
        M = first.shape[0]
        self.M = M
        if len(self.w) != len(self.linears) or len(self.dy) != len(self.linears):
            raise BrqError("one weight and one dY per linear")
        for i, (name, K, N, xin) in enumerate(self.linears):
            if tuple(x[xin].shape) != (M, K):
                raise BrqError(f"{name}: input {xin} is not [{M}, {K}]")
            if tuple(self.w[i].shape) != (N, K) or tuple(self.dy[i].shape) != (M, N):
                raise BrqError(f"{name}: weight or dY shape")
        i8, f32 = torch.int8, torch.float32
        e = lambda *s, dt=f32: torch.empty(s, dtype=dt, device=dev)  # noqa: E731
        self.flags = torch.zeros(1, dtype=torch.int32, device=dev)
        # activation codes and rotated codes, one per distinct input
        self.q_x, self.s_x, self.amax_x, self.q_ut, self.s_u = {}, {}, {}, {}, {}
        for xin, t in x.items():
            K = t.shape[1]
            self.q_x[xin], self.s_x[xin], self.amax_x[xin] = e(M, K, dt=i8), e(1), e(1)
            self.q_ut[xin], self.s_u[xin] = e(K, M, dt=i8), e(1)
        # per linear
        self.q_w, self.q_wt, self.s_w, self.amax_w = [], [], [], []
        self.y, self.q_g, self.s_g, self.amax_g, self.dx = [], [], [], [], []
        self.q_vt, self.s_v = [], []
        sizes = [N * K for _, K, N, _ in self.linears] + [h.shape[1] for _, h, _, _ in self.norms]
        self.arena = e(sum(sizes))
        off = 0
        self.dw = []
        for (name, K, N, _xin) in self.linears:
            self.q_w.append(e(N, K, dt=i8)); self.q_wt.append(e(K, N, dt=i8))
            self.s_w.append(e(N)); self.amax_w.append(e(N))
            self.y.append(e(M, N))
            self.q_g.append(e(M, N, dt=i8)); self.s_g.append(e(1)); self.amax_g.append(e(1))
            self.dx.append(e(M, K))
            self.q_vt.append(e(N, M, dt=i8)); self.s_v.append(e(1))
            self.dw.append(self.arena[off:off + N * K].view(N, K))
            off += N * K
        self.w_outs = list(zip(self.q_w, self.q_wt, self.s_w, self.amax_w))
        self.ny, self.nrstd, self.ndx, self.ndg = [], [], [], []
        for (_name, h, g, ndy) in self.norms:
            T, D = h.shape
            if T != M or tuple(g.shape) != (D,) or tuple(ndy.shape) != (T, D):
                raise BrqError("norm shapes")
            self.ny.append(torch.empty_like(h)); self.nrstd.append(e(T))
            self.ndx.append(torch.empty_like(h))
            self.ndg.append(self.arena[off:off + D])
            off += D
        self.gn = e(2)
        self.digest = torch.empty(32, dtype=torch.uint8, device=dev)
        # the overlapped hash's own workspace, tensor digests and stream (see run)
        hl = self.hash_list()
        self.hws = torch.zeros(hash_digests_workspace_size(hl), dtype=torch.uint8, device=dev)
        self.tdig = torch.empty(32 * len(hl), dtype=torch.uint8, device=dev)
        self._side = None
        self._finish_done = None
        # one workspace, large enough for every call (calls are stream-ordered)
        need = [workspace_size(OP_GRAD_NORM, self.arena.numel(), tune=tune)]
        for xin, t in x.items():
            need.append(workspace_size(OP_QUANTIZE_X_WHT, M, t.shape[1], 0, block, tune=tune))
        for (name, K, N, _xin) in self.linears:
            need += [workspace_size(OP_QUANTIZE, M, N, tune=tune),
                     workspace_size(OP_QGEMM, M, N, K, tune=tune),
                     workspace_size(OP_QGEMM, M, K, N, tune=tune),
                     workspace_size(OP_QGEMM, N, K, M, tune=tune),
                     workspace_size(OP_DY_BWD, M, N, 0, block, tune=tune)]
        for (_n, h, _g, _d) in self.norms:
            need.append(workspace_size(OP_RMSNORM_BWD, *h.shape, tune=tune))
        need.append(hash_state_workspace_size(self.hash_list()))
        self.ws = torch.zeros(max(need), dtype=torch.uint8, device=dev)

    # -- the state-hash contents, in order ------------------------------------
    def hash_list(self):
        out = []
        for i, (name, _K, _N, _x) in enumerate(self.linears):
            out += [(f"{name}.y", self.y[i]), (f"{name}.dx", self.dx[i]), (f"{name}.dw", self.dw[i])]
        for j, (name, _h, _g, _d) in enumerate(self.norms):
            out += [(f"{name}.y", self.ny[j]), (f"{name}.dx", self.ndx[j]),
                    (f"{name}.dg", self.ndg[j])]
        out.append(("grad_norm", self.gn))
        return out

    # -- one step --------------------------------------------------------------
    def run(self, timer=None, hash_outputs=True, overlap_hash=False, digest_out=None):
        """One layer step.  With overlap_hash the state hash's leaf level
        (the only part that reads the outputs) runs on the current stream
        and the levels above it, the tensor digests and the state digest on
        a second stream, overlapping the next step's work; call finish()
        before reading the digest.  digest_out receives the state digest
        (default self.digest)."""
        T = timer or _NoTimer()
        tune, ws, fl, b = self.tune, self.ws, self.flags, self.block
        for j, (_name, h, g, _d) in enumerate(self.norms):
            T.begin("rmsnorm_fwd")
            rmsnorm_fixed_fwd(h, g, self.eps, flags=fl, tune=tune, out=(self.ny[j], self.nrstd[j]))
            T.end("rmsnorm_fwd")
        for xin, t in self.x.items():
            # the activation codes and the rotation of those codes (for dW)
            T.begin("quant_x_wht")
            quantize_x_wht(t, b, tune=tune, ws=ws, flags=fl,
                           out=(self.q_x[xin], self.s_x[xin], self.amax_x[xin], self.q_ut[xin],
                                self.s_u[xin]))
            T.end("quant_x_wht")
        # every linear's per-channel weight steps and codes: one grouped call
        T.begin("quant_w")
        quantize_lsq_rows_multi(self.w, flags=fl, outs=self.w_outs)
        T.end("quant_w")
        for i, (_name, _K, _N, xin) in enumerate(self.linears):
            T.begin("gemm_fwd")
            qgemm_fwd(self.q_x[xin], self.s_x[xin], self.q_w[i], self.s_w[i], tune=tune,
                      out=self.y[i], ws=ws)
            T.end("gemm_fwd")
        for i in range(len(self.linears)):
            T.begin("quant_dy")
            quantize_dy_bwd(self.dy[i], self.s_w[i], b, tune=tune, ws=ws, flags=fl,
                            out=(self.q_g[i], self.s_g[i], self.amax_g[i], self.q_vt[i],
                                 self.s_v[i]))
            T.end("quant_dy")
            T.begin("gemm_dx")
            qgemm_bwd_dx(self.q_g[i], self.s_g[i], self.q_wt[i], tune=tune, out=self.dx[i], ws=ws)
            T.end("gemm_dx")
        for i, (_name, _K, _N, xin) in enumerate(self.linears):
            T.begin("gemm_dw")
            qgemm_dw(self.q_vt[i], self.q_ut[xin], self.s_x[xin], self.s_u[xin], self.s_v[i], b,
                     tune=tune, out=self.dw[i], ws=ws)
            T.end("gemm_dw")
        for j, (_name, h, g, ndy) in enumerate(self.norms):
            T.begin("rmsnorm_bwd")
            rmsnorm_fixed_bwd(h, g, self.nrstd[j], ndy, tune=tune, ws=ws,
                              out=(self.ndx[j], self.ndg[j]))
            T.end("rmsnorm_bwd")
        T.begin("grad_norm")
        grad_norm(self.arena, flags=fl, tune=tune, ws=ws, out=self.gn)
        T.end("grad_norm")
        if hash_outputs:
            dout = self.digest if digest_out is None else digest_out
            T.begin("hash_state")
            if overlap_hash:
                hl = self.hash_list()
                cur = torch.cuda.current_stream()
                if self._finish_done is not None:
                    # the previous step's upper levels still read self.hws
                    cur.wait_event(self._finish_done)
                hash_tensor_leaves(hl, self.hws)
                leaves_done = torch.cuda.Event()
                leaves_done.record(cur)
                if self._side is None:
                    self._side = torch.cuda.Stream(device=self.device)
                self._side.wait_event(leaves_done)
                with torch.cuda.stream(self._side):
                    hash_tensor_finish(hl, self.tdig, self.hws)
                    hash_combine(self.tdig, out=dout)
                    self._finish_done = torch.cuda.Event()
                    self._finish_done.record(self._side)
                # memory the second stream uses is not handed out again by
                # the caching allocator before that stream's work is done
                for t in (self.hws, self.tdig, dout):
                    t.record_stream(self._side)
            else:
                self.finish()
                hash_state(self.hash_list(), ws=ws, out=dout)
            T.end("hash_state")

    def finish(self):
        """Make the current stream wait for the last overlapped hash."""
        if self._finish_done is not None:
            torch.cuda.current_stream().wait_event(self._finish_done)


class OptimizerStep:
    """The optimizer step after a LayerStep (report §3.2 "Optimizer",
    "Optimizer-state precision"; §3.4.2 spike protocol): AdamW on the
    layer's parameters, clipped by the step's global grad-norm, skipped for
    five steps after a spike.

    Parameters live in one bf16 arena laid out like the gradient arena
    (every weight [N][K] in linear order, then every norm gain); the layer's
    weight and gain tensors are rebound to views of it, so the next layer
    step sees the update.  Moments m, v are fp32 arenas of the same layout.
    Per step: the decision on the device from the step's norm, then one
    update of the linear weights (weight decay 0.1) and one of the norm
    gains (no decay).  Nothing leaves the device.
    """

    def __init__(self, step, lr=3e-4, weight_decay=ADAMW_WD, spike_threshold=SPIKE_THRESHOLD):
        self.step, self.lr, self.wd = step, lr, weight_decay
        self.spike_threshold = spike_threshold
        dev = step.device
        n = step.arena.numel()
        self.param = torch.empty(n, dtype=torch.bfloat16, device=dev)
        off = 0
        for i, w in enumerate(step.w):
            if w.dtype != torch.bfloat16:
                raise BrqError("OptimizerStep keeps bf16 parameters")
            k = w.numel()
            self.param[off:off + k].copy_(w.reshape(-1))
            step.w[i] = self.param[off:off + k].view(w.shape)
            off += k
        self.n_linear = off
        for j, (name, h, g, ndy) in enumerate(step.norms):
            k = g.numel()
            self.param[off:off + k].copy_(g.reshape(-1))
            step.norms[j] = (name, h, self.param[off:off + k].view(g.shape), ndy)
            off += k
        self.m = torch.zeros(n, dtype=torch.float32, device=dev)
        self.v = torch.zeros(n, dtype=torch.float32, device=dev)
        self.skip = torch.zeros(1, dtype=torch.int32, device=dev)
        self.ctl = torch.empty(2, dtype=torch.float32, device=dev)
        self.t = 0

    def hash_list(self):
        return [("param", self.param), ("adam.m", self.m), ("adam.v", self.v)]

    def run(self, timer=None):
        T = timer or _NoTimer()
        st, nl = self.step, self.n_linear
        self.t += 1
        bc = adamw_bias_corrections(self.t)
        T.begin("optimizer")
        adamw_decide(st.gn[1:2], self.skip, out=self.ctl, spike_threshold=self.spike_threshold,
                     flags=st.flags)
        adamw_step(self.param[:nl], st.arena[:nl], self.m[:nl], self.v[:nl], self.ctl, self.lr, bc,
                   weight_decay=self.wd)
        if self.param.numel() > nl:
            adamw_step(self.param[nl:], st.arena[nl:], self.m[nl:], self.v[nl:], self.ctl, self.lr,
                       bc, weight_decay=0.0)
        T.end("optimizer")
