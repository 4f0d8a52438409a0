"""Write tests/golden/config_digests.txt: the SHA-256 of every output of the
five workloads, as the plain CPU oracle computes them on the seeded inputs.

Only oracle/ (the arithmetic) and brq_synth (the inputs) are called; no value
comes from the HIP library.  Each line is

    <workload> <tensor> <sha256 of the raw little-endian bytes> <dtype> <shape>

and "<workload> state <digest>" is the on-device state hash's definition
(SHA-256 Merkle tensor digests, then SHA-256 over them in order) evaluated
by the oracle.  Tensors are digested in the layouts the C ABI writes
(rotated codes token-contiguous: q_ut [K][M], q_vt [N][M]).

Usage:  python tests/golden/make_digests.py [tiny qkv mlp norm layer]
Runs with the oracle's OpenMP threads (independent outputs only; every value
is produced by the same sequential code whatever the thread count).
"""
import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import brq_synth as syn  # noqa: E402
import oracle as orc  # noqa: E402

OUT = os.path.join(HERE, "config_digests.txt")
ORDER = ["tiny", "qkv", "mlp", "norm", "layer"]


class Sink:
    """Collects raw-byte digests, and the tensor digests of the state hash."""

    def __init__(self, cfg):
        self.cfg, self.lines, self.state = cfg, [], []

    def put(self, name, a, state=False):
        a = np.ascontiguousarray(a)
        h = hashlib.sha256(a.tobytes()).hexdigest()
        shape = "x".join(str(d) for d in a.shape) or "scalar"
        self.lines.append(f"{self.cfg} {name} {h} {a.dtype.name} {shape}")
        if state:
            self.state.append(orc.tensor_digest(name, a))

    def close(self):
        if self.state:
            d = orc.sha256(b"".join(self.state)).hex()
            self.lines.append(f"{self.cfg} state {d} u8 32")
        return self.lines


def f32(v):
    return np.array([v], np.float32) if np.ndim(v) == 0 else np.asarray(v, np.float32)


def linear_fwd_bwd(sink, x, w, dy, b, prefix="", state=True):
    """One W8A8 QAT linear, forward and backward (the hot-path rows in order)."""
    qx, _, sx, ax, _ = orc.quantize_lsq(x)
    sink.put(prefix + "q_x", qx); sink.put(prefix + "s_x", sx); sink.put(prefix + "amax_x", ax)
    qw, qwt, sw, aw, _ = orc.quantize_lsq(w, per_row=True, want_t=True)
    sink.put(prefix + "q_w", qw); sink.put(prefix + "q_wt", qwt)
    sink.put(prefix + "s_w", sw); sink.put(prefix + "amax_w", aw)
    y = orc.qgemm_fwd(qx, sx, qw, sw)
    sink.put(prefix + "y", y, state)
    del y
    qg, _, sg, ag, _ = orc.quantize_lsq(dy, col_mul=sw)
    sink.put(prefix + "q_g", qg); sink.put(prefix + "s_g", sg); sink.put(prefix + "amax_g", ag)
    dx = orc.qgemm_bwd_dx(qg, sg, qw)
    del qg
    sink.put(prefix + "dx", dx, state)
    del dx
    qu, su, _ = orc.wht_int_quant(qx, b)
    sink.put(prefix + "q_ut", qu.T); sink.put(prefix + "s_u", f32(su))
    qv, sv, _, _ = orc.wht_fp_quant(dy, b)
    sink.put(prefix + "q_vt", qv.T); sink.put(prefix + "s_v", f32(sv))
    dw = orc.dw_gemm(qv, qu, sx[0], su, sv, b)
    sink.put(prefix + "dw", dw, state)


def cfg_tiny():
    s = Sink("tiny")
    d = syn.tiny()
    linear_fwd_bwd(s, d["x"], d["w"], d["dy"], d["block"])
    return s.close()


def cfg_mlp():
    s = Sink("mlp")
    d = syn.mlp()
    linear_fwd_bwd(s, d["x"], d["w"], d["dy"], d["block"])
    return s.close()


def cfg_qkv():
    s = Sink("qkv")
    d = syn.qkv()
    qx, _, sx, ax, _ = orc.quantize_lsq(d["x"])
    s.put("q_x", qx); s.put("s_x", sx); s.put("amax_x", ax)
    qw, _, sw, aw, _ = orc.quantize_lsq(d["w"], per_row=True)
    s.put("q_w", qw); s.put("s_w", sw); s.put("amax_w", aw)
    s.put("y", orc.qgemm_fwd(qx, sx, qw, sw), True)
    # the degenerate per-tensor weight scale
    qp, _, sp, ap, _ = orc.quantize_lsq(d["w"])
    s.put("q_w_pt", qp); s.put("s_w_pt", sp); s.put("amax_w_pt", ap)
    s.put("y_pt", orc.qgemm_fwd(qx, sx, qp, sp), True)
    return s.close()


def cfg_norm():
    s = Sink("norm")
    d = syn.norm()
    y, rstd, _ = orc.rmsnorm_fwd(d["x"], d["g"], 1e-6)
    s.put("y", y, True); s.put("rstd", rstd, True)
    dx, dg = orc.rmsnorm_bwd(d["x"], d["g"], rstd, d["dy"])
    s.put("dx", dx, True); s.put("dg", dg, True)
    del y, dx, d["x"], d["dy"]
    ss, nrm, _ = orc.grad_norm(d["v"])
    s.put("grad_norm", np.array([ss, nrm], np.float32), True)
    return s.close()


def cfg_layer(M=32768, b=128):
    """One decoder layer: the two RMSNorms, seven linears fwd+bwd, the
    grad-norm over the gradient arena (every dW, then every dg), and the
    state hash over every output and gradient."""
    s = Sink("layer")
    xs = {name: syn.layer_input(name, M) for name, _ in syn.LAYER_INPUTS}
    codes = {}
    for name, x in xs.items():
        qx, _, sx, ax, _ = orc.quantize_lsq(x)
        qu, su, _ = orc.wht_int_quant(qx, b)
        codes[name] = (qx, sx, qu, su)
        s.put(f"{name}.q_x", qx); s.put(f"{name}.s_x", sx); s.put(f"{name}.amax_x", ax)
        s.put(f"{name}.q_ut", qu.T); s.put(f"{name}.s_u", f32(su))
    del xs
    state = []  # tensor digests in hash order
    arena = []
    for i, (lname, K, N, xin) in enumerate(syn.LAYER_LINEARS):
        t0 = time.time()
        qx, sx, qu, su = codes[xin]
        w = syn.layer_weight(i)
        dy = syn.layer_dy(i, M)
        qw, qwt, sw, aw, _ = orc.quantize_lsq(w, per_row=True, want_t=True)
        s.put(f"{lname}.q_w", qw); s.put(f"{lname}.q_wt", qwt); s.put(f"{lname}.s_w", sw)
        y = orc.qgemm_fwd(qx, sx, qw, sw)
        s.put(f"{lname}.y", y); state.append(orc.tensor_digest(f"{lname}.y", y))
        del y
        qg, _, sg, _, _ = orc.quantize_lsq(dy, col_mul=sw)
        s.put(f"{lname}.q_g", qg); s.put(f"{lname}.s_g", sg)
        dx = orc.qgemm_bwd_dx(qg, sg, qw)
        del qg
        s.put(f"{lname}.dx", dx); state.append(orc.tensor_digest(f"{lname}.dx", dx))
        del dx
        qv, sv, _, _ = orc.wht_fp_quant(dy, b)
        del dy
        s.put(f"{lname}.q_vt", qv.T); s.put(f"{lname}.s_v", f32(sv))
        dw = orc.dw_gemm(qv, qu, sx[0], su, sv, b)
        del qv
        s.put(f"{lname}.dw", dw); state.append(orc.tensor_digest(f"{lname}.dw", dw))
        arena.append(dw.reshape(-1))
        print(f"  layer {lname}: {time.time() - t0:.1f} s", flush=True)
    for j, (nname, D) in enumerate(syn.LAYER_NORMS):
        h, g, ndy = syn.layer_norm_inputs(j, M)
        y, rstd, _ = orc.rmsnorm_fwd(h, g, 1e-6)
        dx, dg = orc.rmsnorm_bwd(h, g, rstd, ndy)
        s.put(f"{nname}.y", y); s.put(f"{nname}.rstd", rstd)
        s.put(f"{nname}.dx", dx); s.put(f"{nname}.dg", dg)
        state += [orc.tensor_digest(f"{nname}.y", y), orc.tensor_digest(f"{nname}.dx", dx),
                  orc.tensor_digest(f"{nname}.dg", dg)]
        arena.append(dg)
    ss, nrm, _ = orc.grad_norm(np.concatenate(arena))
    gn = np.array([ss, nrm], np.float32)
    s.put("grad_norm", gn)
    state.append(orc.tensor_digest("grad_norm", gn))
    s.lines.append(f"layer state {orc.sha256(b''.join(state)).hex()} u8 32")
    return s.lines


FUNCS = {"tiny": cfg_tiny, "qkv": cfg_qkv, "mlp": cfg_mlp, "norm": cfg_norm, "layer": cfg_layer}


def main(which):
    old = {}
    if os.path.exists(OUT):
        for line in open(OUT):
            if line.strip() and not line.startswith("#"):
                old.setdefault(line.split()[0], []).append(line.rstrip("\n"))
    for cfg in which:
        t0 = time.time()
        print(f"{cfg}: oracle running", flush=True)
        old[cfg] = FUNCS[cfg]()
        print(f"{cfg}: {len(old[cfg])} digests in {time.time() - t0:.1f} s", flush=True)
        with open(OUT + ".tmp", "w") as f:
            f.write("# SHA-256 of every output of each workload, computed by the CPU oracle\n"
                    "# (oracle/) on brq_synth's seeded inputs; written by make_digests.py.\n")
            for c in ORDER:
                for line in old.get(c, []):
                    f.write(line + "\n")
        os.replace(OUT + ".tmp", OUT)


if __name__ == "__main__":
    main(sys.argv[1:] or ORDER)
