"""Planted mistakes in a copy of the oracle must fail the pins.

Each mutant edits one line of oracle.c (a dropped term, a wrong sign, a
transposed operand, a wrong rounding or constant), builds it into a
temporary library, and runs tests/test_oracle_pins.py and
tests/test_oracle_exchange_pins.py against it in a child process.  The
pins pass on the real oracle and must fail on every mutant.  All of this
runs on the CPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "tree_tail_pairs_from_right": (
        "buf[half] = buf[len - 1];", "buf[half] = fadd(buf[len - 1], -0.0f);\n      for (int64_t i = half; i > 0; i--) buf[i] = buf[i - 1]; buf[0] = buf[0];"),
    "tree_sequential": (
        "for (int64_t i = 0; i < half; i++) buf[i] = fadd(buf[2 * i], buf[2 * i + 1]);",
        "for (int64_t i = 1; i < len; i++) buf[0] = fadd(buf[0], buf[i]); len = 1; half = 0; continue;"),
    "quant_truncates": ("float t = rintf(fmul(x, r));", "float t = truncf(fmul(x, r));"),
    "quant_clamp_128": ("if (t < -127.0f) t = -127.0f;", "if (t < -128.0f) t = -128.0f;"),
    "k2_drops_factor_two": ("return fmul(2.0f, rs);", "return rs;"),
    "mean_divides": ("float m = fmul(S, inv_count(n));", "float m = fdiv(S, (float)n);"),
    "no_daz_on_load": ("return orc_flush(((const float*)p)[i]);", "return ((const float*)p)[i];"),
    "dx_transposed_weight": ("acc[k] += g * (int64_t)qw[n * K + k];", "acc[k] += g * (int64_t)qw[(k * N + n) % (N * K)];"),
    "fwd_scale_ignores_sx": ("float c = fmul(sx, orc_flush(w_per_row ? s_w[n] : s_w[0]));",
                             "float c = orc_flush(w_per_row ? s_w[n] : s_w[0]);"),
    "hadamard_or_not_and": ("__builtin_popcount((unsigned)(i & j))", "__builtin_popcount((unsigned)(i | j))"),
    "fp_wht_sign": ("*d = fsub(x0, x1);", "*d = fsub(x1, x0);"),
    "dw_missing_inv_b": ("orc_flush(s_v)), inv_b);", "orc_flush(s_v)), 1.0f);"),
    "rmsnorm_y_groups_rstd_with_g": ("store(y, dtype, t * D + j, fmul(fmul(xs[j], r), load(g, dtype, j)));",
                                     "store(y, dtype, t * D + j, fmul(xs[j], fmul(r, load(g, dtype, j))));"),
    "rmsnorm_no_eps": ("float r = fdiv(1.0f, fsqrt(fadd(ms, e)));", "float r = fdiv(1.0f, fsqrt(ms));"),
    "rmsnorm_bwd_sign": ("fmul(r, fsub(d[j], fmul(xh[j], mu)))", "fmul(r, fadd(d[j], fmul(xh[j], mu)))"),
    "gradnorm_abs_not_square": ("sq[i] = fmul(e, e);", "sq[i] = fabs_(e);"),
    "sha_wrong_rotate": ("uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);",
                         "uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 24);"),
    "merkle_fanin_64": ("const uint64_t LEAF = 4096, FAN = 128;", "const uint64_t LEAF = 4096, FAN = 64;"),
    "bf16_round_truncates": ("u += 0x7fffu + ((u >> 16) & 1u);", "u += 0;"),
    "adamw_beta2_on_m": ("const float mi = fadd(fmul(beta1, orc_flush(m[i])), fmul(omb1, g));",
                         "const float mi = fadd(fmul(beta2, orc_flush(m[i])), fmul(omb1, g));"),
    "adamw_no_bias_correction": ("const float mh = fdiv(mi, bc1);", "const float mh = mi;"),
    "adamw_eps_inside_sqrt": ("const float u = fdiv(mh, fadd(fsqrt(vh), eps));",
                              "const float u = fdiv(mh, fsqrt(fadd(vh, eps)));"),
    "adamw_decay_sign": ("const float pn = fsub(p, fmul(lr, fadd(u, fmul(wd, p))));",
                         "const float pn = fsub(p, fmul(lr, fsub(u, fmul(wd, p))));"),
    "adamw_bias_power_of_beta2": ("    p1 = fmul(p1, beta1);", "    p1 = fmul(p1, beta2);"),
    "spike_skips_four": ("if (!finite || norm > spike_threshold) *skip_state = skip_steps;",
                         "if (!finite || norm > spike_threshold) *skip_state = skip_steps - 1;"),
    "exact_truncates": ("if (half && (sticky || (q & 1u))) q++;", "if (0) q++;"),
    "exact_ties_away": ("if (half && (sticky || (q & 1u))) q++;", "if (half) q++;"),
    "exact_no_sticky": ("for (int i = lo - 2; i >= 0 && !sticky; i--) sticky = exact_bit(w, i);",
                        "(void)0;"),
    "exact_drops_carry": ("add = (add >> 32) + (t >> 32);", "add = (add >> 32);"),
    "exact_unit_off_by_one": ("return orc_flush((float)ldexp((double)q, lo - 149));",
                              "return orc_flush((float)ldexp((double)q, lo - 150));"),
    "exact_inf_before_nan": ("if (any_nan) return u2f(0x7fc00000u);", "if (any_nan) return u2f(0x7f800000u);"),
    "exact_keeps_subnormals": ("uint32_t u = f2u(orc_flush(v[i])) & 0x7fffffffu;",
                               "uint32_t u = f2u(v[i]) & 0x7fffffffu; if (u && u < 0x800000u) "
                               "{ exact_add(w, u, 0); continue; }"),
    "exact_uses_tree": ("    S = orc_exact_abs_sum(v, n);", "    S = orc_tree_sum(v, n);"),
    "rows_wht_sign": ("blk[j + h] = fsub(x0, x1);", "blk[j + h] = fsub(x1, x0);"),
    "rows_wht_no_multiplier": ("if (s_w) e = fmul(e, orc_flush(s_w[i % N]));", "(void)s_w;"),
    "rows_wht_multiplier_by_row": ("if (s_w) e = fmul(e, orc_flush(s_w[i % N]));",
                                   "if (s_w) e = fmul(e, orc_flush(s_w[(i / N) % N]));"),
    "dx_wht_missing_inv_b": ("float c = fmul(fmul(orc_flush(s_g), orc_flush(s_h)), inv_b);",
                             "float c = fmul(orc_flush(s_g), orc_flush(s_h));"),
    "dx_wht_weights_unrotated": ("orc_wht_int_quant(qw, N, K, b, q_h, &s_h, NULL);",
                                 "orc_wht_int_quant(qw, N, K, 1, q_h, &s_h, NULL);"),
    "attn_window_off_by_one": ("if (gj > gi || gj <= gi - window) { S[i][j] = -INFINITY; continue; }",
                               "if (gj > gi || gj < gi - window) { S[i][j] = -INFINITY; continue; }"),
    "attn_sees_next_key": ("if (gj > gi || gj <= gi - window) { S[i][j] = -INFINITY; continue; }",
                           "if (gj > gi + 1 || gj <= gi - window) { S[i][j] = -INFINITY; continue; }"),
    "attn_gqa_modulo": ("const int64_t hk = h / group;", "const int64_t hk = h % Hkv;"),
    "attn_l_not_rescaled": ("l[i] = fadd(fmul(l[i], alpha[i]), tree_inplace(leaves, ATT_BLK));",
                            "l[i] = fadd(l[i], tree_inplace(leaves, ATT_BLK));"),
    "attn_o_not_rescaled": ("acc[i * d + e] = fadd(fmul(acc[i * d + e], alpha[i]), contrib);",
                            "acc[i * d + e] = fadd(acc[i * d + e], contrib);"),
    "attn_no_logit_scale": ("S[i][j] = fmul(dot, c);", "S[i][j] = dot;"),
    "attn_codes_255": ("float s = fmul(amax, fdiv(1.0f, 127.0f));", "float s = fmul(amax, fdiv(1.0f, 255.0f));"),
    "exp_drops_a_term": ("for (int i = 6; i >= 0; i--) p = fadd(fmul(p, r), c[i]);",
                         "for (int i = 5; i >= 0; i--) p = fadd(fmul(p, r), c[i]);"),
    "ascending_sum_descending": (
        "  float acc = orc_flush(parts[0][i]);\n  for (int j = 1; j < count; j++) acc = fadd(acc, orc_flush(parts[j][i]));",
        "  float acc = orc_flush(parts[count - 1][i]);\n  for (int j = count - 2; j >= 0; j--) acc = fadd(acc, orc_flush(parts[j][i]));"),
    "treefold_result_largest_first": (
        "  float acc = stack[depth - 1].val;\n  for (int k = depth - 2; k >= 0; k--) acc = fadd(stack[k].val, acc);",
        "  float acc = stack[0].val;\n  for (int k = 1; k < depth; k++) acc = fadd(acc, stack[k].val);"),
    "treefold_never_merges": ("while (*depth > 0 && stack[*depth - 1].level == e.level) {",
                              "while (0) {"),
    "average_divides": ("for (int64_t i = 0; i < n; i++) out[i] = fmul(orc_flush(x[i]), inv);",
                        "for (int64_t i = 0; i < n; i++) out[i] = fdiv(orc_flush(x[i]), (float)k);"),
    "dp_shard_average_divides": ("if (average) inner = fmul(inner, inv_s);",
                                 "if (average) inner = fdiv(inner, (float)S);"),
    "dp_no_replica_average": ("if (average) res = fmul(res, inv_r);", "(void)inv_r;"),
    "dp_shard_major_mesh": ("parts + (size_t)(r * S + s) * A", "parts + (size_t)(s * R + r) * A"),
    "clip_always_scales": ("*clip = norm > max_norm ? fdiv(orc_flush(max_norm), norm) : 1.0f;",
                           "*clip = fdiv(orc_flush(max_norm), norm);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_pins(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", "-I", os.path.join(ROOT, "oracle"), str(mut), "-o", str(lib), "-lm"],
                   check=True)
    env = dict(os.environ, BRQ_ORACLE_LIB=str(lib), OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_exchange_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
