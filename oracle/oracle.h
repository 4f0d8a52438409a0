/*
 * oracle.h -- plain, sequential CPU oracle for the bitwise-reproducible W8A8
 * QAT linear layer (TEST INFRASTRUCTURE ONLY).
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The product path (libbrq, HIP) shares no code,
 * header, table or constant with it.
 *
 * Every routine is the definition written out, in the order the pages give
 * it (Open-1B: A Fully Auditable Training Run, arXiv 2609.17380):
 *   - §2.1 "Reproducible Operations" and Table 1: one fixed reduction order,
 *     no fused multiply-add, subnormals flushed to zero on input and output.
 *   - §3.1 "int8 quantization-aware training" and §4.2 "Implementation
 *     notes": per-channel weight step size 2*mean(|w|)/sqrt(q_max),
 *     recomputed every step.
 *   - §3.2 "int8 computation": W8A8 with per-channel weight and per-tensor
 *     activation scales, int32 accumulation then dequantisation, both STE
 *     gradient GEMMs in int8, Walsh-Hadamard rotation along the contraction
 *     dimension before the weight-gradient quantisation.
 *   - §3.1 "RMSNorm", "Weights are initialized..." paragraph: normalisation
 *     in FP32, parameters BF16, FP32 gradient reduction.
 *   - §3.2 "Optimizer": global l2 gradient norm; AdamW, clipping;
 *     "Optimizer-state precision": BF16 parameters, FP32 moments.
 *   - §3.4.2: the spike protocol (five skipped optimizer steps).
 *   - App. A.3: every average is a multiply by a precomputed reciprocal.
 *   - App. A.1, A.2: the replicas' TreeFold and the shards' ascending-rank
 *     running sum of the deterministic gradient exchange.
 *   - §5 "Runtime overhead" / App. B: a canonical state hash per step.
 *
 * Arithmetic model: each floating-point operation is one IEEE-754 binary32
 * operation in round-to-nearest-even (gcc, -ffp-contract=off, SSE2, default
 * MXCSR).  A value loaded from memory whose exponent field is zero becomes
 * a zero of the same sign (DAZ); a result that is subnormal becomes a zero
 * of the same sign (FTZ).  Both flushes are explicit in the code.
 *
 * Parity pins (all in tests/, none re-types a formula of this file):
 *   tree sum ........ hand-computed order-sensitive vectors, closed forms on
 *                     powers of two, a second independent (recursive) coding
 *   quantiser ....... quantise(dequant(q)) == q, RNE ties, clamps, fp64
 *                     single-rounding evaluation
 *   int8 GEMMs ...... brute-force int64 dot products (numpy), fp64 dots
 *   int WHT ......... H*H^T = b*I, H(Hv) = b*v, butterfly vs definition
 *   fp WHT .......... integer-valued inputs equal the integer transform
 *   dW .............. (H qx)^T (H qv) = b * qx^T qv exactly
 *   RMSNorm ......... +-1 rows give closed-form rstd; fp64 bounds
 *   grad-norm ....... 2^k leaves of 2^-j give exact closed forms
 *   SHA-256 ......... Python hashlib (FIPS 180-4), independent Python Merkle
 *   AdamW ........... fp64 evaluation within rounding bounds, zero-gradient
 *                     and first-step closed forms, the skip-window sequence
 *   exchange ........ hand-derived order-sensitive vectors for the ascending
 *                     sum and TreeFold, a simulated recursive-doubling
 *                     all-reduce (exact rationals), closed forms on powers
 *                     of two, reciprocal averages within one ulp of the
 *                     correctly rounded quotient
 * The butterfly stage order of the fp WHT and the RMSNorm backward operation
 * order are definitions that no external value fixes: parity unpinned beyond
 * the bounds and special cases above.
 */
#ifndef BRQ_ORACLE_H
#define BRQ_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_I8 = 2, ORC_I32 = 3, ORC_U8 = 4 };
enum { ORC_PER_TENSOR = 0, ORC_PER_ROW = 1 };
enum { ORC_FLAG_NONFINITE = 1 };

/* OpenMP threads available to the loops over independent outputs. */
int orc_num_threads(void);
/* Sets that thread count (n >= 1); every value is computed by the same
   sequential code whatever the count, so results do not depend on it. */
void orc_set_num_threads(int n);

/* ---- arithmetic model helpers, exported so the pins can probe them ---- */
float orc_flush(float v);                 /* subnormal -> signed zero */
float orc_bf16_to_f32(uint16_t h);        /* exact widen, then DAZ */
uint16_t orc_f32_to_bf16(float f);        /* RNE on the bit pattern */
float orc_lsq_k2(void);                   /* 2 * fl(1/fl(sqrt(127))) */
void orc_f32_to_bf16_array(const float* in, int64_t n, uint16_t* out);

/* Primitives over the bit patterns first, first + 1, ... (count of them):
 * prim 0 fl(sqrt(daz(x))), 1 fl(1/daz(x)), 2 fl(1/fl(sqrt(daz(x)))), 3 and 4
 * the bf16 rounding of x (nearest even) in the low 16 bits. */
void orc_prim_sweep(int prim, uint32_t first, int64_t count, uint32_t* out);

/* Canonical pairwise tree over leaves[0..n): node(j+1,i) = node(j,2i) +
 * node(j,2i+1) when the right child exists, else node(j,2i).  Two codings. */
float orc_tree_sum(const float* leaves, int64_t n);
float orc_tree_sum_recursive(const float* leaves, int64_t n);

/* LSQ scale from the tree sum S of |x| over n leaves: s = (S*(1/n))*K2,
 * r = 1/s (0 when s == 0). */
void orc_lsq_scale(float S, int64_t n, float* s, float* r);
/* q = clamp(rint(x*r), -127, 127) */
int8_t orc_quant1(float x, float r);

/* quantize_lsq: x [rows][cols] (F32 or BF16), optional col_mul[cols]
 * multiplied into every element first.  PER_TENSOR writes scale[0],
 * amax[0]; PER_ROW writes scale[rows], amax[rows].  q [rows][cols];
 * q_t [cols][rows] when non-NULL.  Returns flags. */
int orc_quantize_lsq(const void* x, int dtype, int64_t rows, int64_t cols,
                     int gran, const float* col_mul, int8_t* q, int8_t* q_t,
                     float* scale, float* amax);

/* The same with the statistic S the exact sum of |v| rounded once to
 * binary32 (nearest even, subnormal results flushed) in place of the tree. */
int orc_quantize_lsq_exact(const void* x, int dtype, int64_t rows, int64_t cols,
                           int gran, const float* col_mul, int8_t* q, int8_t* q_t,
                           float* scale, float* amax);
/* Exact sum of |v[i]| (each v[i] flushed first) rounded once to binary32;
 * NaN if any v[i] is NaN, else +inf if any is infinite or the sum is out of
 * range. */
float orc_exact_abs_sum(const float* v, int64_t n);

/* qgemm_fwd: y[m][n] = fl(fl(sum_k qx[m][k]*qw[n][k]) * fl(s_x*s_w[n]))
 * (s_w[0] for every n when w_per_row == 0). */
void orc_qgemm_fwd(const int8_t* qx, const float* s_x, const int8_t* qw,
                   const float* s_w, int w_per_row, int64_t M, int64_t N,
                   int64_t K, float* y);

/* qgemm_bwd_dx: dx[m][k] = fl(fl(sum_n qg[m][n]*qw[n][k]) * s_g);
 * qw is the [N][K] weight code (the definition), not a transposed copy. */
void orc_qgemm_bwd_dx(const int8_t* qg, const float* s_g, const int8_t* qw,
                      int64_t M, int64_t N, int64_t K, float* dx);

/* Integer Walsh-Hadamard transform of qx [M][K] along tokens: u [M][K]. */
void orc_wht_int(const int8_t* qx, int64_t M, int64_t K, int b, int32_t* u);

/* Integer Walsh-Hadamard of qx [M][K] along tokens in aligned blocks of b
 * (Sylvester, natural order, unnormalised), exact; S_u = sum |u| (int64);
 * s_u, r_u from S_u; q_u [M][K]. */
void orc_wht_int_quant(const int8_t* qx, int64_t M, int64_t K, int b,
                       int8_t* q_u, float* s_u, int64_t* S_u_out);

/* fp32 Walsh-Hadamard of dy [M][N] (F32 or BF16) along tokens in aligned
 * blocks of b: butterflies in stage order h = 1, 2, ..., b/2, then
 * per-tensor LSQ over the rotated values in row-major order.  v_out
 * (optional, [M][N]) receives the rotated values.  Returns flags. */
int orc_wht_fp_quant(const void* dy, int dtype, int64_t M, int64_t N, int b,
                     int8_t* q_v, float* s_v, float* v_out);

/* dW rows [n_lo, n_hi): dw[n][k] = fl(fl(sum_m qv[m][n]*qu[m][k]) * c_w),
 * c_w = fl(fl(fl(s_x*s_u)*s_v) * 2^-log2(b)).  dw is the full [N][K]. */
void orc_dw_gemm(const int8_t* q_v, const int8_t* q_u, int64_t M, int64_t N,
                 int64_t K, float s_x, float s_u, float s_v, int b,
                 int64_t n_lo, int64_t n_hi, float* dw);

/* The whole qgemm_bwd_dw_wht step: rotate+quantise qx and dy, dW GEMM. */
int orc_qgemm_bwd_dw_wht(const int8_t* qx, const float* s_x, const void* dy,
                         int dtype, int64_t M, int64_t N, int64_t K, int b,
                         float* dw, float* s_u_out, float* s_v_out);

/* Attention forward with an int8 P.V product (variant), definitions in
 * oracle.c: q [Hq][T][d], k, v [Hkv][T][d] bf16 patterns, o [Hq][T][d]
 * fp32; T % 64 == 0, Hq % Hkv == 0; window >= T is plain causal.
 * Returns flags (or -1 for a shape it does not take). */
float orc_exp_f(float x);
int orc_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t Hq,
                 int64_t Hkv, int64_t T, int64_t d, int64_t window, float* o);

/* Rotated input-gradient GEMM (variant): g = fl(dy * s_w[n]) rotated in
 * fp32 along n per row and aligned block of b, per-tensor LSQ -> q_g, s_g;
 * q_w [N][K] rotated exactly along n and requantised -> q_h, s_h;
 * dx[m][k] = fl(fl(sum_n q_g[m][n] q_h[n][k]) * fl(fl(s_g*s_h) * 1/b)).
 * s_w may be NULL (no multiplier) for the rotation alone. */
int orc_wht_fp_rows_quant(const void* dy, int dtype, int64_t M, int64_t N,
                          const float* s_w, int b, int8_t* q, float* s_out,
                          float* v_out);
int orc_qgemm_bwd_dx_wht(const void* dy, int dtype, const float* s_w,
                         const int8_t* qw, int64_t M, int64_t N, int64_t K, int b,
                         float* dx, float* s_g_out, float* s_h_out);

/* RMSNorm forward per row: ss = tree(x*x), ms = ss*(1/D),
 * rstd = 1/sqrt(ms+eps), y = (x*rstd)*g.  x, g, y in `dtype`. */
int orc_rmsnorm_fwd(const void* x, const void* g, int dtype, int64_t T,
                    int64_t D, float eps, void* y, float* rstd);

/* RMSNorm backward: dx (dtype), dg [D] fp32 (tree over tokens). */
void orc_rmsnorm_bwd(const void* x, const void* g, const float* rstd,
                     const void* dy, int dtype, int64_t T, int64_t D,
                     void* dx, float* dg);

/* Global grad-norm: ss = tree(v*v), norm = sqrt(ss). */
int orc_grad_norm(const float* v, int64_t n, float* sumsq, float* norm);

/* AdamW step (decoupled weight decay), global-norm clip and spike skip.
 * bias corrections: bc = 1 - beta^t, beta^t a t-fold rounded product. */
void orc_adamw_bias_corrections(int64_t t, float beta1, float beta2, float* bc1,
                                float* bc2);
/* Step control from the pre-clip norm: apply (1 or 0) and clip scale;
 * skip_state counts the skipped steps still due. */
int orc_adamw_decide(float norm, float max_norm, float spike_threshold,
                     int skip_steps, int32_t* skip_state, float* apply,
                     float* clip);
/* One update of n elements: param (dtype pdtype) and the fp32 moments m, v
 * in place, from grad (dtype gdtype). */
void orc_adamw_step(void* param, int pdtype, const void* grad, int gdtype,
                    float* m, float* v, int64_t n, float lr, float beta1,
                    float beta2, float eps, float wd, float bc1, float bc2,
                    float apply, float clip);

/* Deterministic gradient exchange (App. A).  parts: host array of pointers
 * to [n] fp32 contributions.
 *   orc_ascending_sum: out = (((c_0 + c_1) + c_2) + ...) in index order.
 *   orc_average: out = x * fl(1/k).
 *   orc_treefold: TreeFold (binary-carry Push, Result in ascending level
 *     order, lower replica on the left) over R <= 64 replica partials.
 *   orc_dp_reduce: R*S*A contributions in mesh order (replica-major, then
 *     shard, then microbatch): per shard the microbatch running sum (times
 *     fl(1/A)), per replica the ascending shard sum (times fl(1/S)), then
 *     TreeFold over replicas (times fl(1/R)); averages only when average
 *     != 0.  R*S*A <= 64.  Returns flags (non-finite output), or -1 for a
 *     count it does not take. */
void orc_ascending_sum(const float* const* parts, int count, int64_t n, float* out);
void orc_average(const float* x, int64_t n, int64_t k, float* out);
void orc_treefold(const float* const* parts, int R, int64_t n, float* out);
int orc_dp_reduce(const float* const* parts, int R, int S, int A, int64_t n,
                  int average, float* out);

/* SHA-256 (FIPS 180-4). */
void orc_sha256(const uint8_t* msg, uint64_t len, uint8_t out[32]);

/* Merkle root of a byte buffer: 4096-byte leaves, fan-in 128. */
void orc_merkle_root(const uint8_t* bytes, uint64_t nbytes, uint8_t out[32]);

/* Tensor digest: SHA-256("BRQ1" | dtype u8 | ndim u8 | dims u64le... |
 * name_len u16le | name | merkle root). */
void orc_tensor_digest(const uint8_t* bytes, uint64_t nbytes, int dtype,
                       int ndim, const int64_t* dims, const char* name,
                       uint8_t out[32]);

/* State digest: SHA-256 of the concatenated tensor digests, in call order.
 * ptrs[i] points at tensor i's bytes; dims is concatenated. */
void orc_hash_state(int n, const uint8_t* const* ptrs, const uint64_t* nbytes,
                    const int* dtypes, const int* ndims, const int64_t* dims,
                    const char* const* names, uint8_t out[32]);

#ifdef __cplusplus
}
#endif
#endif
