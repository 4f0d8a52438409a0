/*
 * brq.h -- C ABI of libbrq: the bitwise-reproducible W8A8 quantisation-aware
 * linear layer of the Open-1B report (arXiv 2609.17380), for AMD Instinct
 * MI355X (gfx950).
 *
 * Conventions (all entry points):
 *  - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates or frees device memory; scratch space comes from the
 *    caller's workspace `ws` of at least brq_workspace_size(...) bytes.
 *  - Row-major, contiguous.  int8 / bf16 / fp32 tensors must be 16-byte
 *    aligned; shapes satisfy the per-call rules stated below.
 *  - Every call enqueues its kernels on `stream` (a hipStream_t; NULL is the
 *    null stream) and returns once they are launched.  Nothing synchronises.
 *  - Return value: BRQ_OK (0) or a negative brq_status, detected on the host
 *    before anything is launched (argument errors) or from the launch itself
 *    (BRQ_E_HIP; brq_last_hip_error() has the code).
 *  - Data errors found on the device (a non-finite statistic) are OR-ed into
 *    `dflags` (device int32*, may be NULL) as BRQ_FLAG_*; outputs are
 *    unspecified when a flag is raised.  The caller zeroes `dflags`.
 *  - Results are bit-identical for every `tune` setting and every launch
 *    geometry; `tune` may be NULL (defaults).
 *  - Calls that share a workspace must be ordered (same stream or explicit
 *    synchronisation); calls with distinct workspaces may run concurrently.
 *
 * Numerics (the pages' bitwise-reproducibility contract, §2.1 and Table 1):
 *  every floating-point operation is one IEEE binary32 operation, round to
 *  nearest even, never contracted into a fused multiply-add; inputs whose
 *  exponent field is zero read as signed zero and subnormal results are
 *  replaced by signed zero; every reduction follows one canonical pairwise
 *  tree over the leaves in logical row-major order (pairs (2i, 2i+1), lower
 *  index on the left, an unpaired last node moves up unchanged); every mean
 *  is a multiply by fl(1/n) (App. A.3).
 */
#ifndef BRQ_H
#define BRQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BRQ_SPEC_VERSION 1

enum brq_status {
  BRQ_OK = 0,
  BRQ_E_NULL = -1,        /* a required pointer is NULL */
  BRQ_E_DTYPE = -2,       /* unsupported dtype code */
  BRQ_E_SHAPE = -3,       /* negative size or inconsistent shape */
  BRQ_E_ALIGN = -4,       /* pointer not 16-byte aligned */
  BRQ_E_UNSUPPORTED = -5, /* shape outside the supported set (see call) */
  BRQ_E_RANGE = -6,       /* contraction too long for exact int32 sums */
  BRQ_E_WORKSPACE = -7,   /* workspace missing or too small */
  BRQ_E_HIP = -8,         /* kernel launch failed */
  BRQ_E_ARG = -9,         /* other invalid argument */
  BRQ_E_SCRATCH = -10     /* input too large for the static scratch buffer */
};

enum brq_dtype { BRQ_F32 = 0, BRQ_BF16 = 1, BRQ_I8 = 2, BRQ_I32 = 3, BRQ_U8 = 4 };
enum brq_gran { BRQ_PER_TENSOR = 0, BRQ_PER_ROW = 1 };
enum brq_flag { BRQ_FLAG_NONFINITE = 1 };

/* Longest contraction whose int8 x int8 sums stay inside int32 for any
 * int8 codes, -128 included: 128 * 128 * 131071 < 2^31.  (The quantisers
 * here emit codes in [-127, 127]; the bound does not rely on it.) */
#define BRQ_MAX_CONTRACTION 131071

/* Launch geometry.  None of these fields changes any result bit. */
typedef struct brq_tune {
  int gemm_kernel;   /* 0 default (by shape), 1 reference (one output per
                        thread); register-staged MFMA tiles: 2 128x128,
                        3 256x128, 4 128x256, 5 256x256 (BK 64), 6 256x256,
                        7 256x256 (8 waves, BK 64), 8 256x256 (8 waves);
                        direct-to-LDS 4-stage MFMA tiles (contraction a
                        multiple of 64, else 2 is used): 9 256x256 (4 waves),
                        10 256x256 (8 waves), 11 128x256, 12 128x128,
                        13 256x256 (8 waves) persistent: one work-group
                        per CU walks its tiles with the load pipeline
                        running across tile boundaries (10 is used when a
                        tile's contraction slice has fewer than 4 steps of
                        64 or the slices are unequal), 14 256x256 (8 waves)
                        with 128-byte contraction steps through 2 stages
                        (contraction a multiple of 128, else 10 is used) */
  int split_k;       /* 0 default (by shape), else 1, 2, 4, 8 or 16
                        contraction slices (exact int32 partials) */
  int chunk_log2;    /* 0 default (13), else log2 of the leaves each
                        reduction work-group owns, in [10, 16] */
  int rows_per_block;/* 0 default, else RMSNorm backward rows per block:
                        1..64 power of two */
} brq_tune;

/* Workspace sizing.  `op` is one of brq_op; unused sizes are ignored. */
enum brq_op {
  BRQ_OP_QUANTIZE = 1,     /* a = rows, b = cols */
  BRQ_OP_QGEMM = 2,        /* a = M, b = N, c = K (fwd, dx, dw GEMMs) */
  BRQ_OP_DW_WHT = 3,       /* a = M, b = N, c = K, block = Hadamard block */
  BRQ_OP_RMSNORM_BWD = 4,  /* a = T, b = D */
  BRQ_OP_GRAD_NORM = 5,    /* a = n */
  BRQ_OP_DY_BWD = 6,       /* a = M, b = N, block = Hadamard block */
  BRQ_OP_QUANTIZE_EXACT = 7, /* a = rows, b = cols */
  BRQ_OP_DX_WHT = 8,        /* a = M, b = N, c = K, block = Hadamard block */
  BRQ_OP_DY_ROWS_WHT = 9,   /* a = M, b = N */
  BRQ_OP_QUANTIZE_X_WHT = 10 /* a = M, b = K, block = Hadamard block */
};
size_t brq_workspace_size(int op, int64_t a, int64_t b, int64_t c, int block,
                          const struct brq_tune* tune);

/* ---------------------------------------------------------------------
 * quantize_lsq -- LSQ fake-quantisation to int8 (§3.1 "int8
 * quantization-aware training", §4.2 "Implementation notes", §3.2 "int8
 * computation").
 *
 * x [rows][cols], dtype BRQ_F32 or BRQ_BF16.  When col_mul ([cols] fp32)
 * is given every element is first multiplied by col_mul[col].
 * For each group (the whole tensor for BRQ_PER_TENSOR, each row for
 * BRQ_PER_ROW) of n values v:
 *     S = tree(|v|);  s = fl(fl(S * fl(1/n)) * K2),  K2 = 2*fl(1/fl(sqrt 127))
 *     r = fl(1/s) (0 when s == 0);  q = clamp(rint(fl(v * r)), -127, 127)
 * Outputs: q [rows][cols] int8; q_t [cols][rows] int8 (optional);
 * scale [1] or [rows]; amax [1] or [rows] = max |v| (optional).
 * Raises BRQ_FLAG_NONFINITE when S is not finite.
 * Shapes: cols % 8 == 0 (bf16) / cols % 4 == 0 (fp32); BRQ_PER_ROW needs
 * cols <= 16384.  Workspace: BRQ_OP_QUANTIZE.
 * --------------------------------------------------------------------- */
int brq_quantize_lsq(const void* x, int x_dtype, int64_t rows, int64_t cols,
                     int gran, const float* col_mul, int8_t* q, int8_t* q_t,
                     float* scale, float* amax, void* ws, size_t ws_bytes,
                     int32_t* dflags, const struct brq_tune* tune, void* stream);

/* ---------------------------------------------------------------------
 * quantize_x_wht -- the per-tensor LSQ codes of an activation and the
 * integer Walsh-Hadamard rotation of those codes along tokens with its own
 * step, in one call (§3.1 "int8 quantization-aware training"; §3.2 "int8
 * computation": the rotation in front of the weight-gradient GEMM).
 * x [M][K] (BRQ_F32 or BRQ_BF16); outputs q_x [M][K] int8, s_x [1],
 * amax_x [1] (optional), q_ut [K][M] int8 (token-contiguous), s_u [1].
 * Every output equals brq_quantize_lsq(x, PER_TENSOR) followed by
 * brq_wht_quant_x on its codes, bit for bit; the codes and the rotation's
 * statistic come from one read of x.  Shapes, block and flags as those two
 * calls (M % 64 == 0, K % 64 == 0, M % block == 0, block a power of two in
 * [1, 128], M <= BRQ_MAX_CONTRACTION).  Workspace: BRQ_OP_QUANTIZE_X_WHT.
 * --------------------------------------------------------------------- */
int brq_quantize_x_wht(const void* x, int x_dtype, int64_t M, int64_t K, int block,
                       int8_t* q_x, float* s_x, float* amax_x, int8_t* q_ut,
                       float* s_u, void* ws, size_t ws_bytes, int32_t* dflags,
                       const struct brq_tune* tune, void* stream);

/* ---------------------------------------------------------------------
 * quantize_lsq_rows_multi -- the per-row (BRQ_PER_ROW) brq_quantize_lsq of
 * several tensors in one call: the per-channel weight steps of every linear
 * of a layer (§3.1 "int8 quantization-aware training": learned per-channel
 * step sizes for weights).  Each job is one tensor:
 *     x [rows][cols] (x_dtype BRQ_F32 or BRQ_BF16), q [rows][cols] int8,
 *     q_t [cols][rows] int8 or NULL, scale [rows], amax [rows] or NULL,
 * all device pointers owned by the caller; the results of every job are
 * those of brq_quantize_lsq(x, x_dtype, rows, cols, BRQ_PER_ROW, NULL, q,
 * q_t, scale, amax, ...) bit for bit.  Jobs of one element type and row
 * width class share one launch (up to 16 per launch), and every transpose
 * of the call shares one more.  No workspace.  Errors: count < 0 or
 * count > BRQ_ROWS_MULTI_MAX -> BRQ_E_ARG; a job failing the shape, dtype,
 * null or alignment rules of brq_quantize_lsq per row -> that code, and
 * nothing is launched.  A job with rows == 0 does nothing (its pointers
 * may be NULL).  Jobs must not overlap in their outputs.
 * --------------------------------------------------------------------- */
#define BRQ_ROWS_MULTI_MAX 1024
typedef struct brq_rows_job {
  const void* x;
  int x_dtype;
  int64_t rows, cols;
  int8_t* q;
  int8_t* q_t;
  float* scale;
  float* amax;
} brq_rows_job;
int brq_quantize_lsq_rows_multi(const brq_rows_job* jobs, int count,
                                int32_t* dflags, void* stream);

/* ---------------------------------------------------------------------
 * quantize_lsq_static -- brq_quantize_lsq without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  The per-tensor
 * statistic's tree partials live in one static device array of
 * BRQ_STATIC_SCRATCH_BYTES per GPU, created with the library's code object
 * and held until the process ends; nothing is allocated or freed here.
 * Results, arguments, shapes and flags are those of brq_quantize_lsq with
 * the same x, gran, col_mul and tune.  Nothing in the scratch needs to start
 * at zero (every partial is written before it is read).
 * Limits: a BRQ_PER_TENSOR input whose workspace (brq_workspace_size with
 * BRQ_OP_QUANTIZE) exceeds BRQ_STATIC_SCRATCH_BYTES returns BRQ_E_SCRATCH
 * before anything is launched (about 2^31 values at the default chunk).
 * BRQ_PER_ROW uses no scratch.  The scratch of the current device is used,
 * so `stream` must belong to it.  Every call on one GPU shares that GPU's
 * scratch: calls that may overlap in time on one GPU (different streams, no
 * ordering between them) race and give unspecified results.
 * --------------------------------------------------------------------- */
#define BRQ_STATIC_SCRATCH_BYTES (4u << 20)
int brq_quantize_lsq_static(const void* x, int x_dtype, int64_t rows,
                            int64_t cols, int gran, const float* col_mul,
                            int8_t* q, int8_t* q_t, float* scale, float* amax,
                            int32_t* dflags, const struct brq_tune* tune,
                            void* stream);

/* ---------------------------------------------------------------------
 * quantize_lsq_exact -- brq_quantize_lsq with an exact statistic (a
 * variant: the fixed-point accumulation that §3.2 "int8 computation" uses
 * to make the attention-gradient sum reproducible, applied to S).
 *     S = the exact real sum of |v| over the group, rounded once to
 *         binary32 (nearest even; a subnormal result flushes to +0; NaN if
 *         a v is NaN, else +inf if a v is infinite or the sum passes the
 *         binary32 range)
 * Every other step, argument, layout, shape rule and flag is as in
 * brq_quantize_lsq; amax is the largest |v| (0 if all are zero or
 * subnormal).  The bits depend on no launch shape, tune or add order.
 * Workspace: BRQ_OP_QUANTIZE_EXACT (BRQ_PER_TENSOR only).
 * --------------------------------------------------------------------- */
int brq_quantize_lsq_exact(const void* x, int x_dtype, int64_t rows,
                           int64_t cols, int gran, const float* col_mul,
                           int8_t* q, int8_t* q_t, float* scale, float* amax,
                           void* ws, size_t ws_bytes, int32_t* dflags,
                           const struct brq_tune* tune, void* stream);

/* ---------------------------------------------------------------------
 * qgemm_fwd -- forward W8A8 GEMM with int32 accumulation, then dequant
 * (§3.2 "int8 computation").
 *     acc[m][n] = sum_k q_x[m][k] * q_w[n][k]        (exact int32)
 *     y[m][n]   = fl(fl(acc) * fl(s_x[0] * s_w[n]))  (s_w[0] when
 *                                                     w_per_row == 0)
 * q_x [M][K], q_w [N][K] (nn.Linear layout), y [M][N] fp32.
 * Shapes: K % 16 == 0, K <= BRQ_MAX_CONTRACTION.  Workspace: BRQ_OP_QGEMM
 * (non-zero only when the plan splits the contraction).
 * --------------------------------------------------------------------- */
int brq_qgemm_fwd(const int8_t* q_x, const float* s_x, const int8_t* q_w,
                  const float* s_w, int w_per_row, int64_t M, int64_t N,
                  int64_t K, float* y, void* ws, size_t ws_bytes,
                  const struct brq_tune* tune, void* stream);

/* ---------------------------------------------------------------------
 * qgemm_bwd_dx -- input-gradient GEMM of the straight-through estimator
 * (§3.2 "int8 computation").  q_g is the int8 code of g = dY * s_w[n]
 * (quantize_lsq with col_mul = s_w), s_g its scale:
 *     dx[m][k] = fl(fl(sum_n q_g[m][n] * q_w[n][k]) * s_g[0])
 * q_g [M][N]; q_wt [K][N] is the transposed weight code (quantize_lsq's
 * q_t); dx [M][K] fp32.  Shapes: N % 16 == 0, N <= BRQ_MAX_CONTRACTION.
 * --------------------------------------------------------------------- */
int brq_qgemm_bwd_dx(const int8_t* q_g, const float* s_g, const int8_t* q_wt,
                     int64_t M, int64_t N, int64_t K, float* dx, void* ws,
                     size_t ws_bytes, const struct brq_tune* tune, void* stream);

/* Output-dtype variants of the two GEMMs above (a §8(f) variant: bf16
 * outputs, the dtype the next layer's input and the activation gradient
 * take).  y_dtype / dx_dtype: BRQ_F32 (identical to the calls above) or
 * BRQ_BF16, where each output is the fp32 value of the definition rounded
 * once to bf16 (nearest even).  y / dx must be 16-byte aligned. */
int brq_qgemm_fwd_ex(const int8_t* q_x, const float* s_x, const int8_t* q_w,
                     const float* s_w, int w_per_row, int64_t M, int64_t N, int64_t K,
                     void* y, int y_dtype, void* ws, size_t ws_bytes,
                     const struct brq_tune* tune, void* stream);
int brq_qgemm_bwd_dx_ex(const int8_t* q_g, const float* s_g, const int8_t* q_wt,
                        int64_t M, int64_t N, int64_t K, void* dx, int dx_dtype,
                        void* ws, size_t ws_bytes, const struct brq_tune* tune,
                        void* stream);

/* ---------------------------------------------------------------------
 * qgemm_bwd_dw_wht -- weight-gradient GEMM in int8 after a Walsh-Hadamard
 * rotation along tokens (§3.2 "int8 computation").  With H_b the
 * unnormalised Sylvester matrix, H[i][j] = (-1)^popcount(i & j), applied
 * per aligned block of `block` tokens:
 *     u = H q_x (exact integers); S_u = sum |u| (exact); s_u from S_u as
 *         quantize_lsq (fl(double(S_u)) first); q_u = quantised u
 *     v = fp32 butterflies of dY in stage order h = 1, 2, ..., block/2,
 *         (v_j, v_j+h) <- (fl(v_j + v_j+h), fl(v_j - v_j+h));
 *         per-tensor LSQ over v in row-major [M][N] order -> q_v, s_v
 *     dw[n][k] = fl(fl(sum_m q_v[m][n] * q_u[m][k]) * c_w),
 *     c_w = fl(fl(fl(s_x * s_u) * s_v) * 2^-log2(block))
 * q_x [M][K] (the forward activation code), dy [M][N] (BRQ_F32 or BRQ_BF16),
 * dw [N][K] fp32; s_u_out, s_v_out optional device floats.
 * Shapes: block a power of two in [1, 128], M % block == 0, M % 64 == 0,
 * K % 64 == 0, N % 64 == 0, M <= BRQ_MAX_CONTRACTION.
 * Workspace: BRQ_OP_DW_WHT (it holds the rotated codes q_u^T [K][M] and
 * q_v^T [N][M] at the start, in that order).
 * --------------------------------------------------------------------- */
int brq_qgemm_bwd_dw_wht(const int8_t* q_x, const float* s_x, const void* dy,
                         int dy_dtype, int64_t M, int64_t N, int64_t K,
                         int block, float* dw, float* s_u_out, float* s_v_out,
                         void* ws, size_t ws_bytes, int32_t* dflags,
                         const struct brq_tune* tune, void* stream);

/* The three stages of qgemm_bwd_dw_wht, callable on their own.
 * brq_wht_quant_x: q_x [M][K] -> q_ut [K][M] (token-contiguous), s_u [1].
 * brq_wht_quant_dy: dy [M][N] -> q_vt [N][M], s_v [1].
 * brq_qgemm_dw: dw [N][K] from q_vt, q_ut and the scales (device floats).
 * Workspace for the first two: BRQ_OP_DW_WHT. */
int brq_wht_quant_x(const int8_t* q_x, int64_t M, int64_t K, int block,
                    int8_t* q_ut, float* s_u, void* ws, size_t ws_bytes,
                    const struct brq_tune* tune, void* stream);
int brq_wht_quant_dy(const void* dy, int dy_dtype, int64_t M, int64_t N,
                     int block, int8_t* q_vt, float* s_v, void* ws,
                     size_t ws_bytes, int32_t* dflags,
                     const struct brq_tune* tune, void* stream);
int brq_qgemm_dw(const int8_t* q_vt, const int8_t* q_ut, const float* s_x,
                 const float* s_u, const float* s_v, int64_t M, int64_t N,
                 int64_t K, int block, float* dw, void* ws, size_t ws_bytes,
                 const struct brq_tune* tune, void* stream);

/* ---------------------------------------------------------------------
 * qgemm_bwd_dx_wht -- the input-gradient GEMM with the Walsh-Hadamard
 * rotation along its contraction n (a variant: §3.2 "int8 computation"
 * puts the rotation in front of both straight-through gradient GEMMs).
 *     g   = fl(dy[m][n] * s_w[n]); per row m and aligned block of `block`
 *           consecutive n, fp32 butterflies in stage order h = 1, 2, ...,
 *           block/2: (g_j, g_j+h) <- (fl(g_j + g_j+h), fl(g_j - g_j+h));
 *           per-tensor LSQ over the rotated g (tree statistic) -> q_g, s_g
 *     q_h = q_w [N][K] rotated exactly along n per column k and requantised,
 *           as brq_wht_quant_x does for q_x along tokens -> s_h
 *     dx[m][k] = fl(fl(sum_n q_g[m][n] * q_h[n][k]) * c),
 *     c = fl(fl(s_g * s_h) * 2^-log2(block))
 * dy [M][N] (BRQ_F32 or BRQ_BF16), s_w [N] fp32 (per-channel weight steps),
 * q_w [N][K] int8 (the forward weight code), dx [M][K] fp32; s_g_out and
 * s_h_out optional device floats.  Shapes: block a power of two in
 * [1, 128]; M % 16 == 0; N > 0, N % 64 == 0, N % block == 0; K % 64 == 0;
 * N <= BRQ_MAX_CONTRACTION.  M == 0 or K == 0 computes nothing.  Raises
 * BRQ_FLAG_NONFINITE when s_g's statistic is not finite.
 * Workspace: BRQ_OP_DX_WHT.
 *
 * brq_wht_quant_dy_rows: its first stage on its own, q_g [M][N] and s_g [1].
 * Workspace: BRQ_OP_DY_ROWS_WHT.
 * --------------------------------------------------------------------- */
int brq_qgemm_bwd_dx_wht(const void* dy, int dy_dtype, const float* s_w,
                         const int8_t* q_w, int64_t M, int64_t N, int64_t K,
                         int block, float* dx, float* s_g_out, float* s_h_out,
                         void* ws, size_t ws_bytes, int32_t* dflags,
                         const struct brq_tune* tune, void* stream);
int brq_wht_quant_dy_rows(const void* dy, int dy_dtype, int64_t M, int64_t N,
                          const float* s_w, int block, int8_t* q_g, float* s_g,
                          void* ws, size_t ws_bytes, int32_t* dflags,
                          const struct brq_tune* tune, void* stream);

/* ---------------------------------------------------------------------
 * attn_fwd -- attention forward with an int8 P.V product (a variant:
 * §3.2 "int8 computation" quantises the attention weights and values to
 * int8 per block for the P.V product, QK^T and softmax in higher
 * precision; §3.1: grouped-query attention, causal, sliding window).
 * q [Hq][T][d], k, v [Hkv][T][d] bf16; o [Hq][T][d] fp32.  Query head h
 * reads key/value head h / (Hq / Hkv); key j is visible from query i iff
 * i - window < j <= i (window >= T: plain causal).  Per 64-query block and
 * ascending 64-key blocks, every step one rounded, flushed binary32 op:
 *     S_ij = fl(dot_ij * c), c = fl(1/fl(sqrt d)), dot_ij sequential over
 *            e of the exact bf16 products;
 *     m = max(m, block max); a = exp_f(m_old - m) (0 while m_old = -inf);
 *     p = exp_f(S - m) (0 for a hidden key); l = fl(fl(l * a) + tree(p));
 *     s_p = fl(max_tile p * fl(1/127)), s_v = fl(max_block |v| * fl(1/127));
 *     codes clamp(rint(fl(x * fl(1/s))), -127, 127);
 *     o = fl(fl(o * a) + fl(fl(sum_j qp_ij qv_je) * fl(s_p * s_v)));
 *     finally o = fl(o * fl(1/l)).
 * exp_f: Cody-Waite reduction by ln 2 (head 0x3f317200, tail 0x35bfbe8e,
 * fl(1/ln 2) = 0x3fb8aa3b), n = rint(fl(x / ln 2)), degree-7 Taylor
 * polynomial in Horner form with coefficients fl(1/i!), times 2^n; 0 for
 * x < -104 or n < -126.  A row with no visible key in a block is left as
 * it was.  Shapes: d = 64 or 128, T % 64 == 0, Hq % Hkv == 0.
 * --------------------------------------------------------------------- */
int brq_attn_fwd(const void* q, const void* k, const void* v, int64_t Hq,
                 int64_t Hkv, int64_t T, int64_t d, int64_t window, float* o,
                 int32_t* dflags, const struct brq_tune* tune, void* stream);

/* ---------------------------------------------------------------------
 * quantize_dy_bwd -- both int8 codes of the upstream gradient for the two
 * straight-through gradient GEMMs (§3.2 "int8 computation"), in two passes
 * over dY.  Bit-identical to the two calls it fuses:
 *     q_g, s_g, amax_g  = brq_quantize_lsq(dy, PER_TENSOR, col_mul = s_w)
 *     q_vt, s_v         = brq_wht_quant_dy(dy, block)
 * dy [M][N] (BRQ_F32 or BRQ_BF16), s_w [N] fp32 (the per-channel weight
 * step sizes), q_g [M][N] int8, q_vt [N][M] int8 (token-contiguous),
 * s_g, s_v [1] fp32, amax_g [1] fp32 or NULL.  Shapes as brq_wht_quant_dy.
 * The two-pass form runs for bf16 with M % 128 == 0; other shapes run the
 * two definitions in sequence.  Raises BRQ_FLAG_NONFINITE when a statistic
 * is not finite.  Workspace: BRQ_OP_DY_BWD.
 * --------------------------------------------------------------------- */
int brq_quantize_dy_bwd(const void* dy, int dy_dtype, int64_t M, int64_t N,
                        const float* s_w, int block, int8_t* q_g, float* s_g,
                        float* amax_g, int8_t* q_vt, float* s_v, void* ws,
                        size_t ws_bytes, int32_t* dflags,
                        const struct brq_tune* tune, void* stream);

/* ---------------------------------------------------------------------
 * rmsnorm_fixed -- RMSNorm in FP32 with a fixed reduction order (§3.1
 * "RMSNorm": pre-norm, no bias; normalisation computed in FP32).
 * Forward per row t of x [T][D]:
 *     ss = tree(fl(x*x));  ms = fl(ss * fl(1/D));
 *     rstd[t] = fl(1 / fl(sqrt(fl(ms + eps))));  y = fl(fl(x * rstd) * g)
 * Backward:  xh = fl(x * rstd); d = fl(dy * g); dot = tree(fl(d * xh));
 *     mu = fl(dot * fl(1/D)); dx = fl(rstd * fl(d - fl(xh * mu)));
 *     dg[j] = tree over tokens t of fl(dy[t][j] * xh[t][j])   (fp32)
 * x, g, y, dy, dx share `dtype` (BRQ_F32 or BRQ_BF16; bf16 results round to
 * nearest even); rstd [T] fp32.  Shapes: D % 8 == 0; forward D <= 16384
 * (bf16) or 8192 (fp32); backward D <= 4096 (bf16) or 2048 (fp32).
 * Backward workspace: BRQ_OP_RMSNORM_BWD.
 * --------------------------------------------------------------------- */
int brq_rmsnorm_fixed_fwd(const void* x, const void* g, int dtype, int64_t T,
                          int64_t D, float eps, void* y, float* rstd,
                          int32_t* dflags, const struct brq_tune* tune,
                          void* stream);
int brq_rmsnorm_fixed_bwd(const void* x, const void* g, const float* rstd,
                          const void* dy, int dtype, int64_t T, int64_t D,
                          void* dx, float* dg, void* ws, size_t ws_bytes,
                          const struct brq_tune* tune, void* stream);

/* ---------------------------------------------------------------------
 * grad_norm -- global l2 norm of the FP32 gradients (§3.2 "Optimizer":
 * clipping at global norm 1.0):  ss = tree(fl(v*v)) over v[0..n),
 * norm = fl(sqrt(ss)).  sumsq, norm: device floats.  Raises
 * BRQ_FLAG_NONFINITE when ss is not finite.  Workspace: BRQ_OP_GRAD_NORM.
 * --------------------------------------------------------------------- */
int brq_grad_norm(const float* v, int64_t n, float* sumsq, float* norm,
                  void* ws, size_t ws_bytes, int32_t* dflags,
                  const struct brq_tune* tune, void* stream);

/* ---------------------------------------------------------------------
 * hash_state -- on-device canonical state hash (§5 "Runtime overhead" and
 * App. B: a per-step state hash, computed here on the device).
 *   leaf digests: SHA-256 (FIPS 180-4) of each 4096-byte slice of a
 *     tensor's raw bytes (the last slice may be shorter; an empty tensor
 *     has one empty leaf);
 *   levels: SHA-256 of the concatenation of up to 128 consecutive digests,
 *     repeated until one root remains;
 *   tensor digest: SHA-256("BRQ1" | dtype u8 | ndim u8 | dims u64 LE ... |
 *     name length u16 LE | name bytes | root);
 *   state digest: SHA-256 of the tensor digests in call order.
 * t[i].data are device pointers (16-byte aligned); digest32 is a device
 * buffer of 32 bytes.  Workspace: brq_hash_workspace_size(t, n).
 * --------------------------------------------------------------------- */
typedef struct brq_tensor_ref {
  const void* data;
  int dtype;          /* brq_dtype code, hashed into the tensor digest */
  int ndim;           /* 0..8 */
  int64_t dims[8];
  const char* name;   /* at most 255 bytes */
} brq_tensor_ref;

size_t brq_hash_workspace_size(const brq_tensor_ref* t, int n);
int brq_hash_state(const brq_tensor_ref* t, int n, uint8_t* digest32, void* ws,
                   size_t ws_bytes, void* stream);

/* hash_state in its two halves, so each tensor can be digested as soon as it
 * is final (for instance on a second stream, overlapping other work):
 *   brq_hash_tensor_digests: digests[32 i .. 32 i + 31] = tensor digest of
 *     t[i] (the Merkle root under its typed header, as above); `digests` is
 *     a 16-byte aligned device buffer of 32 n bytes.  Workspace:
 *     brq_hash_digests_workspace_size(t, n); calls that overlap need
 *     distinct workspaces.
 *   brq_hash_combine: digest32 = SHA-256 of the n digests in order.
 * brq_hash_state(t, n) equals brq_hash_combine over the digests of t. */
size_t brq_hash_digests_workspace_size(const brq_tensor_ref* t, int n);
int brq_hash_tensor_digests(const brq_tensor_ref* t, int n, uint8_t* digests,
                            void* ws, size_t ws_bytes, void* stream);
int brq_hash_combine(const uint8_t* digests, int n, uint8_t* digest32,
                     void* stream);

/* brq_hash_tensor_digests in two stages, so that a step's hash need not
 * hold up the next step (same definitions as above):
 *   brq_hash_tensor_leaves: the leaf digests of every t[i] into ws -- the
 *     only stage that reads the tensors; once it has completed on `stream`
 *     they may be overwritten.
 *   brq_hash_tensor_finish: every level above the leaves and the tensor
 *     digests into `digests`, reading only ws (the tensors' sizes, dtypes
 *     and names come from t; t[i].data is checked as by the leaves stage
 *     but not dereferenced), so it may run on another stream once the
 *     leaves stage has completed (§5 "Strong Scaling", Table 11: the
 *     per-step hash lowers the run's throughput).
 * Both take the same t, n and workspace (brq_hash_digests_workspace_size);
 * the workspace must not be used by anything else from the start of the
 * leaves stage until the finish stage has completed.  Errors as
 * brq_hash_tensor_digests. */
int brq_hash_tensor_leaves(const brq_tensor_ref* t, int n, void* ws, size_t ws_bytes,
                           void* stream);
int brq_hash_tensor_finish(const brq_tensor_ref* t, int n, uint8_t* digests, void* ws,
                           size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------
 * Optimizer step after the layer: AdamW with global-norm clipping and the
 * spike protocol (§3.2 "Optimizer": beta1 0.9, beta2 0.95, eps 1e-8,
 * decoupled weight decay 0.1 on linear layers and none on normalisation
 * weights, global l2 clip at 1.0; §3.2 "Optimizer-state precision": BF16
 * parameters, FP32 moments, widen -> update in FP32 -> round to BF16 once;
 * §3.4.2 "Gradient behavior, Clipping, and Spike Protocol": five optimizer
 * steps skipped when the pre-clip norm exceeds 5).
 *
 * Per element, each operation one rounded binary32 operation, flushed:
 *   g = g * clip (when clip != 1)
 *   m = b1*m + (1-b1)*g          v = b2*v + (1-b2)*(g*g)
 *   u = (m / bc1) / (sqrt(v / bc2) + eps)
 *   p = p - lr*(u + wd*p)
 * --------------------------------------------------------------------- */
typedef struct brq_adamw_hparams {
  float lr;
  float beta1, beta2, eps;
  float weight_decay;      /* 0 for normalisation weights */
  float bias_correction1;  /* 1 - beta1^t (brq_adamw_bias_corrections) */
  float bias_correction2;  /* 1 - beta2^t */
} brq_adamw_hparams;

/* Host: bias corrections of optimizer step t >= 1: bc = 1 - beta^t with
 * beta^t the t-fold product of rounded binary32 multiplies (subnormal
 * products flushed).  BRQ_E_ARG for t < 1 or NULL outputs. */
int brq_adamw_bias_corrections(int64_t t, float beta1, float beta2, float* bc1,
                               float* bc2);

/* Device: the step's decision from the pre-clip global norm (norm: device
 * float, e.g. the second output of brq_grad_norm).  A norm above
 * spike_threshold, or not finite, (re)starts a window of skip_steps skipped
 * steps, this one first; inside a window ctl = {0, 0}.  Otherwise
 * ctl = {1, clip} with clip = max_norm / norm for a norm above max_norm, else
 * 1.  skip_state: device int32 [1], the skipped steps still due (start at 0).
 * ctl: device float [2].  A non-finite norm raises BRQ_FLAG_NONFINITE in
 * dflags (may be NULL). */
int brq_adamw_decide(const float* norm, float max_norm, float spike_threshold,
                     int skip_steps, int32_t* skip_state, float* ctl,
                     int32_t* dflags, void* stream);

/* Device: one AdamW update of n elements in place.  param BRQ_BF16 or
 * BRQ_F32, grad BRQ_F32 or BRQ_BF16, m and v fp32; all [n], 16-byte
 * aligned, not overlapping.  ctl: the decision of brq_adamw_decide (device);
 * with ctl[0] == 0 nothing is written.  No workspace. */
int brq_adamw_step(void* param, int param_dtype, const void* grad, int grad_dtype,
                   float* m, float* v, int64_t n, const brq_adamw_hparams* hp,
                   const float* ctl, void* stream);

/* ---------------------------------------------------------------------
 * dp_reduce -- the arithmetic of the deterministic data-parallel gradient
 * exchange (App. A "Deterministic Gradient Reduction"), over contributions
 * resident on this device.  Per element i, every operation one rounded
 * binary32 operation (inputs read with DAZ, results flushed):
 *   for each replica r and shard s: g = c[r][s][0] + c[r][s][1] + ...,
 *     a running sum over the accum microbatches in order; g = fl(g * fl(1/A));
 *   for each replica r: inner = g[r][0] + g[r][1] + ..., a running sum over
 *     the shards in ascending rank order (App. A.2, the local sum of the
 *     deterministic reduce-scatter after its all-to-all);
 *     p[r] = fl(inner * fl(1/S));
 *   TreeFold over p[0..R) (App. A.1, the pairing of the recursive-doubling
 *     all-reduce): each p[r] is pushed once onto a stack of (level, value);
 *     an entry merges with the top while their levels are equal, the
 *     stack's (lower-replica) value on the left, and moves one level up;
 *     the entries left (one per set bit of R) are combined from the lowest
 *     level (the smallest block) up, the lower-replica block on the left.
 *     For R a power of two this is the balanced pairwise tree.
 *   out[i] = fl(result * fl(1/R)).
 * Each fl(1/k) is the binary32 reciprocal of the count (App. A.3: averages
 * are reciprocal multiplies, never divisions); with average == 0 no level
 * multiplies.  Special cases: replicas = accum = 1 is the reduce-scatter's
 * ascending-rank sum; shards = accum = 1 is the replica all-reduce; R = 2,
 * S = A = 1, average = 0 is one recursive-doubling hop fl(lo + hi).
 * parts: HOST array of replicas*shards*accum DEVICE pointers in mesh order
 * (replica-major, then shard, then microbatch), each [n] fp32, 16-byte
 * aligned; out [n] fp32, 16-byte aligned, may be one of the parts (in
 * place).  1 <= replicas*shards*accum <= BRQ_DP_MAX_PARTS.  Raises
 * BRQ_FLAG_NONFINITE when an output is not finite.  No workspace.
 * --------------------------------------------------------------------- */
#define BRQ_DP_MAX_PARTS 64
int brq_dp_reduce(const float* const* parts, int replicas, int shards, int accum,
                  int64_t n, int average, float* out, int32_t* dflags, void* stream);

/* ---------------------------------------------------------------------
 * fp32_primitive -- the device's binary32 primitives over a range of inputs,
 * to check them bit for bit against another machine (§2 "The same
 * operation compiles to different instructions", §2.1 Table 1).  Input i
 * is the binary32 bit pattern x = first + i (mod 2^32), i < count; out[i]
 * (device uint32 [count], 16-byte aligned) receives the result's bits:
 *   BRQ_PRIM_SQRT      fl(sqrt(daz(x)))             (grad-norm, AdamW)
 *   BRQ_PRIM_RCP       fl(1 / daz(x))               (quantiser reciprocal)
 *   BRQ_PRIM_RSQRT     fl(1 / fl(sqrt(daz(x))))     (RMSNorm rstd)
 *   BRQ_PRIM_BF16_CVT  bf16 of x, nearest even, by the conversion
 *                      instruction the bf16 stores use (low 16 bits)
 *   BRQ_PRIM_BF16_INT  bf16 of x, nearest even, by integer arithmetic on
 *                      the bit pattern (low 16 bits)
 * daz() reads a subnormal as a signed zero and fl() flushes a subnormal
 * result, as in every kernel; division and square root are the ones every
 * kernel uses.  A NaN result may carry any quiet-NaN payload.  No
 * workspace; count <= 2^32.
 * --------------------------------------------------------------------- */
enum brq_prim {
  BRQ_PRIM_SQRT = 0,
  BRQ_PRIM_RCP = 1,
  BRQ_PRIM_RSQRT = 2,
  BRQ_PRIM_BF16_CVT = 3,
  BRQ_PRIM_BF16_INT = 4
};
int brq_fp32_primitive(int prim, uint32_t first, int64_t count, uint32_t* out,
                       void* stream);

/* Status text, HIP error of the last BRQ_E_HIP in this thread, version. */
const char* brq_status_string(int status);
int brq_last_hip_error(void);
int brq_spec_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BRQ_H */
