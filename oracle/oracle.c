/*
 * oracle.c -- plain, sequential CPU oracle (TEST INFRASTRUCTURE ONLY).
 *
 * Compiled with gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math on
 * x86-64 (SSE2 scalar arithmetic, default MXCSR: round to nearest even,
 * gradual underflow).  The flush of subnormals is written out below, so
 * the hardware flush modes are never relied upon.
 *
 * OpenMP (when enabled) only splits loops over independent outputs: every
 * output value is produced by the same sequential code whatever the thread
 * count, so results do not depend on it.  Reductions never run in parallel.
 *
 * Page references are to "Open-1B: A Fully Auditable Training Run"
 * (arXiv 2609.17380): section, table or appendix named at each routine.
 */
#include "oracle.h"

#include <assert.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* Threads the OpenMP loops over independent outputs may use (1 without
 * OpenMP); reported next to the oracle's timings. */
int orc_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void orc_set_num_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ------------------------------------------------------------------------
 * Arithmetic model -- §2.1 "Subnormals", "Fused multiply-add", Table 1.
 * Each helper performs exactly one IEEE binary32 operation and then flushes
 * a subnormal result to a zero of the same sign.
 * ---------------------------------------------------------------------- */
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

float orc_flush(float v) {
  uint32_t u = f2u(v);
  if ((u & 0x7f800000u) == 0) u &= 0x80000000u;
  return u2f(u);
}
static float fadd(float a, float b) { return orc_flush(a + b); }
static float fsub(float a, float b) { return orc_flush(a - b); }
static float fmul(float a, float b) { return orc_flush(a * b); }
static float fdiv(float a, float b) { return orc_flush(a / b); }
static float fsqrt(float a) { return orc_flush(sqrtf(a)); }
static float fabs_(float a) { return u2f(f2u(a) & 0x7fffffffu); }

float orc_bf16_to_f32(uint16_t h) { return orc_flush(u2f((uint32_t)h << 16)); }

uint16_t orc_f32_to_bf16(float f) {
  uint32_t u = f2u(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* bf16 rounding of a whole fp32 tensor (the bf16-output variant of the
 * GEMMs: each fp32 result rounded once, nearest even). */
void orc_f32_to_bf16_array(const float* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = orc_f32_to_bf16(in[i]);
}

/* Element i of a tensor of dtype F32 or BF16, after DAZ. */
static float load(const void* p, int dtype, int64_t i) {
  if (dtype == ORC_BF16) return orc_bf16_to_f32(((const uint16_t*)p)[i]);
  return orc_flush(((const float*)p)[i]);
}
static void store(void* p, int dtype, int64_t i, float v) {
  if (dtype == ORC_BF16) ((uint16_t*)p)[i] = orc_f32_to_bf16(v);
  else ((float*)p)[i] = v;
}

/* The model's primitives over a range of bit patterns, input i being the
 * pattern first + i: the host side of a sweep that compares a device's
 * division, square root and bf16 rounding with these (§2 "The same operation
 * compiles to different instructions").  x86 SSE division and square root
 * are the correctly rounded IEEE operations. */
void orc_prim_sweep(int prim, uint32_t first, int64_t count, uint32_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; i++) {
    const float x = u2f(first + (uint32_t)i);
    uint32_t r;
    switch (prim) {
      case 0: r = f2u(fsqrt(orc_flush(x))); break;
      case 1: r = f2u(fdiv(1.0f, orc_flush(x))); break;
      case 2: r = f2u(fdiv(1.0f, fsqrt(orc_flush(x)))); break;
      default: r = orc_f32_to_bf16(x); break;
    }
    out[i] = r;
  }
}

/* ------------------------------------------------------------------------
 * Canonical reduction tree -- §2.1 "Reduction order", Table 1 row 2.
 * Level 0 holds the leaves in logical row-major order; each level pairs
 * neighbours (2i, 2i+1) with the lower index on the left, and an unpaired
 * last node moves up unchanged.  The root is the sum.
 * ---------------------------------------------------------------------- */
static float tree_inplace(float* buf, int64_t n) {
  if (n <= 0) return 0.0f;
  int64_t len = n;
  while (len > 1) {
    int64_t half = len / 2;
    for (int64_t i = 0; i < half; i++) buf[i] = fadd(buf[2 * i], buf[2 * i + 1]);
    if (len & 1) {
      buf[half] = buf[len - 1];
      len = half + 1;
    } else {
      len = half;
    }
  }
  return buf[0];
}

float orc_tree_sum(const float* leaves, int64_t n) {
  if (n <= 0) return 0.0f;
  float* buf = (float*)malloc((size_t)n * sizeof(float));
  assert(buf);
  memcpy(buf, leaves, (size_t)n * sizeof(float));
  float s = tree_inplace(buf, n);
  free(buf);
  return s;
}

/* The same tree, coded top-down: the root's left child covers the largest
 * power of two strictly below n, the right child covers the rest. */
static float tree_rec(const float* l, int64_t n) {
  if (n == 1) return l[0];
  int64_t p = 1;
  while (p * 2 < n) p *= 2;
  return fadd(tree_rec(l, p), tree_rec(l + p, n - p));
}
float orc_tree_sum_recursive(const float* leaves, int64_t n) {
  if (n <= 0) return 0.0f;
  return tree_rec(leaves, n);
}

/* ------------------------------------------------------------------------
 * LSQ quantiser -- §3.1 "int8 quantization-aware training", §4.2: the
 * step size is 2*mean(|w|)/sqrt(q_max) with q_max = 127, re-evaluated from
 * the tensor it quantises.  App. A.3: the mean multiplies by fl(1/n) and
 * the division by sqrt(q_max) is a multiply by its fp32 reciprocal, so the
 * factor is K2 = 2 * fl(1/fl(sqrt(127))).  The quantiser divides by the
 * step as a multiply by r = fl(1/s), rounds half to even, clamps to +-127.
 * ---------------------------------------------------------------------- */
float orc_lsq_k2(void) {
  volatile float q = 127.0f;
  float rs = fdiv(1.0f, fsqrt(q));
  return fmul(2.0f, rs);
}

static float inv_count(int64_t n) { return fdiv(1.0f, (float)n); }

void orc_lsq_scale(float S, int64_t n, float* s_out, float* r_out) {
  if (n == 0) { /* an empty group has step size 0: no mean is taken */
    *s_out = 0.0f;
    *r_out = 0.0f;
    return;
  }
  float m = fmul(S, inv_count(n));
  float s = fmul(m, orc_lsq_k2());
  *s_out = s;
  *r_out = (s == 0.0f) ? 0.0f : fdiv(1.0f, s);
}

int8_t orc_quant1(float x, float r) {
  float t = rintf(fmul(x, r));
  if (t > 127.0f) t = 127.0f;
  if (t < -127.0f) t = -127.0f;
  return (int8_t)t;
}

/* ------------------------------------------------------------------------
 * Exact statistic (a variant of the step-size statistic): the sum of |v|
 * taken exactly and rounded once.  §3.2 "int8 computation" reaches bitwise
 * reproducibility for the ∇Q accumulation of attention by summing in fixed
 * point; here the same idea is applied to Σ|v|.  Every binary32 value is a
 * whole multiple of 2^-149, so Σ|v| is a whole number N of such units.  N
 * is kept in an array of 32-bit words wide enough for any input (the
 * largest finite |v| is below 2^277 units, and n < 2^40), so no addition
 * ever rounds and the order of the additions is immaterial.  N * 2^-149 is
 * then rounded to binary32 once, to nearest, ties to even, and flushed like
 * any other result (§2.1 "Subnormals").  A NaN among the inputs makes the
 * sum NaN, otherwise an infinity makes it +inf; a sum beyond the binary32
 * range rounds to +inf.
 * ---------------------------------------------------------------------- */
#define EXACT_WORDS 10 /* 320 bits */

/* N += m * 2^bit, m < 2^24, with the carry run to the top. */
static void exact_add(uint32_t* w, uint32_t m, int bit) {
  int k = bit / 32;
  uint64_t add = (uint64_t)m << (bit % 32); /* < 2^55: spans words k, k+1 */
  for (; add != 0 && k < EXACT_WORDS; k++) {
    uint64_t t = (uint64_t)w[k] + (add & 0xffffffffu);
    w[k] = (uint32_t)t;
    add = (add >> 32) + (t >> 32);
  }
  assert(add == 0);
}

/* Bit `i` of N. */
static int exact_bit(const uint32_t* w, int i) { return (int)((w[i / 32] >> (i % 32)) & 1u); }

float orc_exact_abs_sum(const float* v, int64_t n) {
  uint32_t w[EXACT_WORDS];
  memset(w, 0, sizeof w);
  int any_nan = 0, any_inf = 0;
  for (int64_t i = 0; i < n; i++) {
    uint32_t u = f2u(orc_flush(v[i])) & 0x7fffffffu;
    uint32_t e = u >> 23, frac = u & 0x7fffffu;
    if (e == 255) {
      if (frac) any_nan = 1; else any_inf = 1;
      continue;
    }
    if (e == 0) continue; /* zero (subnormals were flushed) */
    /* |v| = (2^23 + frac) * 2^(e-150) = (2^23 + frac) * 2^(e-1) units */
    exact_add(w, 0x800000u | frac, (int)e - 1);
  }
  if (any_nan) return u2f(0x7fc00000u);
  if (any_inf) return u2f(0x7f800000u);
  int top = -1; /* index of the highest set bit of N */
  for (int i = 32 * EXACT_WORDS - 1; i >= 0; i--)
    if (exact_bit(w, i)) { top = i; break; }
  if (top < 0) return 0.0f;
  /* keep the 24 bits top..top-23 (fewer when N < 2^24: then exact) */
  int lo = top - 23 < 0 ? 0 : top - 23;
  uint32_t q = 0;
  for (int i = top; i >= lo; i--) q = (q << 1) | (uint32_t)exact_bit(w, i);
  if (lo > 0) {
    int half = exact_bit(w, lo - 1), sticky = 0;
    for (int i = lo - 2; i >= 0 && !sticky; i--) sticky = exact_bit(w, i);
    if (half && (sticky || (q & 1u))) q++;
    if (q == (1u << 24)) { q >>= 1; lo++; }
  }
  /* value = q * 2^(lo - 149); q < 2^24 so the double is exact */
  if (lo - 149 + 23 > 127) return u2f(0x7f800000u);
  return orc_flush((float)ldexp((double)q, lo - 149));
}

/* One quantisation group of n values: the statistic S of |v| (the
 * canonical tree, or the exact sum above), scale, codes. */
static int lsq_group(const float* v, int64_t n, int exact, int8_t* q,
                     float* s_out, float* amax_out) {
  float amax = 0.0f, S;
  for (int64_t i = 0; i < n; i++)
    if (fabs_(v[i]) > amax) amax = fabs_(v[i]);
  if (exact) {
    S = orc_exact_abs_sum(v, n);
  } else {
    float* leaves = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    assert(leaves);
    for (int64_t i = 0; i < n; i++) leaves[i] = fabs_(v[i]);
    S = tree_inplace(leaves, n);
    free(leaves);
  }
  float s, r;
  orc_lsq_scale(S, n, &s, &r);
  for (int64_t i = 0; i < n; i++) q[i] = orc_quant1(v[i], r);
  *s_out = s;
  if (amax_out) *amax_out = amax;
  return isfinite(S) ? 0 : ORC_FLAG_NONFINITE;
}

static int quantize_common(const void* x, int dtype, int64_t rows, int64_t cols,
                           int gran, const float* col_mul, int exact, int8_t* q,
                           int8_t* q_t, float* scale, float* amax) {
  int64_t n = rows * cols;
  float* v = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
  assert(v);
  for (int64_t i = 0; i < n; i++) {
    float e = load(x, dtype, i);
    if (col_mul) e = fmul(e, orc_flush(col_mul[i % cols]));
    v[i] = e;
  }
  int flags = 0;
  if (gran == ORC_PER_TENSOR) {
    flags |= lsq_group(v, n, exact, q, &scale[0], amax ? &amax[0] : NULL);
  } else {
    for (int64_t r = 0; r < rows; r++)
      flags |= lsq_group(v + r * cols, cols, exact, q + r * cols, &scale[r],
                         amax ? &amax[r] : NULL);
  }
  if (q_t)
    for (int64_t r = 0; r < rows; r++)
      for (int64_t c = 0; c < cols; c++) q_t[c * rows + r] = q[r * cols + c];
  free(v);
  return flags;
}

int orc_quantize_lsq(const void* x, int dtype, int64_t rows, int64_t cols,
                     int gran, const float* col_mul, int8_t* q, int8_t* q_t,
                     float* scale, float* amax) {
  return quantize_common(x, dtype, rows, cols, gran, col_mul, 0, q, q_t, scale, amax);
}

int orc_quantize_lsq_exact(const void* x, int dtype, int64_t rows, int64_t cols,
                           int gran, const float* col_mul, int8_t* q, int8_t* q_t,
                           float* scale, float* amax) {
  return quantize_common(x, dtype, rows, cols, gran, col_mul, 1, q, q_t, scale, amax);
}

/* ------------------------------------------------------------------------
 * int8 GEMMs -- §3.2 "int8 computation": int32 accumulation, then
 * dequantisation.  The integer sum is exact, so its order is immaterial;
 * int64 is used here and the int32 range is asserted.
 * ---------------------------------------------------------------------- */
static float acc_to_f32(int64_t acc) {
  assert(acc <= INT32_MAX && acc >= INT32_MIN);
  return (float)(int32_t)acc; /* int32 -> binary32, round to nearest even */
}

void orc_qgemm_fwd(const int8_t* qx, const float* s_x, const int8_t* qw,
                   const float* s_w, int w_per_row, int64_t M, int64_t N,
                   int64_t K, float* y) {
  float sx = orc_flush(s_x[0]);
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int64_t m = 0; m < M; m++) {
    for (int64_t n = 0; n < N; n++) {
      int64_t acc = 0;
      for (int64_t k = 0; k < K; k++)
        acc += (int64_t)qx[m * K + k] * (int64_t)qw[n * K + k];
      float c = fmul(sx, orc_flush(w_per_row ? s_w[n] : s_w[0]));
      y[m * N + n] = fmul(acc_to_f32(acc), c);
    }
  }
}

void orc_qgemm_bwd_dx(const int8_t* qg, const float* s_g, const int8_t* qw,
                      int64_t M, int64_t N, int64_t K, float* dx) {
  float sg = orc_flush(s_g[0]);
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int64_t m = 0; m < M; m++) {
    int64_t* acc = (int64_t*)calloc((size_t)K, sizeof(int64_t));
    assert(acc);
    for (int64_t n = 0; n < N; n++) {
      int64_t g = qg[m * N + n];
      for (int64_t k = 0; k < K; k++) acc[k] += g * (int64_t)qw[n * K + k];
    }
    for (int64_t k = 0; k < K; k++) dx[m * K + k] = fmul(acc_to_f32(acc[k]), sg);
    free(acc);
  }
}

/* ------------------------------------------------------------------------
 * Walsh-Hadamard rotation along tokens -- §3.2 "int8 computation": a
 * Walsh-Hadamard rotation along the contraction dimension (tokens, for the
 * weight gradient) flattens gradient outliers before int8 quantisation.
 * H_b[i][j] = (-1)^popcount(i & j): Sylvester order, unnormalised; the 1/b
 * of H^T H = b I is folded into the dW dequantisation factor.
 * ---------------------------------------------------------------------- */
static int hadamard(int i, int j) { return (__builtin_popcount((unsigned)(i & j)) & 1) ? -1 : 1; }

void orc_wht_int(const int8_t* qx, int64_t M, int64_t K, int b, int32_t* u) {
  /* u[t][k] = sum_j H_b[t mod b][j] * qx[b*floor(t/b) + j][k], exact. */
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int64_t t = 0; t < M; t++) {
    int64_t base = (t / b) * b;
    int i = (int)(t % b);
    for (int64_t k = 0; k < K; k++) u[t * K + k] = 0;
    for (int j = 0; j < b; j++) {
      int h = hadamard(i, j);
      const int8_t* row = qx + (base + j) * K;
      for (int64_t k = 0; k < K; k++) u[t * K + k] += h * (int32_t)row[k];
    }
  }
}

void orc_wht_int_quant(const int8_t* qx, int64_t M, int64_t K, int b,
                       int8_t* q_u, float* s_u_out, int64_t* S_u_out) {
  int64_t n = M * K;
  int32_t* u = (int32_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(int32_t));
  assert(u);
  orc_wht_int(qx, M, K, b, u);
  int64_t S = 0;
  for (int64_t i = 0; i < n; i++) S += (u[i] < 0) ? -(int64_t)u[i] : (int64_t)u[i];
  /* The exact integer sum (below 2^53) goes through double unchanged, then
   * rounds once to binary32. */
  float Sf = (float)(double)S;
  float s, r;
  orc_lsq_scale(Sf, n, &s, &r);
  for (int64_t i = 0; i < n; i++) q_u[i] = orc_quant1((float)u[i], r);
  *s_u_out = s;
  if (S_u_out) *S_u_out = S;
  free(u);
}

int orc_wht_fp_quant(const void* dy, int dtype, int64_t M, int64_t N, int b,
                     int8_t* q_v, float* s_v, float* v_out) {
  int64_t n = M * N;
  float* v = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
  assert(v);
  for (int64_t i = 0; i < n; i++) v[i] = load(dy, dtype, i);
  /* Per column and aligned block of b tokens, butterflies in stage order
   * h = 1, 2, 4, ..., b/2: (v_j, v_j+h) <- (v_j + v_j+h, v_j - v_j+h). */
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int64_t c = 0; c < N; c++) {
    for (int64_t base = 0; base < M; base += b) {
      for (int h = 1; h < b; h *= 2) {
        for (int j = 0; j < b; j++) {
          if ((j % (2 * h)) >= h) continue;
          float* a = &v[(base + j) * N + c];
          float* d = &v[(base + j + h) * N + c];
          float x0 = *a, x1 = *d;
          *a = fadd(x0, x1);
          *d = fsub(x0, x1);
        }
      }
    }
  }
  float amax;
  int flags = lsq_group(v, n, 0, q_v, s_v, &amax);
  if (v_out) memcpy(v_out, v, (size_t)n * sizeof(float));
  free(v);
  return flags;
}

void orc_dw_gemm(const int8_t* q_v, const int8_t* q_u, int64_t M, int64_t N,
                 int64_t K, float s_x, float s_u, float s_v, int b,
                 int64_t n_lo, int64_t n_hi, float* dw) {
  float inv_b = ldexpf(1.0f, -__builtin_ctz((unsigned)b)); /* exact 1/b */
  float c = fmul(fmul(fmul(orc_flush(s_x), orc_flush(s_u)), orc_flush(s_v)), inv_b);
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int64_t n = n_lo; n < n_hi; n++) {
    int64_t* acc = (int64_t*)calloc((size_t)K, sizeof(int64_t));
    assert(acc);
    for (int64_t m = 0; m < M; m++) {
      int64_t g = q_v[m * N + n];
      if (g == 0) continue;
      const int8_t* row = q_u + m * K;
      for (int64_t k = 0; k < K; k++) acc[k] += g * (int64_t)row[k];
    }
    for (int64_t k = 0; k < K; k++) dw[n * K + k] = fmul(acc_to_f32(acc[k]), c);
    free(acc);
  }
}

int orc_qgemm_bwd_dw_wht(const int8_t* qx, const float* s_x, const void* dy,
                         int dtype, int64_t M, int64_t N, int64_t K, int b,
                         float* dw, float* s_u_out, float* s_v_out) {
  int8_t* q_u = (int8_t*)malloc((size_t)(M * K > 0 ? M * K : 1));
  int8_t* q_v = (int8_t*)malloc((size_t)(M * N > 0 ? M * N : 1));
  assert(q_u && q_v);
  float s_u, s_v;
  orc_wht_int_quant(qx, M, K, b, q_u, &s_u, NULL);
  int flags = orc_wht_fp_quant(dy, dtype, M, N, b, q_v, &s_v, NULL);
  orc_dw_gemm(q_v, q_u, M, N, K, s_x[0], s_u, s_v, b, 0, N, dw);
  if (s_u_out) *s_u_out = s_u;
  if (s_v_out) *s_v_out = s_v;
  free(q_u);
  free(q_v);
  return flags;
}

/* ------------------------------------------------------------------------
 * Input-gradient GEMM with the rotation (a variant) -- §3.2 "int8
 * computation" puts a Walsh-Hadamard rotation along the contraction
 * dimension in front of both straight-through gradient GEMMs.  For
 * dX = dY * W^ (W^ = s_w (.) q_w, per output channel n) the contraction runs
 * over n.  The gradient side g = fl(dY * s_w[n]) (the same product the
 * unrotated path quantises) is rotated in fp32 along n, per row m and
 * aligned block of b; the weight side is rotated exactly in integers along
 * n, per column k, and requantised like the rotated activations.  With
 * H H^T = b I:  dX ~= (1/b) * (g H)(H q_w) * s_g * s_w'.
 * ---------------------------------------------------------------------- */
int orc_wht_fp_rows_quant(const void* dy, int dtype, int64_t M, int64_t N,
                          const float* s_w, int b, int8_t* q, float* s_out,
                          float* v_out) {
  int64_t n = M * N;
  float* v = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
  assert(v);
  for (int64_t i = 0; i < n; i++) {
    float e = load(dy, dtype, i);
    if (s_w) e = fmul(e, orc_flush(s_w[i % N]));
    v[i] = e;
  }
  /* Per row and aligned block of b consecutive n, butterflies in stage
   * order h = 1, 2, 4, ..., b/2: (v_j, v_j+h) <- (v_j + v_j+h, v_j - v_j+h),
   * the token rotation's stages, here along the row. */
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int64_t m = 0; m < M; m++) {
    for (int64_t base = 0; base < N; base += b) {
      float* blk = v + m * N + base;
      for (int h = 1; h < b; h *= 2) {
        for (int j = 0; j < b; j++) {
          if ((j % (2 * h)) >= h) continue;
          float x0 = blk[j], x1 = blk[j + h];
          blk[j] = fadd(x0, x1);
          blk[j + h] = fsub(x0, x1);
        }
      }
    }
  }
  float amax;
  int flags = lsq_group(v, n, 0, q, s_out, &amax);
  if (v_out) memcpy(v_out, v, (size_t)n * sizeof(float));
  free(v);
  return flags;
}

int orc_qgemm_bwd_dx_wht(const void* dy, int dtype, const float* s_w,
                         const int8_t* qw, int64_t M, int64_t N, int64_t K, int b,
                         float* dx, float* s_g_out, float* s_h_out) {
  int8_t* q_g = (int8_t*)malloc((size_t)(M * N > 0 ? M * N : 1));
  int8_t* q_h = (int8_t*)malloc((size_t)(N * K > 0 ? N * K : 1));
  assert(q_g && q_h);
  float s_g, s_h;
  int flags = orc_wht_fp_rows_quant(dy, dtype, M, N, s_w, b, q_g, &s_g, NULL);
  /* q_w [N][K] rotated along its rows n, per column k: the same routine as
   * the activation codes' rotation along tokens */
  orc_wht_int_quant(qw, N, K, b, q_h, &s_h, NULL);
  float inv_b = ldexpf(1.0f, -__builtin_ctz((unsigned)b)); /* exact 1/b */
  float c = fmul(fmul(orc_flush(s_g), orc_flush(s_h)), inv_b);
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int64_t m = 0; m < M; m++) {
    int64_t* acc = (int64_t*)calloc((size_t)K, sizeof(int64_t));
    assert(acc);
    for (int64_t nn = 0; nn < N; nn++) {
      int64_t g = q_g[m * N + nn];
      if (g == 0) continue;
      const int8_t* row = q_h + nn * K;
      for (int64_t k = 0; k < K; k++) acc[k] += g * (int64_t)row[k];
    }
    for (int64_t k = 0; k < K; k++) dx[m * K + k] = fmul(acc_to_f32(acc[k]), c);
    free(acc);
  }
  if (s_g_out) *s_g_out = s_g;
  if (s_h_out) *s_h_out = s_h;
  free(q_g);
  free(q_h);
  return flags;
}

/* ------------------------------------------------------------------------
 * Attention forward with an int8 P.V product (a variant) -- §3.2 "int8
 * computation": inside flash attention the P.V product quantises the
 * attention weights and the values to int8 per block and multiplies on
 * int8 tensor cores, while the QK^T logits and the softmax stay in higher
 * precision.  §3.1 gives the shape: grouped-query attention (query head h
 * reads key/value head h / (Hq / Hkv)), causal, with a sliding window.
 *
 * Every step below is one rounded, flushed binary32 operation, in order:
 *   S_ij = fl(dot_ij * c),  c = fl(1 / fl(sqrt(d))),
 *          dot_ij = fl(... fl(fl(q_0 k_0) + fl(q_1 k_1)) ... + fl(q_d-1 k_d-1))
 *          (sequential over e; bf16 products are exact)
 *   key j is visible from query i iff i - window < j <= i
 *   key blocks of 64, ascending; per row: m = max(m, block max of S)
 *   (order-free), a = exp_f(m_old - m) (0 when m_old = -inf),
 *   p_ij = exp_f(S_ij - m) (0 for a hidden key),
 *   l = fl(fl(l * a) + tree_j p_ij)   (canonical pairwise tree over the 64)
 *   P tile (64 queries x 64 keys): s_p = fl(max p * fl(1/127)),
 *   V block (64 keys x d): s_v = fl(max |v| * fl(1/127)); codes
 *   clamp(rint(fl(x * fl(1/s))), -127, 127) (0 when s = 0);
 *   o_ie = fl(fl(o_ie * a) + fl(fl(sum_j qp_ij qv_je) * fl(s_p * s_v)))
 *   (exact integer sum), and at the end o_ie = fl(o_ie * fl(1 / l)).
 * A row with no visible key in a block leaves m, l, o unchanged.
 * ---------------------------------------------------------------------- */
#define ATT_BLK 64

/* exp for x <= 0: Cody-Waite reduction x = n ln2 + r (ln2 split in a
 * 15-bit head and a tail, so n * head is exact), a degree-7 Taylor
 * polynomial of e^r in Horner form, then the exact scaling by 2^n; each
 * step one rounded, flushed binary32 operation.  -inf and x < -104 give 0. */
float orc_exp_f(float x) {
  if (!(x >= -104.0f)) return 0.0f; /* -inf too */
  const float inv_ln2 = u2f(0x3fb8aa3bu); /* fl(1/ln 2) */
  const float ln2_hi = u2f(0x3f317200u);  /* 0.693145751953125 */
  const float ln2_lo = u2f(0x35bfbe8eu);  /* fl(ln 2 - ln2_hi) */
  float n = rintf(fmul(x, inv_ln2));
  float r = fsub(fsub(x, fmul(n, ln2_hi)), fmul(n, ln2_lo));
  float c[8];
  float fact = 1.0f;
  for (int i = 0; i < 8; i++) {
    if (i > 0) fact = fmul(fact, (float)i); /* i! exact for i <= 7 */
    c[i] = fdiv(1.0f, fact);
  }
  float p = c[7];
  for (int i = 6; i >= 0; i--) p = fadd(fmul(p, r), c[i]);
  int ni = (int)n;
  if (ni < -126) return 0.0f;
  return fmul(p, u2f((uint32_t)(ni + 127) << 23));
}

static float att_quant_scale(float amax, float* r) {
  float s = fmul(amax, fdiv(1.0f, 127.0f));
  *r = (s == 0.0f) ? 0.0f : fdiv(1.0f, s);
  return s;
}

int orc_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t Hq,
                 int64_t Hkv, int64_t T, int64_t d, int64_t window, float* o) {
  if (Hkv <= 0 || Hq % Hkv || T % ATT_BLK) return -1;
  const int64_t group = Hq / Hkv, nb = T / ATT_BLK;
  const float c = fdiv(1.0f, fsqrt((float)d));
  int flags = 0;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic) collapse(2)
#endif
  for (int64_t h = 0; h < Hq; h++) {
    for (int64_t qb = 0; qb < nb; qb++) {
      const int64_t hk = h / group;
      const uint16_t* Q = q + h * T * d;
      const uint16_t* K = k + hk * T * d;
      const uint16_t* V = v + hk * T * d;
      float* O = o + h * T * d;
      float S[ATT_BLK][ATT_BLK], P[ATT_BLK][ATT_BLK], m[ATT_BLK], l[ATT_BLK];
      float* acc = (float*)malloc((size_t)(ATT_BLK * d) * sizeof(float));
      int8_t* qv = (int8_t*)malloc((size_t)(ATT_BLK * d));
      assert(acc && qv);
      for (int i = 0; i < ATT_BLK; i++) { m[i] = -INFINITY; l[i] = 0.0f; }
      for (int64_t x = 0; x < ATT_BLK * d; x++) acc[x] = 0.0f;
      for (int64_t kb = 0; kb <= qb; kb++) {
        /* a block no query of this block sees changes nothing: skipped */
        const int64_t i_lo = qb * ATT_BLK, j_hi = kb * ATT_BLK + ATT_BLK - 1;
        if (j_hi <= i_lo - window) continue;
        int any[ATT_BLK];
        float bmax[ATT_BLK];
        for (int i = 0; i < ATT_BLK; i++) {
          const int64_t gi = qb * ATT_BLK + i;
          any[i] = 0;
          bmax[i] = -INFINITY;
          for (int j = 0; j < ATT_BLK; j++) {
            const int64_t gj = kb * ATT_BLK + j;
            if (gj > gi || gj <= gi - window) { S[i][j] = -INFINITY; continue; }
            float dot = 0.0f;
            for (int64_t e = 0; e < d; e++)
              dot = fadd(dot, fmul(orc_bf16_to_f32(Q[gi * d + e]), orc_bf16_to_f32(K[gj * d + e])));
            S[i][j] = fmul(dot, c);
            any[i] = 1;
            if (S[i][j] > bmax[i]) bmax[i] = S[i][j];
          }
        }
        float alpha[ATT_BLK];
        float pmax = 0.0f;
        for (int i = 0; i < ATT_BLK; i++) {
          if (!any[i]) { alpha[i] = 1.0f; for (int j = 0; j < ATT_BLK; j++) P[i][j] = 0.0f; continue; }
          const float mn = bmax[i] > m[i] ? bmax[i] : m[i];
          alpha[i] = (m[i] == -INFINITY) ? 0.0f : orc_exp_f(fsub(m[i], mn));
          for (int j = 0; j < ATT_BLK; j++) {
            P[i][j] = (S[i][j] == -INFINITY) ? 0.0f : orc_exp_f(fsub(S[i][j], mn));
            if (P[i][j] > pmax) pmax = P[i][j];
          }
          float leaves[ATT_BLK];
          for (int j = 0; j < ATT_BLK; j++) leaves[j] = P[i][j];
          l[i] = fadd(fmul(l[i], alpha[i]), tree_inplace(leaves, ATT_BLK));
          m[i] = mn;
        }
        /* the P tile's and the V block's int8 codes */
        float rp, rv, vmax = 0.0f;
        const float sp = att_quant_scale(pmax, &rp);
        for (int j = 0; j < ATT_BLK; j++)
          for (int64_t e = 0; e < d; e++) {
            const float a = fabs_(orc_bf16_to_f32(V[(kb * ATT_BLK + j) * d + e]));
            if (a > vmax) vmax = a;
          }
        const float sv = att_quant_scale(vmax, &rv);
        for (int j = 0; j < ATT_BLK; j++)
          for (int64_t e = 0; e < d; e++)
            qv[j * d + e] = orc_quant1(orc_bf16_to_f32(V[(kb * ATT_BLK + j) * d + e]), rv);
        const float cs = fmul(sp, sv);
        for (int i = 0; i < ATT_BLK; i++) {
          if (!any[i]) continue;
          int8_t qp[ATT_BLK];
          for (int j = 0; j < ATT_BLK; j++) qp[j] = orc_quant1(P[i][j], rp);
          for (int64_t e = 0; e < d; e++) {
            int32_t s32 = 0;
            for (int j = 0; j < ATT_BLK; j++) s32 += (int32_t)qp[j] * (int32_t)qv[j * d + e];
            const float contrib = fmul((float)s32, cs);
            acc[i * d + e] = fadd(fmul(acc[i * d + e], alpha[i]), contrib);
          }
        }
      }
      for (int i = 0; i < ATT_BLK; i++) {
        const float il = fdiv(1.0f, l[i]);
        for (int64_t e = 0; e < d; e++) O[(qb * ATT_BLK + i) * d + e] = fmul(acc[i * d + e], il);
        if (!isfinite(l[i])) flags |= ORC_FLAG_NONFINITE;
      }
      free(acc);
      free(qv);
    }
  }
  return flags;
}

/* ------------------------------------------------------------------------
 * RMSNorm -- §3.1 "RMSNorm" (pre-norm, no bias) and the precision note
 * (normalisation in FP32, parameters BF16): y = x * rsqrt(mean(x^2)+eps)*g
 * with a correctly rounded sqrt followed by a reciprocal.
 * ---------------------------------------------------------------------- */
int orc_rmsnorm_fwd(const void* x, const void* g, int dtype, int64_t T,
                    int64_t D, float eps, void* y, float* rstd) {
  float* xs = (float*)malloc((size_t)D * sizeof(float));
  float* sq = (float*)malloc((size_t)D * sizeof(float));
  assert(xs && sq);
  float invD = inv_count(D);
  float e = orc_flush(eps);
  int flags = 0;
  for (int64_t t = 0; t < T; t++) {
    for (int64_t j = 0; j < D; j++) {
      xs[j] = load(x, dtype, t * D + j);
      sq[j] = fmul(xs[j], xs[j]);
    }
    float ss = tree_inplace(sq, D);
    if (!isfinite(ss)) flags |= ORC_FLAG_NONFINITE;
    float ms = fmul(ss, invD);
    float r = fdiv(1.0f, fsqrt(fadd(ms, e)));
    rstd[t] = r;
    for (int64_t j = 0; j < D; j++)
      store(y, dtype, t * D + j, fmul(fmul(xs[j], r), load(g, dtype, j)));
  }
  free(xs);
  free(sq);
  return flags;
}

/* Backward per row: xh = x*rstd, d = dy*g, dot = tree(d*xh), mu = dot/D,
 * dx = rstd*(d - xh*mu).  dg[j] = tree over tokens of dy*xh. */
void orc_rmsnorm_bwd(const void* x, const void* g, const float* rstd,
                     const void* dy, int dtype, int64_t T, int64_t D,
                     void* dx, float* dg) {
  float invD = inv_count(D);
  float* xh = (float*)malloc((size_t)D * sizeof(float));
  float* d = (float*)malloc((size_t)D * sizeof(float));
  float* p = (float*)malloc((size_t)D * sizeof(float));
  float* col = (float*)malloc((size_t)(T > 0 ? T : 1) * sizeof(float));
  assert(xh && d && p && col);
  for (int64_t t = 0; t < T; t++) {
    float r = orc_flush(rstd[t]);
    for (int64_t j = 0; j < D; j++) {
      xh[j] = fmul(load(x, dtype, t * D + j), r);
      d[j] = fmul(load(dy, dtype, t * D + j), load(g, dtype, j));
      p[j] = fmul(d[j], xh[j]);
    }
    float dot = tree_inplace(p, D);
    float mu = fmul(dot, invD);
    for (int64_t j = 0; j < D; j++)
      store(dx, dtype, t * D + j, fmul(r, fsub(d[j], fmul(xh[j], mu))));
  }
  for (int64_t j = 0; j < D; j++) {
    for (int64_t t = 0; t < T; t++) {
      float xhat = fmul(load(x, dtype, t * D + j), orc_flush(rstd[t]));
      col[t] = fmul(load(dy, dtype, t * D + j), xhat);
    }
    dg[j] = tree_inplace(col, T);
  }
  free(xh);
  free(d);
  free(p);
  free(col);
}

/* ------------------------------------------------------------------------
 * Global gradient norm -- §3.2 "Optimizer" (global l2 clipping) with FP32
 * gradient reduction: ss = tree(v*v), norm = sqrt(ss).
 * ---------------------------------------------------------------------- */
int orc_grad_norm(const float* v, int64_t n, float* sumsq, float* norm) {
  float* sq = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
  assert(sq);
  for (int64_t i = 0; i < n; i++) {
    float e = orc_flush(v[i]);
    sq[i] = fmul(e, e);
  }
  float ss = tree_inplace(sq, n);
  free(sq);
  *sumsq = ss;
  *norm = fsqrt(ss);
  return isfinite(ss) ? 0 : ORC_FLAG_NONFINITE;
}

/* ------------------------------------------------------------------------
 * Optimizer step -- §3.2 "Optimizer" (AdamW with beta1 0.9, beta2 0.95,
 * eps 1e-8 through a reproducible fused kernel; decoupled weight decay 0.1
 * on the linear layers and the LM head, none on normalisation weights;
 * gradients clipped to a global l2 norm of 1.0), §3.2 "Optimizer-state
 * precision" (BF16 parameters, FP32 moments: widen parameter and gradient,
 * update in FP32, round to BF16 once per step), §3.4.2 "Gradient behavior,
 * Clipping, and Spike Protocol" (five optimizer steps skipped when the
 * pre-clip norm exceeds 5).
 *
 * The pages name the algorithm, not its operation order; this is the
 * decoupled form of AdamW written out one rounded operation at a time:
 *   m = b1*m + (1-b1)*g              v = b2*v + (1-b2)*(g*g)
 *   mh = m / bc1    vh = v / bc2     u = mh / (sqrt(vh) + eps)
 *   p = p - lr*(u + wd*p)
 * with bc = 1 - beta^t, beta^t the t-fold product of rounded multiplies.
 * ---------------------------------------------------------------------- */
void orc_adamw_bias_corrections(int64_t t, float beta1, float beta2, float* bc1,
                                float* bc2) {
  float p1 = 1.0f, p2 = 1.0f;
  for (int64_t i = 0; i < t; i++) {
    p1 = fmul(p1, beta1);
    p2 = fmul(p2, beta2);
  }
  *bc1 = fsub(1.0f, p1);
  *bc2 = fsub(1.0f, p2);
}

/* One step's control from the pre-clip global norm.  A norm above
 * spike_threshold, or not finite, (re)starts a window of skip_steps skipped
 * optimizer steps, this one first; inside a window nothing is applied.
 * Otherwise a norm above max_norm scales the gradient by max_norm / norm,
 * and a smaller one leaves it as it is. */
int orc_adamw_decide(float norm, float max_norm, float spike_threshold,
                     int skip_steps, int32_t* skip_state, float* apply,
                     float* clip) {
  norm = orc_flush(norm);
  const int finite = isfinite(norm);
  if (!finite || norm > spike_threshold) *skip_state = skip_steps;
  if (*skip_state > 0) {
    *skip_state -= 1;
    *apply = 0.0f;
    *clip = 0.0f;
  } else {
    *apply = 1.0f;
    *clip = norm > max_norm ? fdiv(orc_flush(max_norm), norm) : 1.0f;
  }
  return finite ? 0 : ORC_FLAG_NONFINITE;
}

void orc_adamw_step(void* param, int pdtype, const void* grad, int gdtype,
                    float* m, float* v, int64_t n, float lr, float beta1,
                    float beta2, float eps, float wd, float bc1, float bc2,
                    float apply, float clip) {
  if (apply == 0.0f) return;
  const float omb1 = fsub(1.0f, beta1), omb2 = fsub(1.0f, beta2);
  for (int64_t i = 0; i < n; i++) {
    float g = load(grad, gdtype, i);
    if (clip != 1.0f) g = fmul(g, clip);
    const float p = load(param, pdtype, i);
    const float mi = fadd(fmul(beta1, orc_flush(m[i])), fmul(omb1, g));
    const float vi = fadd(fmul(beta2, orc_flush(v[i])), fmul(omb2, fmul(g, g)));
    const float mh = fdiv(mi, bc1);
    const float vh = fdiv(vi, bc2);
    const float u = fdiv(mh, fadd(fsqrt(vh), eps));
    const float pn = fsub(p, fmul(lr, fadd(u, fmul(wd, p))));
    m[i] = mi;
    v[i] = vi;
    store(param, pdtype, i, pn);
  }
}

/* ------------------------------------------------------------------------
 * Deterministic data-parallel gradient exchange -- App. A "Deterministic
 * Gradient Reduction".  The gradient of one step is reduced at three
 * levels: microbatches on one rank, the shards of a node (intra-node
 * reduce-scatter), and the replicas (inter-node all-reduce).  Every step is
 * elementwise, so the reduction of element i depends only on the values at
 * index i of the contributions; the routines below take each element
 * through the definition on its own.
 *
 *   App. A.2: the contributions of shards 0 .. S-1 are added into a
 *     running sum in ascending rank order (the inner accumulator); the
 *     microbatch accumulation on a rank is the same running sum over its
 *     microbatches in order.
 *   App. A.3: every average (by the microbatch count, by dp_shard, by
 *     dp_replicate) is a multiply by the binary32 reciprocal fl(1/k), never
 *     a division.
 *   App. A "Deterministic Gradient Reduction": the inner sum is finalised
 *     and averaged once per replica (every dp_shard virtual ranks), and the
 *     averaged replica partials go to TreeFold.
 *   App. A.1: TreeFold pushes each replica partial once onto a stack of
 *     (level, partial) entries; an incoming entry merges with the top while
 *     the two have the same level, the lower replica (the stack entry) on
 *     the left, and the merged entry moves one level up, as in binary
 *     counting.  Result combines the entries left on the stack (one per set
 *     bit of the replica count) in ascending level order: the entry of the
 *     lowest level (the smallest, highest-numbered block) first, each time
 *     with the lower-replica block on the left.  (The page's parenthesis
 *     also calls the lowest level the largest block; the level of an entry
 *     as Push defines it grows with the block, and §5 describes the cluster
 *     combining the largest power-of-two block with the remainder, so the
 *     smallest block is taken first.)
 * ---------------------------------------------------------------------- */
#define ORC_FOLD_MAX 64

/* One element of the running sum over count contributions in ascending
 * order: acc = c_0, then acc = fl(acc + c_j). */
static float ascending_sum1(const float* const* parts, int count, int64_t i) {
  float acc = orc_flush(parts[0][i]);
  for (int j = 1; j < count; j++) acc = fadd(acc, orc_flush(parts[j][i]));
  return acc;
}

void orc_ascending_sum(const float* const* parts, int count, int64_t n, float* out) {
  if (count < 1 || n <= 0) return;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = ascending_sum1(parts, count, i);
}

void orc_average(const float* x, int64_t n, int64_t k, float* out) {
  const float inv = inv_count(k);
  for (int64_t i = 0; i < n; i++) out[i] = fmul(orc_flush(x[i]), inv);
}

/* TreeFold over the values v[0..R) of one element (replica order). */
typedef struct {
  int level;
  float val;
} fold_entry;

static void fold_push(fold_entry* stack, int* depth, float v) {
  fold_entry e = {0, v};
  while (*depth > 0 && stack[*depth - 1].level == e.level) {
    e.val = fadd(stack[*depth - 1].val, e.val);  /* lower replica on the left */
    e.level += 1;
    *depth -= 1;
  }
  stack[(*depth)++] = e;
}

static float fold_result(const fold_entry* stack, int depth) {
  /* the top of the stack holds the lowest level */
  float acc = stack[depth - 1].val;
  for (int k = depth - 2; k >= 0; k--) acc = fadd(stack[k].val, acc);
  return acc;
}

static float treefold1(const float* v, int R) {
  fold_entry stack[ORC_FOLD_MAX];
  int depth = 0;
  for (int r = 0; r < R; r++) fold_push(stack, &depth, v[r]);
  return fold_result(stack, depth);
}

void orc_treefold(const float* const* parts, int R, int64_t n, float* out) {
  if (R < 1 || R > ORC_FOLD_MAX || n <= 0) return;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) {
    float v[ORC_FOLD_MAX];
    for (int r = 0; r < R; r++) v[r] = orc_flush(parts[r][i]);
    out[i] = treefold1(v, R);
  }
}

/* The whole exchange of one step, as a single device would replay it.
 * parts: R*S*A contributions in mesh order (replica-major, then shard,
 * then microbatch), each [n] fp32.  With average != 0 each level
 * multiplies by the reciprocal of its count (App. A.3). */
int orc_dp_reduce(const float* const* parts, int R, int S, int A, int64_t n,
                  int average, float* out) {
  if (R < 1 || S < 1 || A < 1 || R * S * A > ORC_FOLD_MAX || n < 0) return -1;
  const float inv_a = inv_count(A), inv_s = inv_count(S), inv_r = inv_count(R);
  int flags = 0;
#pragma omp parallel for schedule(static) reduction(| : flags)
  for (int64_t i = 0; i < n; i++) {
    float rep[ORC_FOLD_MAX];
    for (int r = 0; r < R; r++) {
      float inner = 0.0f;
      for (int s = 0; s < S; s++) {
        float g = ascending_sum1(parts + (size_t)(r * S + s) * A, A, i);
        if (average) g = fmul(g, inv_a);
        inner = s == 0 ? g : fadd(inner, g);
      }
      if (average) inner = fmul(inner, inv_s);
      rep[r] = inner;
    }
    float res = treefold1(rep, R);
    if (average) res = fmul(res, inv_r);
    out[i] = res;
    if (!isfinite(res)) flags |= ORC_FLAG_NONFINITE;
  }
  return flags;
}

/* ------------------------------------------------------------------------
 * SHA-256, FIPS 180-4 §6.2, and the canonical state hash (§5 "Runtime
 * overhead" and App. B: a canonical per-step hash of the training state;
 * computed here over raw little-endian tensor bytes in a Merkle tree).
 * ---------------------------------------------------------------------- */
static const uint32_t SHA_K[64] = {
    0x428a2f98, 0x71374491, 0xb5c0fbcf, 0xe9b5dba5, 0x3956c25b, 0x59f111f1,
    0x923f82a4, 0xab1c5ed5, 0xd807aa98, 0x12835b01, 0x243185be, 0x550c7dc3,
    0x72be5d74, 0x80deb1fe, 0x9bdc06a7, 0xc19bf174, 0xe49b69c1, 0xefbe4786,
    0x0fc19dc6, 0x240ca1cc, 0x2de92c6f, 0x4a7484aa, 0x5cb0a9dc, 0x76f988da,
    0x983e5152, 0xa831c66d, 0xb00327c8, 0xbf597fc7, 0xc6e00bf3, 0xd5a79147,
    0x06ca6351, 0x14292967, 0x27b70a85, 0x2e1b2138, 0x4d2c6dfc, 0x53380d13,
    0x650a7354, 0x766a0abb, 0x81c2c92e, 0x92722c85, 0xa2bfe8a1, 0xa81a664b,
    0xc24b8b70, 0xc76c51a3, 0xd192e819, 0xd6990624, 0xf40e3585, 0x106aa070,
    0x19a4c116, 0x1e376c08, 0x2748774c, 0x34b0bcb5, 0x391c0cb3, 0x4ed8aa4a,
    0x5b9cca4f, 0x682e6ff3, 0x748f82ee, 0x78a5636f, 0x84c87814, 0x8cc70208,
    0x90befffa, 0xa4506ceb, 0xbef9a3f7, 0xc67178f2};

static uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

static void sha_block(uint32_t H[8], const uint8_t blk[64]) {
  uint32_t W[64];
  for (int t = 0; t < 16; t++)
    W[t] = ((uint32_t)blk[4 * t] << 24) | ((uint32_t)blk[4 * t + 1] << 16) |
           ((uint32_t)blk[4 * t + 2] << 8) | (uint32_t)blk[4 * t + 3];
  for (int t = 16; t < 64; t++) {
    uint32_t s0 = rotr(W[t - 15], 7) ^ rotr(W[t - 15], 18) ^ (W[t - 15] >> 3);
    uint32_t s1 = rotr(W[t - 2], 17) ^ rotr(W[t - 2], 19) ^ (W[t - 2] >> 10);
    W[t] = W[t - 16] + s0 + W[t - 7] + s1;
  }
  uint32_t a = H[0], b = H[1], c = H[2], d = H[3], e = H[4], f = H[5], g = H[6], h = H[7];
  for (int t = 0; t < 64; t++) {
    uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
    uint32_t ch = (e & f) ^ (~e & g);
    uint32_t T1 = h + S1 + ch + SHA_K[t] + W[t];
    uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
    uint32_t maj = (a & b) ^ (a & c) ^ (b & c);
    uint32_t T2 = S0 + maj;
    h = g; g = f; f = e; e = d + T1; d = c; c = b; b = a; a = T1 + T2;
  }
  H[0] += a; H[1] += b; H[2] += c; H[3] += d;
  H[4] += e; H[5] += f; H[6] += g; H[7] += h;
}

void orc_sha256(const uint8_t* msg, uint64_t len, uint8_t out[32]) {
  uint32_t H[8] = {0x6a09e667, 0xbb67ae85, 0x3c6ef372, 0xa54ff53a,
                   0x510e527f, 0x9b05688c, 0x1f83d9ab, 0x5be0cd19};
  uint64_t full = len / 64;
  for (uint64_t i = 0; i < full; i++) sha_block(H, msg + 64 * i);
  uint8_t tail[128];
  uint64_t rem = len - 64 * full;
  memset(tail, 0, sizeof tail);
  if (rem) memcpy(tail, msg + 64 * full, (size_t)rem);
  tail[rem] = 0x80;
  uint64_t tl = (rem + 1 + 8 <= 64) ? 64 : 128;
  uint64_t bits = len * 8;
  for (int i = 0; i < 8; i++) tail[tl - 1 - i] = (uint8_t)(bits >> (8 * i));
  sha_block(H, tail);
  if (tl == 128) sha_block(H, tail + 64);
  for (int i = 0; i < 8; i++) {
    out[4 * i] = (uint8_t)(H[i] >> 24);
    out[4 * i + 1] = (uint8_t)(H[i] >> 16);
    out[4 * i + 2] = (uint8_t)(H[i] >> 8);
    out[4 * i + 3] = (uint8_t)H[i];
  }
}

void orc_merkle_root(const uint8_t* bytes, uint64_t nbytes, uint8_t out[32]) {
  const uint64_t LEAF = 4096, FAN = 128;
  uint64_t cnt = nbytes == 0 ? 1 : (nbytes + LEAF - 1) / LEAF;
  uint8_t* d = (uint8_t*)malloc((size_t)cnt * 32);
  assert(d);
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int64_t i = 0; i < (int64_t)cnt; i++) {
    uint64_t off = (uint64_t)i * LEAF;
    uint64_t len = nbytes - off < LEAF ? nbytes - off : LEAF;
    orc_sha256(bytes + off, nbytes == 0 ? 0 : len, d + 32 * i);
  }
  while (cnt > 1) {
    uint64_t nc = (cnt + FAN - 1) / FAN;
    for (uint64_t j = 0; j < nc; j++) {
      uint64_t k = cnt - FAN * j < FAN ? cnt - FAN * j : FAN;
      uint8_t tmp[32];
      orc_sha256(d + 32 * FAN * j, 32 * k, tmp);
      memcpy(d + 32 * j, tmp, 32); /* j <= FAN*j, so the source is read first */
    }
    cnt = nc;
  }
  memcpy(out, d, 32);
  free(d);
}

void orc_tensor_digest(const uint8_t* bytes, uint64_t nbytes, int dtype,
                       int ndim, const int64_t* dims, const char* name,
                       uint8_t out[32]) {
  uint8_t root[32];
  orc_merkle_root(bytes, nbytes, root);
  size_t nl = strlen(name);
  size_t hl = 4 + 1 + 1 + 8 * (size_t)ndim + 2 + nl + 32;
  uint8_t* h = (uint8_t*)malloc(hl);
  assert(h);
  size_t o = 0;
  memcpy(h, "BRQ1", 4); o = 4;
  h[o++] = (uint8_t)dtype;
  h[o++] = (uint8_t)ndim;
  for (int i = 0; i < ndim; i++)
    for (int b = 0; b < 8; b++) h[o++] = (uint8_t)((uint64_t)dims[i] >> (8 * b));
  h[o++] = (uint8_t)(nl & 0xff);
  h[o++] = (uint8_t)(nl >> 8);
  memcpy(h + o, name, nl); o += nl;
  memcpy(h + o, root, 32); o += 32;
  orc_sha256(h, o, out);
  free(h);
}

void orc_hash_state(int n, const uint8_t* const* ptrs, const uint64_t* nbytes,
                    const int* dtypes, const int* ndims, const int64_t* dims,
                    const char* const* names, uint8_t out[32]) {
  uint8_t* cat = (uint8_t*)malloc((size_t)(n > 0 ? n : 1) * 32);
  assert(cat);
  const int64_t* dp = dims;
  for (int i = 0; i < n; i++) {
    orc_tensor_digest(ptrs[i], nbytes[i], dtypes[i], ndims[i], dp, names[i], cat + 32 * i);
    dp += ndims[i];
  }
  orc_sha256(cat, 32 * (uint64_t)n, out);
  free(cat);
}
