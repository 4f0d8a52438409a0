/*
 * philox.c -- seeded, counter-based synthetic input generator.
 *
 * This module only makes input tensors.  It holds none of the quantiser,
 * GEMM, rotation, normalisation or hash arithmetic; both the CPU oracle and
 * the GPU path consume the tensors it writes.
 *
 * Generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11).  Element i of a tensor is a pure
 * function of (seed, tag, i): the counter is (i_lo, i_hi, lane, 0) and the
 * key is (seed, tag), following the counter-based stream of the Open-1B
 * report (§2.1 "Random number generation").  Values never depend on the
 * thread count.
 *
 * Normals: Box-Muller in double from two 53-bit uniforms in (0, 1), then one
 * rounding to binary32 (and, for BF16 tensors, one more round-to-nearest-
 * even to bfloat16).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static void mulhilo(uint32_t a, uint32_t b, uint32_t* hi, uint32_t* lo) {
  uint64_t p = (uint64_t)a * (uint64_t)b;
  *hi = (uint32_t)(p >> 32);
  *lo = (uint32_t)p;
}

void syn_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int r = 0; r < 10; r++) {
    uint32_t hi0, lo0, hi1, lo1;
    mulhilo(PHILOX_M0, c0, &hi0, &lo0);
    mulhilo(PHILOX_M1, c2, &hi1, &lo1);
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += PHILOX_W0;
    k1 += PHILOX_W1;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static void draw(uint32_t seed, uint32_t tag, uint64_t i, uint32_t lane, uint32_t w[4]) {
  uint32_t ctr[4] = {(uint32_t)i, (uint32_t)(i >> 32), lane, 0};
  uint32_t key[2] = {seed, tag};
  syn_philox4x32_10(ctr, key, w);
}

/* 53-bit uniform strictly inside (0, 1). */
static double unif53(uint32_t a, uint32_t b) {
  uint64_t m = ((uint64_t)(a >> 5) << 26) | (uint64_t)(b >> 6);
  return ((double)m + 0.5) * 0x1p-53;
}

static double normal_from(const uint32_t w[4]) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = unif53(w[0], w[1]);
  double u2 = unif53(w[2], w[3]);
  return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static void put(void* out, int bf16, int64_t i, double v) {
  float f = (float)v;
  if (bf16) ((uint16_t*)out)[i] = to_bf16(f);
  else ((float*)out)[i] = f;
}

/* out[i] = mean + std * N(0,1)_i for i in [0, n). */
void syn_normal(uint32_t seed, uint32_t tag, int64_t n, double mean, double std,
                int bf16, void* out) {
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int64_t i = 0; i < n; i++) {
    uint32_t w[4];
    draw(seed, tag, (uint64_t)i, 0, w);
    put(out, bf16, i, mean + std * normal_from(w));
  }
}

/* out[i] = scale * t_3, a Student-t variate with 3 degrees of freedom built
 * as Z0 / sqrt((Z1^2 + Z2^2 + Z3^2) / 3) from four independent normals. */
void syn_student_t3(uint32_t seed, uint32_t tag, int64_t n, double scale, int bf16,
                    void* out) {
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int64_t i = 0; i < n; i++) {
    uint32_t w[4];
    double z[4];
    for (uint32_t l = 0; l < 4; l++) {
      draw(seed, tag, (uint64_t)i, l, w);
      z[l] = normal_from(w);
    }
    double chi = (z[1] * z[1] + z[2] * z[2] + z[3] * z[3]) / 3.0;
    put(out, bf16, i, scale * z[0] / sqrt(chi));
  }
}

/* Pick `count` distinct indices in [0, range) for a tensor tag: candidate j
 * is philox((j, 0, 7, 0), (seed, tag))[0] mod range; duplicates skipped. */
void syn_pick_distinct(uint32_t seed, uint32_t tag, int64_t range, int count,
                       int64_t* out) {
  int got = 0;
  for (uint64_t j = 0; got < count; j++) {
    uint32_t w[4];
    draw(seed, tag, j, 7, w);
    int64_t c = (int64_t)(((uint64_t)w[0] | ((uint64_t)w[1] << 32)) % (uint64_t)range);
    int dup = 0;
    for (int q = 0; q < got; q++) dup |= (out[q] == c);
    if (!dup) out[got++] = c;
  }
}

/* Multiply the listed columns of a row-major [rows][cols] tensor by `mul`. */
void syn_scale_columns(void* data, int bf16, int64_t rows, int64_t cols,
                       const int64_t* which, int count, double mul) {
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int64_t r = 0; r < rows; r++) {
    for (int q = 0; q < count; q++) {
      int64_t i = r * cols + which[q];
      if (bf16) {
        uint32_t u = (uint32_t)((uint16_t*)data)[i] << 16;
        float f;
        memcpy(&f, &u, 4);
        ((uint16_t*)data)[i] = to_bf16((float)(f * mul));
      } else {
        float* p = (float*)data + i;
        *p = (float)(*p * mul);
      }
    }
  }
}

/* Replace about one element in `every` of a BF16 tensor by a bfloat16
 * subnormal (random sign, mantissa 1..127): element i is replaced when
 * philox((i, 0, 5, 0), (seed, tag))[0] mod every == 0. */
void syn_bf16_subnormals(uint32_t seed, uint32_t tag, int64_t n, uint32_t every,
                         uint16_t* data) {
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int64_t i = 0; i < n; i++) {
    uint32_t w[4];
    draw(seed, tag, (uint64_t)i, 5, w);
    if (w[0] % every) continue;
    uint16_t mant = (uint16_t)(1 + (w[1] % 127u));
    uint16_t sign = (uint16_t)((w[2] & 1u) << 15);
    data[i] = (uint16_t)(sign | mant);
  }
}

int syn_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
