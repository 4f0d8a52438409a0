/* Exhaustive CPU check behind the attention softmax's unflushed exp: for
 * every binary32 x in [-104, 0] with x = 0 or |x| >= 2^-100, the Cody-Waite
 * reduction and Horner polynomial evaluated without flushes produce no
 * subnormal value, so they equal the flushed evaluation bit for bit.
 * Prints the number of violations (0 expected) and the smallest nonzero
 * |r| seen.  Test infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static int sub(float v) { return v != 0.0f && fabsf(v) < 0x1p-126f; }

int main(void) {
  const float inv_ln2 = u2f(0x3fb8aa3bu), hi = u2f(0x3f317200u), lo = u2f(0x35bfbe8eu);
  float c[8];
  float fact = 1.0f;
  for (int i = 0; i < 8; i++) {
    if (i > 0) fact = fact * (float)i;
    c[i] = 1.0f / fact;
  }
  long bad = 0;
  float rmin = INFINITY;
  /* negative floats from -2^-100 down to -104: bit patterns increase */
  const uint32_t first = 0x80000000u | 0x0d800000u; /* -2^-100 */
  const uint32_t last = 0xc2d00000u;                /* -104 */
#pragma omp parallel for reduction(+ : bad) reduction(min : rmin) schedule(static)
  for (int64_t b = first; b <= (int64_t)last; b++) {
    const volatile float x = u2f((uint32_t)b);
    const float t = x * inv_ln2;
    const float n = rintf(t);
    const float a = n * hi, e = n * lo, r1 = x - a, r = r1 - e;
    int s = sub(t) || sub(a) || sub(e) || sub(r1) || sub(r);
    if (r != 0.0f && fabsf(r) < rmin) rmin = fabsf(r);
    float p = c[7];
    for (int i = 6; i >= 0; i--) {
      const float pr = p * r;
      p = pr + c[i];
      s = s || sub(pr) || sub(p);
    }
    bad += s;
  }
  printf("%ld %a\n", bad, rmin);
  return 0;
}
