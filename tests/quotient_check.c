/* Checks the quotient used by the FP8 quantise-and-append kernel.
 *
 * The kernel turns a bfloat16 value x and a positive descale d into an E4M3
 * code of fp32(x / d) (round to nearest even, saturating at 448).  For
 * descales in [2^-80, 2^100] it does not divide per value: with r = 1/d
 * correctly rounded,
 *     q0 = clamp(RN(x * r), -1024, 1024)
 *     q  = fma(fma(-q0, d, x), r, q0)        (Markstein's correction)
 *     y  = clamp(copysign(q, x), -448, 448)
 * This program repeats that arithmetic in C (fmaf is correctly rounded) and
 * compares the E4M3 code of y with the code of the IEEE quotient x / d.
 *
 *   full   every computed descale d = fp32(amax / 448), amax a positive
 *          finite bfloat16, with every bfloat16 x of |x| <= amax; then 20000
 *          seeded descales in [2^-125, 2^125] with every finite bfloat16 x
 *          (about 2.4e9 pairs, minutes)
 *   quick  every 97th amax and 300 seeded descales (seconds)
 *
 * Exit status 0 when every code matches.  Compile with -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bf16(uint32_t h) {
  uint32_t u = h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static float clampf(float v, float lim) { return fmaxf(fminf(v, lim), -lim); }

/* OCP E4M3 code of v, |v| <= 448, round to nearest even. */
static int e4m3(float v) {
  const int s = signbit(v) ? 0x80 : 0;
  const float a = fabsf(v);
  if (a < 0x1p-6f) return s | (int)nearbyintf(a * 512.0f); /* subnormals (8 = 2^-6) */
  int e;
  const float f = frexpf(a, &e); /* a = f * 2^e, f in [0.5, 1) */
  float m = nearbyintf((2.0f * f - 1.0f) * 8.0f);
  int be = e - 1 + 7;
  if (m == 8.0f) {
    m = 0.0f;
    ++be;
  }
  return s | (be << 3) | (int)m;
}

static long long checked = 0, bad = 0;

static void check(float x, float d, float r) {
  const int want = e4m3(clampf(x / d, 448.0f));
  float y;
  if (d >= 0x1p-80f && d <= 0x1p100f) {
    const float q0 = clampf(x * r, 1024.0f);
    const float q = fmaf(fmaf(-q0, d, x), r, q0);
    y = clampf(copysignf(q, x), 448.0f);
  } else {
    y = clampf(x / d, 448.0f);
  }
  const int got = e4m3(y);
  ++checked;
  if (got != want) {
    if (bad < 10) printf("mismatch: x=%a d=%a want %02x got %02x\n", x, d, want, got);
    ++bad;
  }
}

int main(int argc, char** argv) {
  const int full = argc > 1 && strcmp(argv[1], "full") == 0;
  /* encoder sanity: 448 -> 7e, 1 -> 38, 2^-9 -> 01, 2^-10 -> 00 (tie to even), 240 -> 77, -0 -> 80 */
  if (e4m3(448.0f) != 0x7e || e4m3(1.0f) != 0x38 || e4m3(0x1p-9f) != 0x01 || e4m3(0x1p-10f) != 0x00 ||
      e4m3(0x1.8p-10f) != 0x01 || e4m3(240.0f) != 0x77 || e4m3(232.0f) != 0x76 || e4m3(-0.0f) != 0x80) {
    printf("E4M3 encoder self-check failed\n");
    return 2;
  }
  const uint32_t amax_step = full ? 1 : 97;
  for (uint32_t a = 1; a < 0x7f80; a += amax_step) {
    volatile float dv = bf16(a) / 448.0f;
    const float d = dv;
    volatile float rv = 1.0f / d;
    const float r = rv;
    for (uint32_t h = 0; h <= a; ++h) {
      check(bf16(h), d, r);
      check(-bf16(h), d, r);
    }
  }
  const long long computed = checked;
  srand(12345);
  const int ndesc = full ? 20000 : 300;
  for (int i = 0; i < ndesc; ++i) {
    const int e = rand() % 250 - 125;
    uint32_t m = (((uint32_t)rand() << 8) ^ (uint32_t)rand()) & 0x7fffffu;
    if (i < 32) m = 0x7fffffu - (uint32_t)i; /* significands of all ones */
    else if (i < 64) m = (uint32_t)(i - 32); /* near powers of two */
    const uint32_t u = ((uint32_t)(e + 127) << 23) | m;
    float d;
    memcpy(&d, &u, 4);
    volatile float rv = 1.0f / d;
    const float r = rv;
    for (uint32_t h = 0; h < 0x7f80; ++h) {
      check(bf16(h), d, r);
      check(-bf16(h), d, r);
    }
  }
  printf("%s: %lld pairs with computed descales, %lld with seeded descales, %lld mismatches\n",
         full ? "full" : "quick", computed, checked - computed, bad);
  return bad != 0;
}
