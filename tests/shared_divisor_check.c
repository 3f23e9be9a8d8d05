/* CPU check of the division the GPU quantizers use for the 32 codes of a
 * block: with y = RN(1/b), q0 = RN(a*y), r = RN(a - q0*b) (one fma) and
 * q = RN(q0 + r*y) (one fma), the rounded code round(q), clamped to the
 * format's range, must equal round(RN(a/b)) clamped the same way.
 * Divisors b: every positive finite fp16 value (Q4_0 / Q8_0 scales) and
 * fp16 values times 1..127 (Q4_K-style sub-block scales, 1..63, and
 * Q6_K-style ones, 1..127). Numerators a:
 * quotients spread over the code ranges, the neighbourhood (a few ulps) of
 * every half-integer quotient, and random bit patterns.
 * Usage: shared_divisor_check N_SAMPLES SEED; prints "ok" or the first
 * mismatches and exits nonzero. Built with -ffp-contract=off so that a*y and
 * a/b are single roundings; fmaf is the C library's correctly rounded fma. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t st;
static uint64_t next(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }

static float half_to_float(uint16_t h) {
  int e = (h >> 10) & 31, m = h & 1023;
  float v = e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(m | 1024), e - 25);
  return (h & 0x8000) ? -v : v;
}

static float code(float q, float lo, float hi) { return fminf(fmaxf(roundf(q), lo), hi); }

int main(int argc, char **argv) {
  long long n = argc > 1 ? atoll(argv[1]) : 10000000;
  st = argc > 2 ? strtoull(argv[2], 0, 10) * 2654435761ull + 1 : 1;
  long long bad = 0, checked = 0;
  for (long long it = 0; it < n; ++it) {
    float b = half_to_float((uint16_t)(1 + next() % 0x7BFF));  /* positive finite fp16 */
    int q4k = it & 1;
    if (q4k) b *= (float)(1 + next() % 127);
    float a;
    switch ((it >> 1) % 3) {
      case 0:
        a = b * (float)((int64_t)(next() % 270001) - 135000) / 1000.0f;
        break;
      case 1: {
        float t = (float)((int)(next() % 271) - 135) + 0.5f;
        a = t * b;
        for (int k = (int)(next() % 5); k > 0; --k) a = nextafterf(a, (next() & 1) ? INFINITY : -INFINITY);
        break;
      }
      default: {
        uint32_t bits = (uint32_t)next();
        memcpy(&a, &bits, 4);
        if (!isfinite(a)) continue;
      }
    }
    float ref = a / b;
    if (!isfinite(ref) || fabsf(ref) > 1e30f) continue; /* no valid block reaches these */
    float y = 1.0f / b, q0 = a * y, q = fmaf(fmaf(-q0, b, a), y, q0);
    ++checked;
    float lo[4] = {-8.0f, -127.0f, 0.0f, -32.0f}, hi[4] = {7.0f, 127.0f, 15.0f, 31.0f};
    for (int f = 0; f < 4; ++f) {
      if (code(q, lo[f], hi[f]) != code(ref, lo[f], hi[f])) {
        if (++bad <= 5) printf("mismatch a=%a b=%a ieee=%a shared=%a\n", a, b, ref, q);
        break;
      }
    }
  }
  if (bad) { printf("%lld of %lld differ\n", bad, checked); return 1; }
  printf("ok %lld\n", checked);
  return 0;
}
