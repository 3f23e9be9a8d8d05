/* Runs the oracle (qmat_oracle.c, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer) over the cases its Python pins use: every
 * format's quantizer on random, tied, zero, subnormal-scale and extreme
 * blocks, the round-trip bound of Q4_0 / Q8_0, dequantization, the
 * brute-force 4 x 64 products, the KV-cache write (with and without the
 * bias, touching only its cells) and the refused arguments. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint16_t oracle_f32_to_f16(float f);
double oracle_f16_to_f64(uint16_t h);
int64_t oracle_block_elems(int fmt);
int64_t oracle_block_bytes(int fmt);
int oracle_quantize(int fmt, const float *W, uint8_t *out, int64_t rows, int64_t K);
int oracle_dequant(int fmt, const uint8_t *blocks, double *out, int64_t rows, int64_t K);
int oracle_gemv(int fmt, const uint8_t *blocks, const float *x, double *y, int64_t M, int64_t K);
int oracle_gemm(int fmt, const uint8_t *blocks, const uint8_t *Xq8, double *Y, int64_t M,
                int64_t K, int64_t N);
int oracle_kv_write(int fmt, const float *rows, const float *bias, uint8_t *cache,
                    int64_t cell0, int64_t n, int64_t cells, int64_t dim);

static int failures = 0;
#define CHECK(c)                                               \
  do {                                                         \
    if (!(c)) {                                                \
      fprintf(stderr, "FAIL line %d: %s\n", __LINE__, #c);     \
      ++failures;                                              \
    }                                                          \
  } while (0)

static uint64_t rs = 88172645463325252ull;
static double urand(void) { /* xorshift64, uniform in [0, 1) */
  rs ^= rs << 13;
  rs ^= rs >> 7;
  rs ^= rs << 17;
  return (double)(rs >> 11) / 9007199254740992.0;
}

/* rows of several populations, as the GPU tests' mixed matrices */
static void fill(float *W, int64_t rows, int64_t K) {
  for (int64_t r = 0; r < rows; ++r) {
    int kind = (int)(r % 7);
    for (int64_t k = 0; k < K; ++k) {
      double u = 2.0 * urand() - 1.0, v;
      switch (kind) {
        case 0: v = 0.02 * u; break;
        case 1: v = u; break;
        case 2: v = 1e-6 * u; break;            /* fp16-subnormal scales */
        case 3: v = 0.0; break;                 /* zero blocks */
        case 4: v = (double)((int)(u * 14)) * 0.25; break;  /* ties */
        case 5: v = (k % 32 == 0) ? 3.5 : 0.25 * (double)((int)(u * 14)); break;
        default: v = (k % 97 == 0) ? 60000.0 * u : 0.5 * u; break;
      }
      W[r * K + k] = (float)v;
    }
  }
}

int main(void) {
  const int64_t rows = 21, K = 1024;
  float *W = malloc(sizeof(float) * rows * K);
  double *D = malloc(sizeof(double) * rows * K);
  fill(W, rows, K);
  for (int fmt = 0; fmt < 4; ++fmt) {
    const int64_t be = oracle_block_elems(fmt), bb = oracle_block_bytes(fmt);
    uint8_t *B = malloc((size_t)(rows * (K / be) * bb));
    CHECK(oracle_quantize(fmt, W, B, rows, K) == 0);
    CHECK(oracle_dequant(fmt, B, D, rows, K) == 0);
    if (fmt < 2) { /* round trip within half a step of a normal fp16 scale (a
                      subnormal one can round down so far that codes clamp) */
      for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < K / 32; ++b) {
          const uint8_t *blk = B + (r * (K / 32) + b) * bb;
          double d = oracle_f16_to_f64((uint16_t)(blk[0] | blk[1] << 8));
          for (int e = 0; e < 32; ++e) {
            double w = W[r * K + b * 32 + e], wq = D[r * K + b * 32 + e];
            CHECK(fabs(w - wq) <= d / 2 * (1 + 1e-12) || d < 0x1p-14);
          }
        }
    }
    /* brute-force 4 x 64 products */
    const int64_t m = 4, k = 256, n = 3;
    uint8_t *Bs = malloc((size_t)(m * (k / be) * bb)), *Xq = malloc((size_t)(n * (k / 32) * 34));
    float x[256], X[3 * 256];
    double y[4], Y[12], Wd[4 * 256], Xd[3 * 256];
    for (int i = 0; i < 256; ++i) x[i] = (float)(2.0 * urand() - 1.0);
    for (int i = 0; i < 3 * 256; ++i) X[i] = (float)(4.0 * urand() - 2.0);
    float Wm[4 * 256];
    for (int i = 0; i < 4 * 256; ++i) Wm[i] = W[i];
    CHECK(oracle_quantize(fmt, Wm, Bs, m, k) == 0);
    CHECK(oracle_quantize(1, X, Xq, n, k) == 0);
    CHECK(oracle_dequant(fmt, Bs, Wd, m, k) == 0);
    CHECK(oracle_dequant(1, Xq, Xd, n, k) == 0);
    CHECK(oracle_gemv(fmt, Bs, x, y, m, k) == 0);
    CHECK(oracle_gemm(fmt, Bs, Xq, Y, m, k, n) == 0);
    for (int i = 0; i < m; ++i) {
      double s = 0;
      for (int j = 0; j < k; ++j) s += Wd[i * k + j] * (double)x[j];
      CHECK(fabs(s - y[i]) <= 1e-12 * (1 + fabs(s)));
      for (int t = 0; t < n; ++t) {
        double u = 0;
        for (int j = 0; j < k; ++j) u += Wd[i * k + j] * Xd[t * k + j];
        CHECK(fabs(u - Y[t * m + i]) <= 1e-12 * (1 + fabs(u)));
      }
    }
    /* refused arguments */
    CHECK(oracle_quantize(fmt, W, B, rows, be + 1) == -1);
    CHECK(oracle_quantize(fmt, W, B, -1, K) == -1);
    CHECK(oracle_gemv(fmt, B, x, y, 1, -be) == -1);
    CHECK(oracle_gemm(fmt, B, Xq, Y, 1, be + 32 * (be > 32), -1) == -1);
    free(Bs);
    free(Xq);
    free(B);
  }
  CHECK(oracle_quantize(7, W, NULL, rows, K) == -1);
  /* KV-cache write: only the written cells change */
  for (int fmt = 0; fmt < 2; ++fmt) {
    const int64_t dim = 256, cells = 9, rb = dim / 32 * oracle_block_bytes(fmt);
    uint8_t *cache = malloc((size_t)(cells * rb)), *copy = malloc((size_t)(cells * rb));
    for (int64_t i = 0; i < cells * rb; ++i) cache[i] = (uint8_t)(urand() * 256);
    memcpy(copy, cache, (size_t)(cells * rb));
    float bias[256];
    for (int i = 0; i < 256; ++i) bias[i] = (float)urand();
    CHECK(oracle_kv_write(fmt, W, fmt ? NULL : bias, cache, 3, 4, cells, dim) == 0);
    CHECK(memcmp(cache, copy, (size_t)(3 * rb)) == 0);
    CHECK(memcmp(cache + 7 * rb, copy + 7 * rb, (size_t)(2 * rb)) == 0);
    CHECK(oracle_kv_write(fmt, W, NULL, cache, 8, 2, cells, dim) == -1);
    CHECK(oracle_kv_write(fmt, W, NULL, cache, INT64_MAX, 2, cells, dim) == -1);
    CHECK(oracle_kv_write(fmt, W, NULL, cache, 2, INT64_MAX, cells, dim) == -1);
    CHECK(oracle_kv_write(fmt, W, NULL, cache, -1, 1, cells, dim) == -1);
    CHECK(oracle_kv_write(fmt, W, NULL, cache, 0, 1, cells, 48) == -1);
    CHECK(oracle_kv_write(2, W, NULL, cache, 0, 1, cells, dim) == -1);
    free(cache);
    free(copy);
  }
  /* fp16 codec over every half */
  for (uint32_t h = 0; h < 65536; ++h) {
    double v = oracle_f16_to_f64((uint16_t)h);
    if (v == v && fabs(v) <= 65504.0) CHECK(oracle_f32_to_f16((float)v) == h || v == 0.0);
  }
  free(W);
  free(D);
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("oracle driver: all cases ok\n");
  return 0;
}
