/*
 * qmat_oracle.c — plain, slow, obviously correct CPU oracle of the
 * block-quantized weight matmul.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the benchmark's CPU
 * baseline do. It shares no code, header or constant with the HIP library.
 *
 * Sources (web pages; each function cites the passage it follows):
 *   [LC05] "05. llama.cpp：从 GGUF 文件到本地推理服务", table in section
 *          "量化类型：Q4_K_M 到底是什么": legacy formats group 32 weights
 *          under one fp16 scale (Q4_0 4.5 bits/weight, Q8_0 about 8.5);
 *          k-quants use a 256-weight superblock of eight 32-element
 *          sub-blocks whose scales are themselves quantized to 6 bits.
 *   [LCHW] "llama.cpp 原理：如何在普通硬件跑本地大模型", section
 *          "量化：内存真正去哪了": Q4_0 = 32 weights, one fp16 scale, each
 *          weight a 4-bit integer, 18 bytes per block.
 *   [KVQ]  lpnh.cn KV-cache article, section "kv-mean-center 进阶技巧",
 *          paragraph "问题": Q4_0 is symmetric, value ≈ scale × q, with no
 *          zero point; the same section subtracts a fixed per-channel bias
 *          from K before it is quantized into the cache.
 *   [BARE] xdnf.cn llama.cpp article, section 3.2: its dequant snippet reads
 *          the fp16 parameters first, then 16 code bytes whose low nibbles
 *          are the block's first 16 elements and high nibbles the last 16,
 *          little-endian.
 * Where the pages are silent the readings are: Q4_0 scale amax/7 and code
 * offset 8; Q8_0 scale amax/127; round half away from zero; fp32→fp16 round
 * to nearest even keeping subnormals; codes from the stored (rounded) scale;
 * an all-zero block gets the zero code; the Q4_K field packing and
 * min-offset rule as written below (this library's own layout); the Q6_K
 * superblock as sixteen 16-weight sub-blocks with int8 scales (the only
 * k-quant split that gives the 210 bytes per 256 weights implied by
 * [LC05]'s 121.71 MiB q6_K embedding: eight 32-weight sub-blocks with 6-bit
 * scales and mins give 208, with int8 scales alone 202), symmetric codes
 * under scale amax/31, and this library's own byte order.
 *
 * Parity pins (tests/test_oracle_pins.py): fp16 codec against numpy on every
 * half and on a float32 sweep; block sizes against the sizes the pages print
 * (18 B, 4.5 bpw; the Qwen3-0.6B file sizes 604.15 MiB and 372.65 MiB);
 * hand-built golden blocks for byte layout and nibble order; the round-trip
 * bound scale/2; brute-force code optimality; idempotence; exact-grid
 * inputs; one-hot and all-ones activations; brute-force 4×64 products.
 * The Q4_K and Q6_K code arithmetic has no value printed on the pages to
 * pin it to: beyond size, layout, round-trip, optimality and exact-grid
 * inputs it is "parity unpinned".
 *
 * Arithmetic: quantizers use IEEE fp32 with correctly rounded + - * / and no
 * contraction (build with -ffp-contract=off); dequantization and every
 * matmul accumulate in fp64 in plain index order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_Q4_0 = 0, ORC_Q8_0 = 1, ORC_Q4_K = 2, ORC_Q6_K = 3 };

/* ---------------------------------------------------------------- fp16 -- */

/* IEEE-754 binary16 from binary32: round to nearest, ties to even; values
 * below the smallest subnormal's half round to zero; overflow gives inf;
 * NaN gives a quiet NaN. Written from the definition of the two formats:
 * |f| = sig * 2^p exactly, then rounded to a multiple of the binary16
 * quantum at that magnitude (2^(e-10) for normal results, 2^-24 below). */
uint16_t oracle_f32_to_f16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  uint32_t ex = (u >> 23) & 0xFFu, man = u & 0x7FFFFFu;
  if (ex == 0xFFu) return (uint16_t)(sign | (man ? 0x7E00u : 0x7C00u));
  if (ex == 0 && man == 0) return sign;
  uint64_t sig;
  int p;
  if (ex == 0) { sig = man; p = -149; }
  else { sig = man | 0x800000u; p = (int)ex - 150; }
  while (sig < 0x800000u) { sig <<= 1; p -= 1; }
  int e = p + 23;                      /* |f| in [2^e, 2^(e+1)) */
  int q = (e < -14 ? -14 : e) - 10;    /* binary16 quantum is 2^q */
  int shift = q - p;                   /* >= 13 */
  uint64_t n;
  if (shift >= 60) {
    n = 0;
  } else {
    uint64_t whole = sig >> shift;
    uint64_t rem = sig & ((1ull << shift) - 1);
    uint64_t half = 1ull << (shift - 1);
    n = whole + ((rem > half || (rem == half && (whole & 1u))) ? 1u : 0u);
  }
  if (n >= 2048) { n >>= 1; q += 1; }  /* carried into the next binade */
  if (n < 1024) return (uint16_t)(sign | n); /* subnormal (q == -24) */
  int E = q + 25;                      /* biased binary16 exponent */
  if (E >= 31) return (uint16_t)(sign | 0x7C00u);
  return (uint16_t)(sign | ((uint32_t)E << 10) | (uint32_t)(n - 1024));
}

/* binary16 to binary64 (exact). */
double oracle_f16_to_f64(uint16_t h) {
  int s = h >> 15, E = (h >> 10) & 31, m = h & 1023;
  double v;
  if (E == 0) v = ldexp((double)m, -24);
  else if (E == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), E - 25);
  return s ? -v : v;
}

/* binary16 to binary32 (exact: every binary16 value is a binary32 value). */
float oracle_f16_to_f32(uint16_t h) { return (float)oracle_f16_to_f64(h); }

/* Array forms of the two conversions above (for exhaustive checks). */
void oracle_f32_to_f16_array(const float *in, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_f16(in[i]);
}

void oracle_f16_to_f64_array(const uint16_t *in, double *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f64(in[i]);
}

/* ----------------------------------------------------------- formats -- */

/* [LCHW]: Q4_0 block = 32 weights, 18 bytes. [LC05 table]: Q8_0 groups 32
 * weights under one fp16 scale with 8-bit values (34 bytes); k-quants use a
 * 256-weight superblock (Q4_K 144 bytes in this layout: 2+2+12+128; Q6_K
 * 210 bytes, [LC05] section 量化类型 and the 121.71 MiB embedding of section
 * KV Cache 类型: 2 + 8 groups of (2 scales + 16 + 8 code bytes)). */
int64_t oracle_block_elems(int fmt) {
  switch (fmt) {
    case ORC_Q4_0: return 32;
    case ORC_Q8_0: return 32;
    case ORC_Q4_K: return 256;
    case ORC_Q6_K: return 256;
    default: return 0;
  }
}

int64_t oracle_block_bytes(int fmt) {
  switch (fmt) {
    case ORC_Q4_0: return 2 + 16;
    case ORC_Q8_0: return 2 + 32;
    case ORC_Q4_K: return 2 + 2 + 12 + 128;
    case ORC_Q6_K: return 2 + 8 * (2 + 16 + 8);
    default: return 0;
  }
}

/* round half away from zero of an fp32 value (C roundf). */
static float rnd(float t) { return roundf(t); }

static float clampf(float v, float lo, float hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

static void put_f16(uint8_t *dst, uint16_t h) {
  dst[0] = (uint8_t)(h & 0xFFu);
  dst[1] = (uint8_t)(h >> 8);
}

static uint16_t get_f16(const uint8_t *src) {
  return (uint16_t)(src[0] | (src[1] << 8));
}

/* Q4_0 quantizer, one block of 32 ([LCHW]: one fp16 scale, 4-bit integers;
 * [KVQ]: symmetric, value = scale × q). */
static void quant_q4_0_block(const float *x, uint8_t *blk) {
  float amax = 0.0f;
  for (int i = 0; i < 32; ++i) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  float d = amax / 7.0f;
  uint16_t h = oracle_f32_to_f16(d);
  float D = oracle_f16_to_f32(h);
  uint8_t code[32];
  for (int i = 0; i < 32; ++i) {
    if (D == 0.0f) {
      code[i] = 8;
    } else {
      float q = clampf(rnd(x[i] / D), -8.0f, 7.0f);
      code[i] = (uint8_t)((int)q + 8);
    }
  }
  put_f16(blk, h);
  /* [BARE 3.2]: byte t = element t (low nibble) | element t+16 (high). */
  for (int t = 0; t < 16; ++t)
    blk[2 + t] = (uint8_t)(code[t] | (code[t + 16] << 4));
}

/* Q8_0 quantizer, one block of 32 ([LC05 table]: 32 weights, one fp16
 * scale, 8-bit values). */
static void quant_q8_0_block(const float *x, uint8_t *blk) {
  float amax = 0.0f;
  for (int i = 0; i < 32; ++i) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  float d = amax / 127.0f;
  uint16_t h = oracle_f32_to_f16(d);
  float D = oracle_f16_to_f32(h);
  put_f16(blk, h);
  for (int i = 0; i < 32; ++i) {
    int8_t q = 0;
    if (D != 0.0f) q = (int8_t)(int)clampf(rnd(x[i] / D), -127.0f, 127.0f);
    memcpy(blk + 2 + i, &q, 1);
  }
}

/* Q4_K-style quantizer, one superblock of 256 ([LC05 table]: superblock of
 * eight 32-element sub-blocks, sub-block scales quantized to 6 bits under
 * an fp16 super-scale; the affine min follows the scale-plus-offset reading
 * of [BARE 3.2]). Steps in order:
 *   1. per sub-block j: lo_j = min(0, min x), hi_j = max x
 *   2. scale_j = (hi_j - lo_j)/15, off_j = -lo_j
 *   3. d = max scale_j / 63, dmin = max off_j / 63, both stored as fp16
 *   4. sc_j = rnd(scale_j/D), mn_j = rnd(off_j/Dmin), clamped to [0,63]
 *   5. S_j = D*sc_j, O_j = Dmin*mn_j (exact in fp32)
 *   6. q_i = clamp(rnd((x_i + O_j)/S_j), 0, 15) */
static void quant_q4_k_block(const float *x, uint8_t *blk) {
  float scale[8], off[8];
  for (int j = 0; j < 8; ++j) {
    const float *s = x + 32 * j;
    float mn = s[0], mx = s[0];
    for (int i = 1; i < 32; ++i) {
      if (s[i] < mn) mn = s[i];
      if (s[i] > mx) mx = s[i];
    }
    float lo = mn < 0.0f ? mn : 0.0f;
    float hi = mx;
    scale[j] = (hi - lo) / 15.0f;
    off[j] = -lo;
  }
  float smax = 0.0f, omax = 0.0f;
  for (int j = 0; j < 8; ++j) {
    if (scale[j] > smax) smax = scale[j];
    if (off[j] > omax) omax = off[j];
  }
  float d = smax / 63.0f, dmin = omax / 63.0f;
  uint16_t hd = oracle_f32_to_f16(d), hm = oracle_f32_to_f16(dmin);
  float D = oracle_f16_to_f32(hd), Dm = oracle_f16_to_f32(hm);
  int sc[8], mnq[8];
  for (int j = 0; j < 8; ++j) {
    sc[j] = (D == 0.0f) ? 0 : (int)clampf(rnd(scale[j] / D), 0.0f, 63.0f);
    mnq[j] = (Dm == 0.0f) ? 0 : (int)clampf(rnd(off[j] / Dm), 0.0f, 63.0f);
  }
  put_f16(blk, hd);
  put_f16(blk + 2, hm);
  /* 96-bit little-endian field store: field f at bits 6f..6f+5. */
  uint8_t fields[12];
  memset(fields, 0, sizeof fields);
  for (int f = 0; f < 16; ++f) {
    int v = f < 8 ? sc[f] : mnq[f - 8];
    for (int bit = 0; bit < 6; ++bit) {
      int pos = 6 * f + bit;
      if ((v >> bit) & 1) fields[pos / 8] |= (uint8_t)(1u << (pos % 8));
    }
  }
  memcpy(blk + 4, fields, 12);
  for (int j = 0; j < 8; ++j) {
    float S = D * (float)sc[j];
    float O = Dm * (float)mnq[j];
    uint8_t q[32];
    for (int i = 0; i < 32; ++i) {
      if (S == 0.0f) q[i] = 0;
      else q[i] = (uint8_t)(int)clampf(rnd((x[32 * j + i] + O) / S), 0.0f, 15.0f);
    }
    for (int t = 0; t < 16; ++t)
      blk[16 + 16 * j + t] = (uint8_t)(q[t] | (q[t + 16] << 4));
  }
}

/* Q6_K-style quantizer, one superblock of 256 ([LC05] section 量化类型:
 * 256-weight superblock whose sub-block scales are themselves quantized;
 * Q6_K is the near-lossless 6-bit member). Sub-block j is the 16 weights
 * 16j..16j+15. Steps in order:
 *   1. s_j = amax_j / 31 (symmetric: codes -31..31 around zero)
 *   2. d = max s_j / 127, stored as fp16
 *   3. sc_j = rnd(s_j / D), clamped to [0, 127] (int8)
 *   4. S_j = D * sc_j (exact in fp32)
 *   5. q_i = clamp(rnd(x_i / S_j), -32, 31), stored as the 6-bit code q+32
 * Byte order: fp16 d, then for each 32-weight group g = 0..7 (sub-blocks
 * 2g and 2g+1): sc_2g, sc_2g+1 as int8; 16 bytes whose byte t holds the
 * low 4 bits of code 32g+t (low nibble) and of code 32g+16+t (high
 * nibble); two little-endian 32-bit words H0, H1 where bits 2w..2w+1 of
 * byte b of H0 are the high 2 bits of code 32g+4w+b, and of H1 those of
 * code 32g+16+4w+b. */
static void quant_q6_k_block(const float *x, uint8_t *blk) {
  float s[16];
  for (int j = 0; j < 16; ++j) {
    float amax = 0.0f;
    for (int i = 0; i < 16; ++i) {
      float a = fabsf(x[16 * j + i]);
      if (a > amax) amax = a;
    }
    s[j] = amax / 31.0f;
  }
  float smax = 0.0f;
  for (int j = 0; j < 16; ++j)
    if (s[j] > smax) smax = s[j];
  float d = smax / 127.0f;
  uint16_t hd = oracle_f32_to_f16(d);
  float D = oracle_f16_to_f32(hd);
  int sc[16];
  uint8_t code[256];
  for (int j = 0; j < 16; ++j) {
    sc[j] = (D == 0.0f) ? 0 : (int)clampf(rnd(s[j] / D), 0.0f, 127.0f);
    float S = D * (float)sc[j];
    for (int i = 0; i < 16; ++i) {
      int q = 0;
      if (S != 0.0f) q = (int)clampf(rnd(x[16 * j + i] / S), -32.0f, 31.0f);
      code[16 * j + i] = (uint8_t)(q + 32);
    }
  }
  put_f16(blk, hd);
  for (int g = 0; g < 8; ++g) {
    uint8_t *grp = blk + 2 + 26 * g;
    const uint8_t *c = code + 32 * g;
    int8_t sa = (int8_t)sc[2 * g], sb = (int8_t)sc[2 * g + 1];
    memcpy(grp, &sa, 1);
    memcpy(grp + 1, &sb, 1);
    for (int t = 0; t < 16; ++t)
      grp[2 + t] = (uint8_t)((c[t] & 15) | ((c[16 + t] & 15) << 4));
    uint32_t h0 = 0, h1 = 0;
    for (int w = 0; w < 4; ++w)
      for (int b = 0; b < 4; ++b) {
        h0 |= (uint32_t)(c[4 * w + b] >> 4) << (8 * b + 2 * w);
        h1 |= (uint32_t)(c[16 + 4 * w + b] >> 4) << (8 * b + 2 * w);
      }
    for (int b = 0; b < 4; ++b) {
      grp[18 + b] = (uint8_t)(h0 >> (8 * b));
      grp[22 + b] = (uint8_t)(h1 >> (8 * b));
    }
  }
}

/* Quantize a [rows][K] fp32 matrix into rows*(K/block_elems) blocks, row
 * after row. Returns 0, or -1 for an unknown format or a ragged K. */
int oracle_quantize(int fmt, const float *W, uint8_t *out, int64_t rows,
                    int64_t K) {
  int64_t be = oracle_block_elems(fmt), bb = oracle_block_bytes(fmt);
  if (be == 0 || K < 0 || rows < 0 || K % be != 0) return -1;
  int64_t nb = K / be;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const float *x = W + r * K + b * be;
      uint8_t *blk = out + (r * nb + b) * bb;
      if (fmt == ORC_Q4_0) quant_q4_0_block(x, blk);
      else if (fmt == ORC_Q8_0) quant_q8_0_block(x, blk);
      else if (fmt == ORC_Q4_K) quant_q4_k_block(x, blk);
      else quant_q6_k_block(x, blk);
    }
  }
  return 0;
}

/* KV-cache write ([KVQ] section "量化 KV Cache 的一键配置方法": K and V are
 * stored as q8_0 or q4_0 blocks; section "kv-mean-center 进阶技巧": a fixed
 * per-(head, channel) bias is subtracted from K before Q4_0 quantization).
 * Row i of `rows` ([n][dim] fp32), minus `bias` ([dim], fp32 subtraction)
 * when given, is quantized into cache row cell0 + i; every other cache byte
 * is left as it was. Returns 0, or -1 for a bad format or shape. */
int oracle_kv_write(int fmt, const float *rows, const float *bias, uint8_t *cache,
                    int64_t cell0, int64_t n, int64_t cells, int64_t dim) {
  if (fmt != ORC_Q4_0 && fmt != ORC_Q8_0) return -1;
  if (dim < 0 || dim % 32 != 0 || n < 0 || cell0 < 0 || n > cells || cell0 > cells - n)
    return -1;
  int64_t nb = dim / 32, bb = oracle_block_bytes(fmt);
  float x[32];
  for (int64_t i = 0; i < n; ++i) {
    for (int64_t b = 0; b < nb; ++b) {
      for (int e = 0; e < 32; ++e) {
        float v = rows[i * dim + b * 32 + e];
        x[e] = bias ? v - bias[b * 32 + e] : v;
      }
      uint8_t *blk = cache + ((cell0 + i) * nb + b) * bb;
      if (fmt == ORC_Q4_0) quant_q4_0_block(x, blk);
      else quant_q8_0_block(x, blk);
    }
  }
  return 0;
}

/* ------------------------------------------------------ dequantization -- */

/* 6-bit field f of the 96-bit little-endian integer at p. */
static int field6(const uint8_t *p, int f) {
  int v = 0;
  for (int bit = 0; bit < 6; ++bit) {
    int pos = 6 * f + bit;
    v |= ((p[pos / 8] >> (pos % 8)) & 1) << bit;
  }
  return v;
}

/* Code e (0..31) of a Q6_K group: low 4 bits from the nibble bytes, high
 * 2 bits from H0 (e < 16) or H1 (layout at quant_q6_k_block). */
static int code6(const uint8_t *grp, int e) {
  int half = e >> 4, r = e & 15, t = r, w = r >> 2, b = r & 3;
  int lo = half ? (grp[2 + t] >> 4) : (grp[2 + t] & 15);
  int hi = (grp[18 + 4 * half + b] >> (2 * w)) & 3;
  return lo | (hi << 4);
}

/* Dequantize one block into fp64 (exact for all four formats). */
static void dequant_block(int fmt, const uint8_t *blk, double *w) {
  if (fmt == ORC_Q4_0) {
    double D = oracle_f16_to_f64(get_f16(blk));
    for (int t = 0; t < 16; ++t) {
      int lo = blk[2 + t] & 15, hi = blk[2 + t] >> 4;
      w[t] = D * (double)(lo - 8);
      w[t + 16] = D * (double)(hi - 8);
    }
  } else if (fmt == ORC_Q8_0) {
    double D = oracle_f16_to_f64(get_f16(blk));
    for (int i = 0; i < 32; ++i) {
      int8_t q;
      memcpy(&q, blk + 2 + i, 1);
      w[i] = D * (double)q;
    }
  } else if (fmt == ORC_Q6_K) {
    double D = oracle_f16_to_f64(get_f16(blk));
    for (int g = 0; g < 8; ++g) {
      const uint8_t *grp = blk + 2 + 26 * g;
      for (int e = 0; e < 32; ++e) {
        int8_t sc;
        memcpy(&sc, grp + (e >> 4), 1);
        w[32 * g + e] = D * (double)sc * (double)(code6(grp, e) - 32);
      }
    }
  } else {
    double D = oracle_f16_to_f64(get_f16(blk));
    double Dm = oracle_f16_to_f64(get_f16(blk + 2));
    for (int j = 0; j < 8; ++j) {
      double S = D * (double)field6(blk + 4, j);
      double O = Dm * (double)field6(blk + 4, 8 + j);
      const uint8_t *c = blk + 16 + 16 * j;
      for (int t = 0; t < 16; ++t) {
        w[32 * j + t] = S * (double)(c[t] & 15) - O;
        w[32 * j + t + 16] = S * (double)(c[t] >> 4) - O;
      }
    }
  }
}

/* Dequantize rows*(K/block_elems) blocks into fp64 [rows][K]. */
int oracle_dequant(int fmt, const uint8_t *blocks, double *out, int64_t rows,
                   int64_t K) {
  int64_t be = oracle_block_elems(fmt), bb = oracle_block_bytes(fmt);
  if (be == 0 || K < 0 || rows < 0 || K % be != 0) return -1;
  int64_t nb = K / be;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b)
      dequant_block(fmt, blocks + (r * nb + b) * bb, out + r * K + b * be);
  return 0;
}

/* ------------------------------------------------------------- matmul -- */

/* y[m] = sum_k W'[m][k] * x[k], W' the dequantized weights, fp64, k in
 * order. x is used exactly as given (fp32 widened to fp64). */
int oracle_gemv(int fmt, const uint8_t *blocks, const float *x, double *y,
                int64_t M, int64_t K) {
  int64_t be = oracle_block_elems(fmt), bb = oracle_block_bytes(fmt);
  if (be == 0 || K < 0 || M < 0 || K % be != 0) return -1;
  int64_t nb = K / be;
  int bad = 0;
#pragma omp parallel
  {
    double *w = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    if (!w) {
#pragma omp atomic write
      bad = 1;
    }
#pragma omp for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
      if (!w) continue;
      for (int64_t b = 0; b < nb; ++b)
        dequant_block(fmt, blocks + (m * nb + b) * bb, w + b * be);
      double s = 0.0;
      for (int64_t k = 0; k < K; ++k) s += w[k] * (double)x[k];
      y[m] = s;
    }
    free(w);
  }
  return bad ? -2 : 0;
}

/* Y[n][m] = sum_k W'[m][k] * X'[n][k] with W' the dequantized weights (fmt)
 * and X' the dequantized Q8_0 activation blocks, fp64, k in order. */
int oracle_gemm(int fmt, const uint8_t *blocks, const uint8_t *Xq8, double *Y,
                int64_t M, int64_t K, int64_t N) {
  int64_t be = oracle_block_elems(fmt), bb = oracle_block_bytes(fmt);
  if (be == 0 || K < 0 || M < 0 || N < 0 || K % be != 0 || K % 32 != 0)
    return -1;
  int64_t nb = K / be, nbx = K / 32;
  double *X = (double *)malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
  if (!X) return -2;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t b = 0; b < nbx; ++b)
      dequant_block(ORC_Q8_0, Xq8 + (n * nbx + b) * 34, X + n * K + b * 32);
  int bad = 0;
#pragma omp parallel
  {
    double *w = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    if (!w) {
#pragma omp atomic write
      bad = 1;
    }
#pragma omp for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
      if (!w) continue;
      for (int64_t b = 0; b < nb; ++b)
        dequant_block(fmt, blocks + (m * nb + b) * bb, w + b * be);
      for (int64_t n = 0; n < N; ++n) {
        const double *xr = X + n * K;
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) s += w[k] * xr[k];
        Y[n * M + m] = s;
      }
    }
    free(w);
  }
  free(X);
  return bad ? -2 : 0;
}

/* Number of OpenMP threads the oracle's parallel loops use. */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Set the number of OpenMP threads for the oracle's later parallel loops
 * (n < 1 leaves it unchanged); returns the number now in effect. Used by the
 * benchmark's CPU baseline to time one thread beside all of them. */
int oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}
