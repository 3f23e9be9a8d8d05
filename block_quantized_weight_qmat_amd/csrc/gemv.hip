// gemv.hip — decode-time y = dequant(W) x for Q4_0 / Q8_0 / Q4_K-style W.
//
// Source: "05. llama.cpp：从 GGUF 文件到本地推理服务", section "性能直觉：带宽
// 决定 Decode，算力决定 Prefill": single-token decode reads every weight once,
// so its speed limit is memory bandwidth divided by weight bytes. The kernel
// is therefore built around the HBM stream of packed blocks, and its integer
// work per block is kept small enough to hide under that stream.
//
// Work split. Two kernels share the arithmetic below. Rows of 128 to 512
// slices (K = 4096 .. 16384), and of 32 to 127 slices in matrices of at most
// 8192 rows, use gemv_rows_kernel: a workgroup of 16 waves owns 16 rows, one
// per wave; the activations are converted once per workgroup into LDS digit
// records shared by the 16 rows (see the kernel). Other rows (shorter, or
// short rows of taller matrices, where the row kernel's per-workgroup
// conversion repeats too often) use gemv_kernel:
//   * A workgroup owns G groups of R consecutive rows and all of K. Its waves
//     split K into strips of 64 slices; lane l of a strip owns one
//     32-element slice (one Q4_0/Q8_0 block, or one sub-block of a Q4_K
//     superblock) of every row, so neighbouring lanes read neighbouring
//     blocks.
//   * A wave first sends its strip of activations (64 x 128 bytes) from
//     memory straight into LDS, then issues the R rows' weight loads: each
//     lane reads its block with 4-byte-aligned 16- and 2-byte loads. Once
//     the activation loads have landed (loads complete in issue order) the
//     lane reads its slice back from LDS and converts it while the weights
//     stream in; the converted slice serves all G x R rows from registers.
//     D row groups are requested before the conversion; group g+D is
//     requested as soon as group g has been consumed.
//     Activations loaded straight into registers, 128 bytes per lane, cost
//     far more load bandwidth than the same bytes staged through LDS.
//   * Row base addresses are wave-uniform (scalar registers), lane offsets
//     32-bit. When the row stride is 2 mod 4, even and odd rows have
//     different block alignments and get their own fixed load offsets.
//   * Per-lane partial sums of the G x R rows are reduced across the wave
//     with VALU lane exchanges that halve the live values at each step, then
//     across the strips in LDS in a fixed order (deterministic).
//
// Arithmetic: exact integer dot products per block
//   * Each lane turns its 32 activations into 20-bit fixed point with a
//     power-of-two scale: X = rint(x * 2^s), s = 19 - exponent(amax), one
//     lower if the largest value would round beyond the digit range. The
//     step is then at most 2^-17.9 of the slice's largest value. (16 bits
//     are not enough: a row of large weights with a small dot product turns
//     a 2^-15 activation step into a relative error near 1e-3.)
//   * The rounding needs no integer conversion: fma(x, 2^s, 1.5*2^23 + b)
//     is a float whose low 20 bits are V = X + b, for a bias b that makes V
//     non-negative.
//   * 4-bit formats: b = 0x88888, so V's five nibbles minus 8 are signed
//     digits with X = sum_i 16^i (nibble_i - 8). They are packed in the
//     codes' own nibble order (byte t of a code word holds elements t and
//     t+16) and multiplied with v_dot8_i32_i4. The codes become signed
//     4-bit values c - 8 with one XOR (c ^ 8 read as a signed nibble is
//     c - 8), so a Q4_0 block needs no offset term at all:
//       sum (c - 8) X = sum_i 16^i dot8(c ^ 0x8..8, digit_i).
//   * Q8_0: b = 0x88080, signed byte digits b0 - 128, b1 - 128, b2 - 8,
//     multiplied with v_dot4_i32_i8 against the int8 codes.
//   * Per (row, slice) the exact integer is converted to fp32, scaled by the
//     block scale and 2^-s, and accumulated in fp32.
//
// The file also holds the batched GEMV (many GEMVs per launch, the job taken
// from blockIdx.y) and the few-token products of the decode batch that do
// not run on the matrix cores (decode_rows_kernel, gemm_small_kernel), each
// described where it is defined.
#include "qmat_device.hpp"
#include "qmat_launch.hpp"

namespace qmat {
namespace {

// Waves per workgroup: 7 strips of activations (56 KB) plus the row sums
// stay inside the default 64 KB of LDS a workgroup may allocate.
constexpr int kMaxStrips = 7;

__device__ __forceinline__ int32_t sdot4(uint32_t a, uint32_t b, int32_t c) {
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

__device__ __forceinline__ int32_t sdot8(uint32_t a, uint32_t b, int32_t c) {
  return __builtin_amdgcn_sdot8((int)a, (int)b, c, false);
}

// (m & a) | (~m & b): v_bfi_b32
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) {
  return (m & a) | (~m & b);
}

__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_fmaxf(__builtin_fmaxf(a, b), c);  // v_max3_f32
}

__device__ __forceinline__ void load_x32(const float* __restrict__ x, f32x4 (&v)[8]) {
  const f32x4* p = reinterpret_cast<const f32x4*>(x);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = p[i];
}

// Scale the slice to 20-bit fixed point. Returns the multiplier 2^s (after
// an exact 2^64 pre-scale of v when s is too large for one factor) and sets
// inv = 2^-s. `lim` is the largest |X| the digit split accepts.
__device__ __forceinline__ float slice_scale(f32x4 (&v)[8], float lim, float& inv) {
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    am = max3f(am, fabsf(v[i].x), fabsf(v[i].y));
    am = max3f(am, fabsf(v[i].z), fabsf(v[i].w));
  }
  int e;
  frexpf(am, &e);  // am = m 2^e, m in [0.5, 1) (e = 0 for am = 0)
  int s = 19 - e;  // am 2^s in [2^18, 2^19)
  if (ldexpf(am, s) >= lim + 0.5f) s -= 1;
  // 2^-149 is the smallest float: subnormal x are integer multiples of it,
  // so with s = 149 they scale to exact integers and 2^-s stays a float
  s = min(s, 149);
  inv = ldexpf(1.0f, -s);
  if (__builtin_expect(s > 120, 0)) {
    // tiny activations: pre-scale by 2^64 so that 2^s stays a finite float
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i].x = ldexpf(v[i].x, 64);
      v[i].y = ldexpf(v[i].y, 64);
      v[i].z = ldexpf(v[i].z, 64);
      v[i].w = ldexpf(v[i].w, 64);
    }
    s -= 64;
  }
  return ldexpf(1.0f, s);
}

// Elements 4i..4i+3 scaled and biased: bytes 0, 1 and 2 of the four 20-bit
// values V = rint(x 2^s) + bias, packed one per byte (lo, hi, top). The
// float fma(x, 2^s, 1.5*2^23 + bias) is exact (it stays below 2^24) and its
// bits are 0x4B400000 + bias + X, whose low 20 bits are V; byte 2 of the
// float carries 0x40 above V's fifth nibble.
__device__ __forceinline__ void bias20(const f32x4& v, float scale, float magic, uint32_t& lo,
                                       uint32_t& hi, uint32_t& top) {
  uint32_t t[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) t[k] = __builtin_bit_cast(uint32_t, fmaf(v[k], scale, magic));
  const uint32_t p = perm_b32(t[1], t[0], 0x05040100u);  // {V0, V1} low halves
  const uint32_t q = perm_b32(t[3], t[2], 0x05040100u);  // {V2, V3}
  lo = perm_b32(q, p, 0x06040200u);
  hi = perm_b32(q, p, 0x07050301u);
  // byte 2 of each (0x0c selects a zero byte)
  top = perm_b32(t[1], t[0], 0x0c0c0602u) | perm_b32(t[3], t[2], 0x06020c0cu);
}

constexpr float kMagicF = 12582912.0f;  // 1.5 * 2^23

// 4-bit digits: d[i][t] holds signed digit i of elements 4t+b (low nibble of
// byte b) and 4t+b+16 (high nibble), the layout of code word t.
struct XNib {
  uint32_t d[5][4];
  int32_t sx;  // sum of X (used by Q4_K only)
  float inv;   // 2^-s
};

// X in [-0x88888, 0xFFFFF - 0x88888]: V = X + 0x88888 has five nibbles.
constexpr uint32_t kNibBias = 0x88888u;
constexpr float kNibLim = (float)(0xFFFFF - kNibBias);  // 489335

__device__ __forceinline__ void nib_digits(uint32_t a, uint32_t b, uint32_t (&d)[2]) {
  // low nibbles of a's bytes with b's low nibbles above them, then the high
  // nibbles likewise; signed by flipping each nibble's top bit
  constexpr uint32_t kHi = 0xF0F0F0F0u, kSign = 0x88888888u;
  d[0] = bfi(kHi, b << 4, a) ^ kSign;
  d[1] = bfi(kHi, b, a >> 4) ^ kSign;
}

__device__ __forceinline__ void prep_nib(f32x4 (&v)[8], XNib& xp, bool want_sum) {
  const float scale = slice_scale(v, kNibLim, xp.inv);
  const float magic = kMagicF + (float)kNibBias;  // exact: below 2^24
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    uint32_t aL, aH, aT, bL, bH, bT;
    bias20(v[t], scale, magic, aL, aH, aT);      // elements 4t..4t+3
    bias20(v[t + 4], scale, magic, bL, bH, bT);  // elements 16+4t..
    uint32_t d[2];
    nib_digits(aL, bL, d);
    xp.d[0][t] = d[0];
    xp.d[1][t] = d[1];
    nib_digits(aH, bH, d);
    xp.d[2][t] = d[0];
    xp.d[3][t] = d[1];
    nib_digits(aT, bT, d);  // byte 2 holds one nibble: d[1] would be all -8
    xp.d[4][t] = d[0];
  }
  xp.sx = 0;
  if (want_sum) {
    uint32_t a[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      int32_t acc = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) acc = sdot8(xp.d[i][t], 0x11111111u, acc);
      a[i] = (uint32_t)acc;
    }
    xp.sx = (int32_t)((((a[4] * 16u + a[3]) * 16u + a[2]) * 16u + a[1]) * 16u + a[0]);
  }
}

// Digit accumulators carried from row to row: v_dot8/v_dot4 accumulate in
// place, so instead of clearing them for every block (one move each) a row's
// exact sum is the difference of the combined totals after and before it.
// Differences are taken modulo 2^32, which is exact because every block's
// sum fits in int32.
struct NibAcc {
  int32_t a[5];
  uint32_t prev;  // combined total before the current block
};

// sum_e w_e X_e for 32 signed nibbles w (code word layout), exact.
__device__ __forceinline__ int32_t nib_dot(const uint32_t (&w)[4], const XNib& xp, NibAcc& ac) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 5; ++i) ac.a[i] = sdot8(w[t], xp.d[i][t], ac.a[i]);
  const uint32_t tot = (((((uint32_t)ac.a[4] * 16u + (uint32_t)ac.a[3]) * 16u +
                          (uint32_t)ac.a[2]) * 16u + (uint32_t)ac.a[1]) * 16u) +
                       (uint32_t)ac.a[0];
  const int32_t r = (int32_t)(tot - ac.prev);
  ac.prev = tot;
  return r;
}

// 8-bit digits: xl[i] / xh[i] / xt[i] hold the low / middle / top signed
// digit of elements 4i..4i+3, X = 65536 xt + 256 xh + xl.
struct XByte {
  uint32_t xl[8], xh[8], xt[8];
  int32_t sx;
  int32_t sxh[2];  // sums of X over elements 0..15 and 16..31 (Q6_K only)
  float inv;
};

struct ByteAcc {
  int32_t l, h, t;
  uint32_t prev;
};

// X in [-0x88080, 0xFFFFF - 0x88080]: V = X + 0x88080 has bytes b0, b1 in
// [0, 255] and b2 in [0, 15], digits b0 - 128, b1 - 128, b2 - 8. The bound
// also keeps |sum q X| over 32 int8 codes below 2^31.
constexpr uint32_t kByteBias = 0x88080u;
constexpr float kByteLim = (float)(0xFFFFF - kByteBias);  // 491391

__device__ __forceinline__ void prep_byte(f32x4 (&v)[8], XByte& xp, bool want_sum) {
  const float scale = slice_scale(v, kByteLim, xp.inv);
  const float magic = kMagicF + (float)kByteBias;  // exact: below 2^24
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t lo, hi, top;
    bias20(v[i], scale, magic, lo, hi, top);
    xp.xl[i] = lo ^ 0x80808080u;
    xp.xh[i] = hi ^ 0x80808080u;
    // byte 2 of the float is 0x40 | b2: keep b2, then b2 - 8 as a signed byte
    xp.xt[i] = ((top & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
  }
  xp.sx = 0;
  xp.sxh[0] = xp.sxh[1] = 0;
  if (want_sum) {
    // X = xl + 256 xh + 65536 xt per element; each half's sum is exact
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int32_t l = 0, m = 0, t = 0;
#pragma unroll
      for (int i = 4 * h; i < 4 * h + 4; ++i) {
        l = sdot4(xp.xl[i], 0x01010101u, l);
        m = sdot4(xp.xh[i], 0x01010101u, m);
        t = sdot4(xp.xt[i], 0x01010101u, t);
      }
      xp.sxh[h] = (t * 256 + m) * 256 + l;
    }
  }
}

// A lane's fixed load offsets and alignment case for one 18- or 34-byte
// block at byte offset o of a row whose base has alignment parity p (row
// bases are 2-byte aligned): if (base + o) = 0 mod 4 the 16-byte load at o
// holds the scale and the first code bytes and the 2-byte load at o+B-2 the
// last two code bytes; if it is 2 mod 4 the 2-byte load at o is the scale
// and the 16-byte load(s) at o+2 hold the codes. Both cases read exactly
// the block with 4-byte-aligned 16-byte loads.
struct BlockLane {
  uint32_t o16;  // offset of the (first) 16-byte load
  uint32_t o2;   // offset of the 2-byte load
  uint32_t sel;  // v_perm selector realigning the codes to 4-byte words
  bool mis;      // block starts at 2 mod 4
  uint32_t o8;   // Q6_K: offset of the 8-byte load
  uint32_t od;   // Q6_K: offset of the superblock's scale d
};

__device__ __forceinline__ BlockLane block_lane(uint32_t o, uint32_t p, uint32_t bytes) {
  BlockLane b;
  b.mis = ((o + p) & 2u) != 0;
  b.o16 = o + (b.mis ? 2u : 0u);
  b.o2 = o + (b.mis ? 0u : bytes - 2u);
  b.sel = b.mis ? 0x03020100u : 0x05040302u;
  return b;
}

// ------------------------------------------------------------------ Q4_0 --
// 18-byte blocks: fp16 scale, 16 code bytes; weight = d * (c - 8).
struct FmtQ4_0 {
  static constexpr int kBytes = 18;
  static constexpr int kLoads = 2;  // memory instructions per row
  typedef XNib XP;
  typedef NibAcc Acc;
  struct Raw {
    u32x4 v;
    uint16_t s;  // widened where it is used, after the load has landed
  };
  static constexpr bool kSum = false;  // records need sums of X
  __host__ __device__ static int64_t row_bytes(int64_t K) { return (K >> 5) * 18; }
  // loads of slice j in a row whose start has alignment parity p (0 or 2)
  __device__ static BlockLane lane(int j, uint32_t p) {
    return block_lane((uint32_t)j * 18u, p, 18);
  }
  __device__ static void prep(f32x4 (&v)[8], XP& xp) { prep_nib(v, xp, false); }
  __device__ static void load(const uint8_t* __restrict__ row, const BlockLane& L, Raw& r) {
    r.v = *reinterpret_cast<const u32x4_a4*>(row + L.o16);
    r.s = *reinterpret_cast<const uint16_t*>(row + L.o2);
  }
  // the same bytes through a buffer resource over the row
  __device__ static void load(__amdgpu_buffer_rsrc_t rs, const BlockLane& L, Raw& r) {
    r.v = __builtin_amdgcn_raw_buffer_load_b128(rs, L.o16, 0, 0);
    r.s = __builtin_amdgcn_raw_buffer_load_b16(rs, L.o2, 0, 0);
  }
  // D * sum (c - 8) X (still to be scaled by 2^-s)
  __device__ static float apply(const Raw& r, const BlockLane& L, const XP& xp, int /*j*/,
                               Acc& ac) {
    uint32_t w[4];
    w[0] = perm_b32(r.v.y, r.v.x, L.sel) ^ 0x88888888u;
    w[1] = perm_b32(r.v.z, r.v.y, L.sel) ^ 0x88888888u;
    w[2] = perm_b32(r.v.w, r.v.z, L.sel) ^ 0x88888888u;
    w[3] = perm_b32(r.s, r.v.w, L.sel) ^ 0x88888888u;
    return f16_bits_to_f32(L.mis ? r.s : r.v.x) * (float)nib_dot(w, xp, ac);
  }
};

// ------------------------------------------------------------------ Q8_0 --
// 34-byte blocks: fp16 scale, 32 int8; weight = d * q.
struct FmtQ8_0 {
  static constexpr int kBytes = 34;
  static constexpr int kLoads = 3;
  typedef XByte XP;
  typedef ByteAcc Acc;
  struct Raw {
    u32x4 v0, v1;
    uint16_t s;
  };
  static constexpr bool kSum = false;
  __host__ __device__ static int64_t row_bytes(int64_t K) { return (K >> 5) * 34; }
  __device__ static BlockLane lane(int j, uint32_t p) {
    return block_lane((uint32_t)j * 34u, p, 34);
  }
  __device__ static void prep(f32x4 (&v)[8], XP& xp) { prep_byte(v, xp, false); }
  __device__ static void load(const uint8_t* __restrict__ row, const BlockLane& L, Raw& r) {
    r.v0 = *reinterpret_cast<const u32x4_a4*>(row + L.o16);
    r.v1 = *reinterpret_cast<const u32x4_a4*>(row + L.o16 + 16);
    r.s = *reinterpret_cast<const uint16_t*>(row + L.o2);
  }
  __device__ static void load(__amdgpu_buffer_rsrc_t rs, const BlockLane& L, Raw& r) {
    r.v0 = __builtin_amdgcn_raw_buffer_load_b128(rs, L.o16, 0, 0);
    r.v1 = __builtin_amdgcn_raw_buffer_load_b128(rs, L.o16 + 16u, 0, 0);
    r.s = __builtin_amdgcn_raw_buffer_load_b16(rs, L.o2, 0, 0);
  }
  __device__ static float apply(const Raw& r, const BlockLane& L, const XP& xp, int /*j*/,
                               Acc& ac) {
    const uint32_t w[9] = {r.v0.x, r.v0.y, r.v0.z, r.v0.w, r.v1.x, r.v1.y, r.v1.z, r.v1.w, r.s};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t q = perm_b32(w[i + 1], w[i], L.sel);  // q[4i..4i+3], int8
      ac.l = sdot4(q, xp.xl[i], ac.l);
      ac.h = sdot4(q, xp.xh[i], ac.h);
      ac.t = sdot4(q, xp.xt[i], ac.t);
    }
    // combined modulo 2^32 (sum q X itself fits in int32)
    const uint32_t tot = ((uint32_t)ac.t * 256u + (uint32_t)ac.h) * 256u + (uint32_t)ac.l;
    const int32_t S = (int32_t)(tot - ac.prev);
    ac.prev = tot;
    return f16_bits_to_f32(L.mis ? r.s : r.v0.x) * (float)S;  // D * sum q X
  }
};

// ------------------------------------------------------------------ Q4_K --
// 144-byte superblocks (16-byte aligned whenever the buffer is): header
// (d, dmin, 96-bit field word) then 8 x 16 code bytes. Slice j is sub-block
// j % 8 of superblock j / 8; weight = (d sc) q - (dmin mn).
struct FmtQ4_K {
  static constexpr int kBytes = 144;
  static constexpr int kLoads = 2;
  typedef XNib XP;
  typedef NibAcc Acc;
  struct Raw {
    u32x4 h, c;
  };
  static constexpr bool kSum = true;
  __host__ __device__ static int64_t row_bytes(int64_t K) { return (K >> 8) * 144; }
  // the superblock header and the sub-block's 16 code bytes (rows are
  // 16-byte aligned: p is 0)
  __device__ static BlockLane lane(int j, uint32_t /*p*/) {
    BlockLane L;
    const uint32_t o = (uint32_t)(j >> 3) * 144u;
    L.o16 = o;
    L.o2 = o + 16u + 16u * (uint32_t)(j & 7);
    L.sel = 0;
    L.mis = false;
    L.o8 = L.od = 0;
    return L;
  }
  __device__ static void prep(f32x4 (&v)[8], XP& xp) { prep_nib(v, xp, true); }
  __device__ static void load(const uint8_t* __restrict__ row, const BlockLane& L, Raw& r) {
    r.h = *reinterpret_cast<const u32x4*>(row + L.o16);
    r.c = *reinterpret_cast<const u32x4*>(row + L.o2);
  }
  __device__ static void load(__amdgpu_buffer_rsrc_t rs, const BlockLane& L, Raw& r) {
    r.h = __builtin_amdgcn_raw_buffer_load_b128(rs, L.o16, 0, 0);
    r.c = __builtin_amdgcn_raw_buffer_load_b128(rs, L.o2, 0, 0);
  }
  __device__ static float apply(const Raw& r, const BlockLane& /*L*/, const XP& xp, int j,
                               Acc& ac) {
    const int sub = j & 7;
    // 6-bit fields: sc at bit 6*sub, mn at bit 48 + 6*sub of {w, z, y}
    const int ps = 6 * sub, pm = 48 + 6 * sub;
    const uint32_t slo = ps < 32 ? r.h.y : r.h.z, shi = ps < 32 ? r.h.z : r.h.w;
    const uint32_t mlo = pm < 64 ? r.h.z : r.h.w, mhi = pm < 64 ? r.h.w : 0u;
    const uint32_t sc = __builtin_amdgcn_alignbit(shi, slo, ps & 31) & 63u;
    const uint32_t mn = __builtin_amdgcn_alignbit(mhi, mlo, pm & 31) & 63u;
    const float S = f16_bits_to_f32(r.h.x) * (float)sc;
    const float O = f16_bits_to_f32(r.h.x >> 16) * (float)mn;
    const uint32_t w[4] = {r.c.x ^ 0x88888888u, r.c.y ^ 0x88888888u, r.c.z ^ 0x88888888u,
                           r.c.w ^ 0x88888888u};
    // sum q X = sum (q - 8) X + 8 sum X
    const int32_t Q8 = nib_dot(w, xp, ac);
    return fmaf(S, (float)Q8, fmaf(8.0f, S, -O) * (float)xp.sx);
  }
};

// ------------------------------------------------------------------ Q6_K --
// 210-byte superblocks: fp16 d, then per 32-weight group g (slice j = 8 s +
// g of superblock s) 26 bytes at 2 + 26 g: int8 scales of sub-blocks 2g and
// 2g+1, 16 bytes of low nibbles (byte t: code t | code 16+t), high-bit
// words H0, H1 (bits 2w..2w+1 of byte b: code 4w+b, code 16+4w+b).
// weight = d sc_j (c - 32). A lane loads its group as 16 + 8 + 2 bytes at
// 4-byte-aligned offsets (which pieces depends on the group's alignment)
// plus d, realigns with one v_perm selector, rebuilds the 6-bit codes as
// bytes and takes exact byte-digit dot products per 16-weight half:
// sum (c - 32) X = sum c X - 32 sum X, the half sums of X coming with the
// converted activations.
struct ByteAcc2 {
  ByteAcc h[2];
};

struct FmtQ6_K {
  static constexpr int kBytes = 210;
  static constexpr int kLoads = 4;
  static constexpr bool kSum = true;
  typedef XByte XP;
  typedef ByteAcc2 Acc;
  struct Raw {
    u32x4 v;
    uint32_t u0, u1;
    uint16_t s;  // widened where it is used, after the load has landed
    uint16_t d;
  };
  __host__ __device__ static int64_t row_bytes(int64_t K) { return (K >> 8) * 210; }
  __device__ static void prep(f32x4 (&v)[8], XP& xp) { prep_byte(v, xp, true); }
  // group bytes [G, G + 26): if G is 4-byte aligned, 16 bytes at G, 8 at
  // G + 16, 2 at G + 24; else 2 at G, 16 at G + 2, 8 at G + 18
  __device__ static BlockLane lane(int j, uint32_t p) {
    BlockLane L;
    const uint32_t sb = (uint32_t)(j >> 3) * 210u, G = sb + 2u + 26u * (uint32_t)(j & 7);
    L.mis = ((G + p) & 2u) != 0;
    L.o16 = L.mis ? G + 2u : G;
    L.o8 = L.mis ? G + 18u : G + 16u;
    L.o2 = L.mis ? G : G + 24u;
    L.od = sb;
    L.sel = L.mis ? 0x03020100u : 0x05040302u;
    return L;
  }
  __device__ static void load(const uint8_t* __restrict__ row, const BlockLane& L, Raw& r) {
    r.v = *reinterpret_cast<const u32x4_a4*>(row + L.o16);
    r.u0 = *reinterpret_cast<const uint32_t*>(row + L.o8);
    r.u1 = *reinterpret_cast<const uint32_t*>(row + L.o8 + 4);
    r.s = *reinterpret_cast<const uint16_t*>(row + L.o2);
    r.d = *reinterpret_cast<const uint16_t*>(row + L.od);
  }
  __device__ static void load(__amdgpu_buffer_rsrc_t rs, const BlockLane& L, Raw& r) {
    r.v = __builtin_amdgcn_raw_buffer_load_b128(rs, L.o16, 0, 0);
    const uint2 u = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, L.o8, 0, 0));
    r.u0 = u.x;
    r.u1 = u.y;
    r.s = __builtin_amdgcn_raw_buffer_load_b16(rs, L.o2, 0, 0);
    r.d = __builtin_amdgcn_raw_buffer_load_b16(rs, L.od, 0, 0);
  }
  __device__ static float apply(const Raw& r, const BlockLane& L, const XP& xp, int /*j*/,
                               Acc& ac) {
    // the group's words: 16 nibble bytes N, then H0, H1; in the aligned
    // case they start 2 bytes into the loaded words, after the scales
    const uint32_t x[7] = {r.v.x, r.v.y, r.v.z, r.v.w, r.u0, r.u1, (uint32_t)r.s};
    uint32_t N[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) N[k] = perm_b32(x[k + 1], x[k], L.sel);
    const uint32_t H[2] = {perm_b32(x[5], x[4], L.sel), perm_b32(x[6], x[5], L.sel)};
    const uint32_t scw = L.mis ? (uint32_t)r.s : r.v.x;
    const float sc[2] = {(float)(int8_t)(scw & 0xFFu), (float)(int8_t)((scw >> 8) & 0xFFu)};
    float out = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ByteAcc& a = ac.h[h];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // codes of elements 16h + 4w .. 16h + 4w + 3 as bytes 0..63
        const uint32_t lo = h ? (N[w] >> 4) & 0x0F0F0F0Fu : N[w] & 0x0F0F0F0Fu;
        const uint32_t c = lo | (((H[h] >> (2 * w)) & 0x03030303u) << 4);
        a.l = sdot4(c, xp.xl[4 * h + w], a.l);
        a.h = sdot4(c, xp.xh[4 * h + w], a.h);
        a.t = sdot4(c, xp.xt[4 * h + w], a.t);
      }
      const uint32_t tot = ((uint32_t)a.t * 256u + (uint32_t)a.h) * 256u + (uint32_t)a.l;
      const int32_t S = (int32_t)(tot - a.prev) - 32 * xp.sxh[h];  // sum (c - 32) X
      a.prev = tot;
      out = fmaf(sc[h], (float)S, out);
    }
    return f16_bits_to_f32(r.d) * out;
  }
};

// Cross-lane exchange at distance `mask` (32, 16, 8, 4, 2 or 1), all in
// VALU: v_permlane32_swap / v_permlane16_swap swap the upper half of the
// first operand with the lower half of the second (lanes 32-63 <-> 0-31, or
// odd <-> even rows of 16), and DPP moves read a partner lane within a row
// of 16 (row_ror:8 is lane ^ 8; row_half_mirror pairs lane i with 7 - i
// inside each group of 8, which also crosses bit 2; quad_perm gives ^2, ^1).
//
// halve(mask, a, b): lanes whose `mask` bit is clear return a + partner's a,
// the others b + partner's b.
template <int kMask>
__device__ __forceinline__ float dpp_other(float v) {
  static_assert(kMask == 8 || kMask == 4 || kMask == 2 || kMask == 1, "DPP partner");
  // row_ror:8, row_half_mirror, quad_perm [2,3,0,1], quad_perm [1,0,3,2]
  constexpr int kCtrl = kMask == 8 ? 0x128 : kMask == 4 ? 0x141 : kMask == 2 ? 0x4E : 0xB1;
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}

template <int kMask>
__device__ __forceinline__ float halve(float a, float b, int lane) {
  if constexpr (kMask == 32 || kMask == 16) {
    // after the swap the first result holds a on the low side and the
    // partner's b on the high side, the second the partner's a on the low
    // side and b on the high side
    const auto r = kMask == 32
                       ? __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a),
                                                          __builtin_bit_cast(uint32_t, b), false,
                                                          false)
                       : __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, a),
                                                          __builtin_bit_cast(uint32_t, b), false,
                                                          false);
    // bit-cast the whole pair: a bit-cast of one subscripted element would
    // read element 0
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 f = __builtin_bit_cast(f32x2, r);
    return f.x + f.y;
  } else {
    const bool up = (lane & kMask) != 0;
    const float keep = up ? b : a, send = up ? a : b;
    return keep + dpp_other<kMask>(send);
  }
}

// Reduction of R per-lane values over the wave: every exchange sends the
// half of the live values that the partner keeps (R/2 + R/4 + ... + 1
// exchanges), then the groups left holding one row are summed. On return
// lane l holds the wave sum of row (l >> (6 - log2 R)) & (R - 1).
template <int kMask, int kHalf, int R>
__device__ __forceinline__ void reduce_level(float (&v)[R], int lane) {
  if constexpr (kMask >= 1) {
    if constexpr (kHalf >= 1) {
#pragma unroll
      for (int i = 0; i < kHalf; ++i) v[i] = halve<kMask>(v[i], v[i + kHalf], lane);
      reduce_level<kMask / 2, kHalf / 2, R>(v, lane);
    } else {
      v[0] = halve<kMask>(v[0], v[0], lane);
      reduce_level<kMask / 2, 0, R>(v, lane);
    }
  }
}

template <int R>
__device__ __forceinline__ float wave_reduce_rows(float (&v)[R], int lane) {
  reduce_level<32, R / 2, R>(v, lane);
  return v[0];
}

template <int R>
constexpr int log2i() {
  return R <= 1 ? 0 : 1 + log2i<R / 2>();
}

// The activation slices of a strip go through LDS: 64 slices x 128 bytes
// per wave, written by direct global->LDS loads (each instruction moves 1 KB,
// 16 bytes per lane) so that no lane's registers wait on them, and read back
// one slice per lane. Slice s keeps its 16-byte part k in column
// (k + s) mod 8 of its 128-byte row, so the eight lanes of one LDS access
// phase read eight different columns (no bank conflicts).
constexpr int kXStripBytes = kWave * 128;


__device__ __forceinline__ void x_to_lds(const float* __restrict__ xs, int nsl, uint8_t* strip,
                                         int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int s = 8 * i + (lane >> 3);  // slice filled by this lane's column
    const int k = (lane - s) & 7;       // its part stored in column lane & 7
    if (s < nsl)
      __builtin_amdgcn_global_load_lds(xs + 32 * s + 4 * k, (lds_ptr_t)(strip + 1024 * i), 16, 0,
                                       0);
  }
}

__device__ __forceinline__ void x_from_lds(const uint8_t* strip, int lane, f32x4 (&v)[8]) {
  const uint8_t* row = strip + 128 * lane;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    v[k] = *reinterpret_cast<const f32x4*>(row + 16 * ((k + lane) & 7));
}

// A workgroup owns G groups of R rows, D groups of loads in flight per
// wave. kOdd: the row stride is 2 mod 4
// (K/32 odd for Q4_0/Q8_0), so even and odd rows have different block
// alignments; row m0 + r has parity r & 1 since m0 and the group size are
// even.
// kPair (rows of at most 32 slices, one strip): each half of the wave takes
// its own G x R rows, lane l working on slice l & 31, so that no lane idles;
// the workgroup then owns 2 x G x R rows.
// The body of the strip kernel for workgroup `wg` of one matrix (rows
// wg * kRows ..); the workgroup's waves split K into strips. Waves past the
// matrix's strips add nothing.
template <int R, int G, bool kPair>
constexpr int strip_rows() {
  return kPair ? 2 * R * G : R * G;
}

template <class F, int R, int G, int D, bool kOdd, bool kPair>
__device__ __forceinline__ void gemv_strips(const uint8_t* __restrict__ B,
                                            const float* __restrict__ x, float* __restrict__ y,
                                            int64_t M, int K, int64_t wg, uint8_t* xlds,
                                            float (*red)[strip_rows<R, G, kPair>()]) {
  constexpr int RG = R * G;
  constexpr int kRows = strip_rows<R, G, kPair>();
  static_assert(kRows <= kWave && (RG & (RG - 1)) == 0, "rows per workgroup");
  static_assert(D >= 1 && D <= G, "groups in flight");
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int ns = K >> 5;
  const int64_t rb = F::row_bytes(K);
  const int64_t m0 = wg * kRows;
  // the slice lane and the first row of this lane's half (RG is even, so
  // row parity is still r & 1)
  const int sl = kPair ? (lane & 31) : lane;
  const int64_t mh = kPair ? m0 + (lane >> 5) * RG : m0;
  uint8_t* strip = xlds + wv * kXStripBytes;

  float part[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) part[r] = 0.0f;

  for (int base = wv * kWave; base < ns; base += nw * kWave) {
    const int j = base + sl;
    x_to_lds(x + (int64_t)base * 32, ns - base, strip, lane);
    if (j < ns) {
      BlockLane L[2];
      L[0] = F::lane(j, 0u);
      L[1] = F::lane(j, kOdd ? 2u : 0u);
      typename F::Raw raw[D][R];
      auto load_group = [&](int g, typename F::Raw(&dst)[R]) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          // rows past M re-read the last row of the same parity (their
          // sums are discarded); with an odd stride M >= 2 here
          int64_t m = mh + g * R + r;
          if (m >= M) m = kOdd ? M - 1 - ((M - 1 - r) & 1) : M - 1;
          F::load(B + m * rb, L[kOdd ? (r & 1) : 0], dst[r]);
        }
      };
      // D groups are in flight from the start, so the activation
      // conversion below overlaps them; group g + D is requested as soon as
      // group g has been consumed.
#pragma unroll
      for (int g = 0; g < D; ++g) load_group(g, raw[g]);
      // Memory loads complete in issue order, so once no more than the
      // weight loads of those D groups are outstanding, every activation
      // load issued before them has landed in LDS. (The compiler does not
      // track direct-to-LDS loads, hence the explicit wait.)
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm<D * R * F::kLoads>());
      __builtin_amdgcn_sched_barrier(0);
      f32x4 xv[8];
      x_from_lds(strip, sl, xv);
      typename F::XP xp;
      F::prep(xv, xp);
      typename F::Acc ac = {};
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int r = 0; r < R; ++r)
          part[g * R + r] = fmaf(F::apply(raw[g % D][r], L[kOdd ? (r & 1) : 0], xp, j, ac),
                                 xp.inv, part[g * R + r]);
        if (g + D < G) {
          __builtin_amdgcn_sched_barrier(0);
          load_group(g + D, raw[g % D]);
        }
      }
    }
  }

  if constexpr (kPair) {
    // each half reduces its own rows (exchanges within 32 lanes)
    static_assert(RG <= 32, "rows per half");
    constexpr int kShift = 5 - log2i<RG>();
    reduce_level<16, RG / 2, RG>(part, lane);
    const int row = (lane >> 5) * RG + ((lane >> kShift) & (RG - 1));
    if ((lane & ((1 << kShift) - 1)) == 0) red[wv][row] = part[0];
  } else {
    constexpr int kShift = 6 - log2i<RG>();
    const int row = (lane >> kShift) & (RG - 1);
    const float sum = wave_reduce_rows<RG>(part, lane);
    if ((lane & ((1 << kShift) - 1)) == 0) red[wv][row] = sum;
  }
  __syncthreads();
  if ((int)threadIdx.x < kRows) {
    float t = 0.0f;
    for (int w = 0; w < nw; ++w) t += red[w][threadIdx.x];
    if (m0 + threadIdx.x < M) y[m0 + threadIdx.x] = t;
  }
}

template <class F, int R, int G, int D, bool kOdd, bool kPair>
__global__ __launch_bounds__(kMaxStrips * kWave) void gemv_kernel(const uint8_t* __restrict__ B,
                                                                  const float* __restrict__ x,
                                                                  float* __restrict__ y,
                                                                  int64_t M, int K) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xlds[];
  __shared__ float red[kPair ? 1 : kMaxStrips][strip_rows<R, G, kPair>()];
  gemv_strips<F, R, G, D, kOdd, kPair>(B, x, y, M, K, blockIdx.x, xlds, red);
}

// Many independent GEMVs in one launch: job blockIdx.y, its workgroup
// blockIdx.x. Each job's pointers and sizes travel in the kernel arguments;
// workgroups past a job's rows end at once. The jobs of one launch share the
// row-stride parity, the pair mode and the number of strips.
constexpr int kBatchJobs = 96;  // 3.4 KB of kernel arguments
struct GemvBatchArgs {
  const uint8_t* B[kBatchJobs];
  const float* x[kBatchJobs];
  float* y[kBatchJobs];
  int64_t M[kBatchJobs];
  int K[kBatchJobs];
};

template <class F, int R, int G, int D, bool kOdd, bool kPair>
__global__ __launch_bounds__(kMaxStrips * kWave) void gemv_batch_kernel(GemvBatchArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xlds[];
  constexpr int kRows = strip_rows<R, G, kPair>();
  __shared__ float red[kPair ? 1 : kMaxStrips][kRows];
  const int j = blockIdx.y;
  const int64_t M = a.M[j];
  if ((int64_t)blockIdx.x * kRows >= M) return;  // the whole workgroup
  gemv_strips<F, R, G, D, kOdd, kPair>(a.B[j], a.x[j], a.y[j], M, a.K[j], blockIdx.x, xlds, red);
}

// -------------------------------------------------- GEMV, a row per wave --
// A workgroup of kRowWaves waves owns kRowWaves rows, one per wave, and all
// of K (at most kRowMaxSlices slices, kRowMaxStrips strips of 64). LDS holds one 8 KB
// slot per strip. At the start, wave w copies strip w of the activations
// from memory into slot w (all copies ahead of any weight load), requests
// the weight blocks of its row's first kD strips, and then converts the slot
// in place into digit records (one lane per slice, as in gemv_kernel),
// shared by all the rows, and raises the slot's ready flag. Each wave
// streams its row strip by strip (lane = slice) and waits only for the flag
// of the strip it is about to use, not for the whole workgroup: the
// converting waves run at raised priority, and the blocks of kD strips stay
// in flight in kD register buffers that an unrolled loop rotates.
//
// Every weight load is issued on every lane and path: lanes out of range
// read past the end of their buffer resource, which returns zeros without a
// memory access. Zero blocks have scale 0 and the records of the padding
// slices have inv = 0, so those lanes add exactly 0 and need no branch. This
// keeps the compiler's load counting exact (a load skipped on some path
// makes every later wait a full one).
#ifndef QMAT_GEMV_ROW_WAVES
#define QMAT_GEMV_ROW_WAVES 16
#define QMAT_GEMV_ROW_R 1
#endif
// strips of weight blocks in flight per wave (measured best at 4096x11008;
// more in flight lengthens the queues that the slowest workgroups wait in)
#ifndef QMAT_GEMV_ROW_DEPTH_Q4_0
#define QMAT_GEMV_ROW_DEPTH_Q4_0 1
#define QMAT_GEMV_ROW_DEPTH_Q8_0 1
#define QMAT_GEMV_ROW_DEPTH_Q4_K 2
#define QMAT_GEMV_ROW_DEPTH_Q6_K 1
#endif
constexpr int kRowWaves = QMAT_GEMV_ROW_WAVES;
constexpr int kRowSlot = 8192;  // one strip of fp32 activations
// A wait for a ready flag gives up after this many polls (each with a short
// sleep, some tens of milliseconds in all) instead of hanging the device if
// a flag were never raised; the flags are raised unconditionally. A wave
// that gave up writes NaN to its rows, so the failure cannot pass as a
// plausible result.
constexpr int kRowSpinLimit = 1 << 20;

// LDS flags as relaxed workgroup-scope atomics: read afresh on every poll
// but, unlike volatile accesses, without a wait for all outstanding memory
// operations; the ordering with the records comes from explicit waits.
__device__ __forceinline__ void flag_set(int* f, int v) {
  __hip_atomic_store(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ int flag_get(int* f) {
  return __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
#ifndef QMAT_GEMV_ROW_STRIPS
#define QMAT_GEMV_ROW_STRIPS 8
#endif
// Strips (LDS slots) of the longest row the kernel takes, at most one per
// wave (wave w converts strip w). The slots are dynamic LDS, so 16 (128 KB)
// would fit; measured against the strip kernel on rows of 640 to 1024
// slices, 16 won only where the grid is one workgroup per CU (Q4_0
// 4096 x 20480: 11.4 against 12.7 us) and tied or lost elsewhere (8192 x
// 28672: Q4_0 30.9 against 32.6, Q4_K-style 32.0 against 30.5; 2048 x 32768:
// 14.6 against 11.1 with half the CUs idle), so longer rows stay with the
// strip kernel.
constexpr int kRowMaxStrips = QMAT_GEMV_ROW_STRIPS;
constexpr int kRowMaxSlices = kRowMaxStrips * kWave;
static_assert(kRowWaves >= kRowMaxStrips, "wave w converts strip w");

// Records of the 64 slices of a slot (they replace the activations). Nibble
// digits: word t of digit i of slice l at byte 1024 i + 16 l + 4 t (a lane
// reads consecutive 16-byte groups), inv at 5120 + 4 l, sx at 5376 + 4 l.
// Byte digits: words 4h..4h+3 of kind j (xl, xh, xt) at 1024 (2j + h) +
// 16 l, inv at 6144 + 4 l, half sums of X (Q6_K) at 6400 + 4 l, 6656 + 4 l.
__device__ __forceinline__ void put_rec(uint8_t* slot, int l, const XNib& xp, bool sum) {
#pragma unroll
  for (int i = 0; i < 5; ++i)
    *reinterpret_cast<u32x4*>(slot + 1024 * i + 16 * l) =
        u32x4{xp.d[i][0], xp.d[i][1], xp.d[i][2], xp.d[i][3]};
  reinterpret_cast<float*>(slot + 5120)[l] = xp.inv;
  if (sum) reinterpret_cast<int32_t*>(slot + 5376)[l] = xp.sx;
}

__device__ __forceinline__ void get_rec(const uint8_t* slot, int l, XNib& xp, bool sum) {
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(slot + 1024 * i + 16 * l);
    xp.d[i][0] = v.x;
    xp.d[i][1] = v.y;
    xp.d[i][2] = v.z;
    xp.d[i][3] = v.w;
  }
  xp.inv = reinterpret_cast<const float*>(slot + 5120)[l];
  xp.sx = sum ? reinterpret_cast<const int32_t*>(slot + 5376)[l] : 0;
}

__device__ __forceinline__ void put_rec(uint8_t* slot, int l, const XByte& xp, bool sum) {
  const uint32_t* src[3] = {xp.xl, xp.xh, xp.xt};
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      *reinterpret_cast<u32x4*>(slot + 1024 * (2 * j + h) + 16 * l) =
          u32x4{src[j][4 * h], src[j][4 * h + 1], src[j][4 * h + 2], src[j][4 * h + 3]};
  reinterpret_cast<float*>(slot + 6144)[l] = xp.inv;
  if (sum) {
    reinterpret_cast<int32_t*>(slot + 6400)[l] = xp.sxh[0];
    reinterpret_cast<int32_t*>(slot + 6656)[l] = xp.sxh[1];
  }
}

__device__ __forceinline__ void get_rec(const uint8_t* slot, int l, XByte& xp, bool sum) {
  uint32_t* dst[3] = {xp.xl, xp.xh, xp.xt};
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(slot + 1024 * (2 * j + h) + 16 * l);
      dst[j][4 * h + 0] = v.x;
      dst[j][4 * h + 1] = v.y;
      dst[j][4 * h + 2] = v.z;
      dst[j][4 * h + 3] = v.w;
    }
  xp.inv = reinterpret_cast<const float*>(slot + 6144)[l];
  xp.sx = 0;
  xp.sxh[0] = sum ? reinterpret_cast<const int32_t*>(slot + 6400)[l] : 0;
  xp.sxh[1] = sum ? reinterpret_cast<const int32_t*>(slot + 6656)[l] : 0;
}

// The body for workgroup wg of one matrix (rows from wg * kRowWaves * R).
template <class F, int R, int kD, bool kOdd>
__device__ __forceinline__ void gemv_rows(const uint8_t* __restrict__ B,
                                          const float* __restrict__ x, float* __restrict__ y,
                                          int64_t M, int K, int64_t wg, uint8_t* slots,
                                          int* ready) {
  // strip s's records are in slot s when ready[s] != 0
  typedef typename F::XP XP;
  constexpr uint32_t kOut = 0x80000000u;  // an offset past the end of any row
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int ns = K >> 5;
  const int nstrips = (ns + kWave - 1) / kWave;
  const int64_t rb = F::row_bytes(K);
  const int64_t m0 = (wg * kRowWaves + wv) * R;  // this wave's first row
  // with an odd row stride, row m starts at 2 (m & 1) mod 4; a row past M
  // re-reads the last row of the same parity (M >= 2 then)
  __amdgpu_buffer_rsrc_t rrs[R];
  uint32_t par[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t m = m0 + r;
    par[r] = kOdd ? (uint32_t)(m & 1) : 0u;
    const int64_t mr = m < M ? m : (kOdd ? M - 1 - ((M - 1 - (int64_t)par[r]) & 1) : M - 1);
    rrs[r] = make_rsrc(B + mr * rb, rb);
  }

  // LDS holds whatever the last workgroup left: clear the flags first
  if (threadIdx.x < kRowMaxStrips) flag_set(&ready[threadIdx.x], 0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // strip wv of the activations into slot wv, first among this wave's loads
  const bool conv = wv < nstrips;
  uint8_t* const own = slots + wv * kRowSlot;
  if (conv) __builtin_amdgcn_s_setprio(2);
  if (conv) x_to_lds(x + (int64_t)wv * kWave * 32, min(ns - wv * kWave, kWave), own, lane);
  // every wave's weight loads queue behind all of the copies
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  auto lane_of = [&](int st, uint32_t p) { return F::lane(st * kWave + lane, 2u * p); };
  typename F::Raw wb[kD][R];
  auto load_w = [&](int st, typename F::Raw (&dst)[R]) {
    const bool ok = st < nstrips && st * kWave + lane < ns;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      BlockLane L = lane_of(st, par[r]);
      if (!ok) L.o16 = L.o2 = L.o8 = L.od = kOut;
      F::load(rrs[r], L, dst[r]);
    }
  };
  // strip by strip, in the order the loop below counts them
#pragma unroll
  for (int u = 0; u < kD; ++u) {
    load_w(u, wb[u]);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Loads complete in issue order: with only the weight loads left, the
  // copy has landed. Every wave waits (a no-op without a copy), so that on
  // no path does the compiler see copies into LDS still in flight, which
  // would make it wait for all loads before each LDS read in the loop.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm<kD * R * F::kLoads>());
  __builtin_amdgcn_sched_barrier(0);
  if (conv) {
    f32x4 v[8];
    x_from_lds(own, lane, v);
    XP xp;
    F::prep(v, xp);
    if (wv * kWave + lane >= ns) xp.inv = 0.0f;  // padding slice
    put_rec(own, lane, xp, F::kSum);
    // records first (LDS completes a wave's accesses in order once waited
    // for), then the flag; the memory clobbers keep the compiler's LDS
    // accesses on their side
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (lane == 0) flag_set(&ready[wv], 1);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_setprio(0);
  }

  typename F::Acc ac = {};
  float part[R];
#pragma unroll
  for (int r = 0; r < R; ++r) part[r] = 0.0f;
  bool lost = false;  // a flag wait gave up
  // strip st from buffer w, then (if `next`) strip st + kD into w
  auto step = [&](int st, typename F::Raw (&w)[R], bool next) {
    const int j = st * kWave + lane;
    int n = 0;
    for (; flag_get(&ready[st]) == 0 && n < kRowSpinLimit; ++n) __builtin_amdgcn_s_sleep(1);
    lost |= n == kRowSpinLimit;
    asm volatile("" ::: "memory");
    XP xp;
    get_rec(slots + st * kRowSlot, lane, xp, F::kSum);
#pragma unroll
    for (int r = 0; r < R; ++r)
      part[r] = fmaf(F::apply(w[r], lane_of(st, par[r]), xp, j, ac), xp.inv, part[r]);
    if (next) load_w(st + kD, w);
    // the next strip's arithmetic must not move above these loads
    __builtin_amdgcn_sched_barrier(0);
  };
  // Whole rounds of kD strips while every strip they request exists:
  // no path through this loop skips a load, so each wait counts exactly the
  // loads after it. The last kD to 2 kD - 1 strips request only what
  // exists (their waits may be full ones: nothing is left to overlap).
  int s0 = 0;
  for (; s0 + 2 * kD <= nstrips; s0 += kD) {
#pragma unroll
    for (int u = 0; u < kD; ++u) step(s0 + u, wb[u], true);
  }
#pragma unroll
  for (int u = 0; u < kD; ++u)
    if (s0 + u < nstrips) step(s0 + u, wb[u], s0 + u + kD < nstrips);
#pragma unroll
  for (int u = 0; u + 1 < kD; ++u)
    if (s0 + kD + u < nstrips) step(s0 + kD + u, wb[u], false);
  constexpr int kShift = 6 - log2i<R>();
  const int r = (lane >> kShift) & (R - 1);
  const float sum = wave_reduce_rows<R>(part, lane);
  if ((lane & ((1 << kShift) - 1)) == 0 && m0 + r < M)
    y[m0 + r] = lost ? __builtin_nanf("") : sum;
}

template <class F, int R, int kD, bool kOdd>
__global__ __launch_bounds__(kRowWaves * kWave) void gemv_rows_kernel(
    const uint8_t* __restrict__ B, const float* __restrict__ x, float* __restrict__ y,
    int64_t M, int K) {
  extern __shared__ __attribute__((aligned(16))) uint8_t slots[];
  __shared__ int ready[kRowMaxStrips];
  gemv_rows<F, R, kD, kOdd>(B, x, y, M, K, blockIdx.x, slots, ready);
}

// Many GEMVs of the row kernel's shape in one launch: job blockIdx.y, its
// workgroup blockIdx.x (the jobs of a launch share the row-stride parity
// and the number of strips, which sizes the LDS); workgroups past a job's
// rows end at once.
template <class F, int R, int kD, bool kOdd>
__global__ __launch_bounds__(kRowWaves * kWave) void gemv_rows_batch_kernel(GemvBatchArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t slots[];
  __shared__ int ready[kRowMaxStrips];
  const int j = blockIdx.y;
  const int64_t M = a.M[j];
  if ((int64_t)blockIdx.x * kRowWaves * R >= M) return;  // the whole workgroup
  gemv_rows<F, R, kD, kOdd>(a.B[j], a.x[j], a.y[j], M, a.K[j], blockIdx.x, slots, ready);
}

#ifndef QMAT_GEMV_CFG
// rows per group, groups per workgroup, groups in flight
#define QMAT_GEMV_R_Q4_0 2
#define QMAT_GEMV_G_Q4_0 4
#define QMAT_GEMV_D_Q4_0 2
#define QMAT_GEMV_R_Q8_0 2
#define QMAT_GEMV_G_Q8_0 4
#define QMAT_GEMV_D_Q8_0 2
#define QMAT_GEMV_R_Q4_K 2
#define QMAT_GEMV_G_Q4_K 8
#define QMAT_GEMV_D_Q4_K 3
#define QMAT_GEMV_R_Q6_K 2
#define QMAT_GEMV_G_Q6_K 4
#define QMAT_GEMV_D_Q6_K 2
#endif

#ifndef QMAT_GEMV_ROWS
#define QMAT_GEMV_ROWS 1
#endif
// Which rows go to the row-per-wave kernel (measured crossovers against the
// strip kernel, Q4_0 / Q8_0 / Q4_K-style): from 128 slices up to
// kRowMaxSlices always (11008 x 4096: 8.1 against 8.7 us); from 32 slices in
// matrices of at most 8192 rows (4096 x 2048: 3.4 against 4.5 us; 1024 x
// 1024: 3.1 against 3.7), but not in taller ones, whose several workgroups
// per CU each repeat the activation conversion (11008 x 2048: 6.2 against
// 5.8 us; 16384 x 2048: 7.6 against 6.4).
constexpr int64_t kRowsMinSlices = 128;
constexpr int64_t kRowsShortMinSlices = 32;
constexpr int64_t kRowsShortMaxRows = 8192;
__host__ __device__ constexpr bool rows_kernel_takes(int64_t M, int64_t ns) {
  return QMAT_GEMV_ROWS && ns <= kRowMaxSlices &&
         (ns >= kRowsMinSlices || (ns >= kRowsShortMinSlices && M <= kRowsShortMaxRows));
}
// In a batch the row kernel takes only rows of 256 slices and more: on the
// Qwen3-like set (rows of 32 to 96 slices) batched row-kernel launches took
// 137.6 us against the strip kernel's 67.6 (Q4_0), each 16-row workgroup
// converting the activations for one or two strips of work per wave.
constexpr int64_t kBatchRowsMinSlices = 256;

// How the strip kernel covers a matrix: strips (waves) per workgroup, the
// row-stride parity and the pair mode.
struct StripShape {
  int waves;
  bool odd, pair;
  constexpr int64_t rows(int rg) const { return pair ? 2 * rg : rg; }
};

template <class F>
StripShape strip_shape(int64_t M, int64_t K) {
  const int64_t ns = K / 32;
  int waves = (int)((ns + kWave - 1) / kWave);
  if (waves < 1) waves = 1;
  if (waves > kMaxStrips) waves = kMaxStrips;
  // a single row has only the even parity: the aligned variant covers it
  const bool odd = (F::row_bytes(K) & 2) != 0 && M > 1;  // rows start 2 mod 4
  // rows of at most half a strip: both halves of the wave take rows
  return {waves, odd, ns <= kWave / 2 && M > 1};
}

template <class F, int RR, int RD>
hipError_t launch_rows(const void* blocks, const float* x, float* y, int64_t M, int64_t K,
                       hipStream_t stream) {
  const int64_t ns = K / 32;
  const int64_t grid = (M + kRowWaves * RR - 1) / (kRowWaves * RR);
  const size_t lds = (size_t)((ns + kWave - 1) / kWave) * kRowSlot;
  const bool odd = (F::row_bytes(K) & 2) != 0 && M > 1;  // rows start 2 mod 4
  if (odd)
    hipLaunchKernelGGL((gemv_rows_kernel<F, RR, RD, true>), dim3((unsigned)grid),
                       dim3(kRowWaves * kWave), lds, stream, static_cast<const uint8_t*>(blocks),
                       x, y, M, (int)K);
  else
    hipLaunchKernelGGL((gemv_rows_kernel<F, RR, RD, false>), dim3((unsigned)grid),
                       dim3(kRowWaves * kWave), lds, stream, static_cast<const uint8_t*>(blocks),
                       x, y, M, (int)K);
  return hipGetLastError();
}

// Two rows per wave (32 rows per workgroup) for the 4-bit formats in tall
// matrices: with one row per wave they would queue more than three 16-row
// workgroups per CU. Measured (one against two rows per wave): Q4_0 14336 x
// 4096 9.6 -> 8.4 us, 14336 x 8192 15.5 -> 14.7, 28672 x 4096 18.0 -> 15.1;
// Q4_K-style 14336 x 4096 12.6 -> 10.6, 28672 x 4096 21.7 -> 20.3; Q8_0 and
// Q6_K-style no better (11008 x 8192 Q8_0: 18.4 -> 21.8), nor shorter 4-bit
// matrices (Q4_0 4096 x 11008: 7.45 -> 9.42, 11008 x 8192: 13.2 -> 13.6).
constexpr int64_t kRows2MinM = 12288;

template <class F, int R, int G, int D, int RD>
hipError_t launch_fmt(const void* blocks, const float* x, float* y, int64_t M, int64_t K,
                      hipStream_t stream) {
  const int64_t ns = K / 32;
  if (rows_kernel_takes(M, ns)) {
    constexpr bool k4bit = F::kBytes == 18 || F::kBytes == 144;
    if (k4bit && QMAT_GEMV_ROW_R == 1 && M > kRows2MinM)
      return launch_rows<F, 2, RD>(blocks, x, y, M, K, stream);
    return launch_rows<F, QMAT_GEMV_ROW_R, RD>(blocks, x, y, M, K, stream);
  }
  const StripShape sh = strip_shape<F>(M, K);
  const int64_t grid = (M + sh.rows(R * G) - 1) / sh.rows(R * G);
  const dim3 block(sh.waves * kWave);
  const size_t lds = (size_t)sh.waves * kXStripBytes;
  const uint8_t* B = static_cast<const uint8_t*>(blocks);
  if (sh.odd && sh.pair)
    hipLaunchKernelGGL((gemv_kernel<F, R, G, D, true, true>), dim3((unsigned)grid), block, lds,
                       stream, B, x, y, M, (int)K);
  else if (sh.odd)
    hipLaunchKernelGGL((gemv_kernel<F, R, G, D, true, false>), dim3((unsigned)grid), block, lds,
                       stream, B, x, y, M, (int)K);
  else if (sh.pair)
    hipLaunchKernelGGL((gemv_kernel<F, R, G, D, false, true>), dim3((unsigned)grid), block, lds,
                       stream, B, x, y, M, (int)K);
  else
    hipLaunchKernelGGL((gemv_kernel<F, R, G, D, false, false>), dim3((unsigned)grid), block, lds,
                       stream, B, x, y, M, (int)K);
  return hipGetLastError();
}

// rows per group, groups per workgroup and groups in flight of the strip
// kernel inside a batch launch
#ifndef QMAT_BATCH_CFG
#define QMAT_BATCH_R_Q4_0 QMAT_GEMV_R_Q4_0
#define QMAT_BATCH_G_Q4_0 QMAT_GEMV_G_Q4_0
#define QMAT_BATCH_D_Q4_0 QMAT_GEMV_D_Q4_0
#define QMAT_BATCH_R_Q8_0 QMAT_GEMV_R_Q8_0
#define QMAT_BATCH_G_Q8_0 QMAT_GEMV_G_Q8_0
#define QMAT_BATCH_D_Q8_0 QMAT_GEMV_D_Q8_0
#define QMAT_BATCH_R_Q4_K QMAT_GEMV_R_Q4_K
#define QMAT_BATCH_G_Q4_K QMAT_GEMV_G_Q4_K
#define QMAT_BATCH_D_Q4_K QMAT_GEMV_D_Q4_K
#define QMAT_BATCH_R_Q6_K QMAT_GEMV_R_Q6_K
#define QMAT_BATCH_G_Q6_K QMAT_GEMV_G_Q6_K
#define QMAT_BATCH_D_Q6_K QMAT_GEMV_D_Q6_K
#endif

// A batch of GEMVs of one format, in launches of up to kBatchJobs jobs
// grouped so that every workgroup is sized for its own job: jobs with rows
// of 256 to 512 slices go to the row kernel, grouped by row-stride parity
// and strip count; the others to the strip kernel, grouped by parity and
// workgroup shape (pair mode, or the number of strips). A group of more than
// kBatchJobs jobs is split into launches of equal size (a small last launch
// is mostly ramp and tail: 12 of the Qwen3-like set's jobs took 6.9 us).
template <class F, int R, int G, int D, int RD>
hipError_t launch_batch_fmt(const GemvJob* jobs, int64_t count, hipStream_t stream) {
  constexpr int RG = R * G;
  constexpr int RR = QMAT_GEMV_ROW_R;
  constexpr int kShapes = kMaxStrips + 1;  // strip kernel: 0 pair mode, w: w strips
  constexpr int kRowShapes = kRowMaxSlices / kWave + 1;  // row kernel: strips
  struct Group {
    GemvBatchArgs a;
    int n;
    int64_t tiles;
  };
  static_assert(sizeof(Group) < 4096, "batch group");
  Group grp[2][kShapes];
  Group rgrp[2][kRowShapes];
  for (auto& go : grp)
    for (auto& g : go) g.n = 0, g.tiles = 0;
  for (auto& go : rgrp)
    for (auto& g : go) g.n = 0, g.tiles = 0;
  // jobs per launch of each group: its jobs over as few launches as allowed
  int per[2][kShapes], rper[2][kRowShapes];
  {
    int64_t cnt[2][kShapes] = {}, rcnt[2][kRowShapes] = {};
    for (int64_t i = 0; i < count; ++i) {
      const GemvJob& jb = jobs[i];
      if (jb.M == 0) continue;
      const int64_t ns = jb.K / 32;
      if (QMAT_GEMV_ROWS && ns >= kBatchRowsMinSlices && ns <= kRowMaxSlices) {
        ++rcnt[((F::row_bytes(jb.K) & 2) != 0 && jb.M > 1) ? 1 : 0][(ns + kWave - 1) / kWave];
      } else {
        const StripShape sh = strip_shape<F>(jb.M, jb.K);
        ++cnt[sh.odd ? 1 : 0][sh.pair ? 0 : sh.waves];
      }
    }
    auto chunk = [](int64_t c) {
      const int64_t launches = (c + kBatchJobs - 1) / kBatchJobs;
      return launches > 0 ? (int)((c + launches - 1) / launches) : kBatchJobs;
    };
    for (int o = 0; o < 2; ++o) {
      for (int w = 0; w < kShapes; ++w) per[o][w] = chunk(cnt[o][w]);
      for (int st = 0; st < kRowShapes; ++st) rper[o][st] = chunk(rcnt[o][st]);
    }
  }
  auto flush = [&](int o, int w) -> hipError_t {
    Group& g = grp[o][w];
    if (g.n == 0) return hipSuccess;
    const dim3 grid((unsigned)g.tiles, (unsigned)g.n);
    const int waves = w == 0 ? 1 : w;
    const dim3 block(waves * kWave);
    const size_t lds = (size_t)waves * kXStripBytes;
    if (o && w == 0)
      hipLaunchKernelGGL((gemv_batch_kernel<F, R, G, D, true, true>), grid, block, lds, stream,
                         g.a);
    else if (o)
      hipLaunchKernelGGL((gemv_batch_kernel<F, R, G, D, true, false>), grid, block, lds, stream,
                         g.a);
    else if (w == 0)
      hipLaunchKernelGGL((gemv_batch_kernel<F, R, G, D, false, true>), grid, block, lds, stream,
                         g.a);
    else
      hipLaunchKernelGGL((gemv_batch_kernel<F, R, G, D, false, false>), grid, block, lds, stream,
                         g.a);
    g.n = 0;
    g.tiles = 0;
    return hipGetLastError();
  };
  auto flush_rows = [&](int o, int st) -> hipError_t {
    Group& g = rgrp[o][st];
    if (g.n == 0) return hipSuccess;
    const dim3 grid((unsigned)g.tiles, (unsigned)g.n);
    const size_t lds = (size_t)st * kRowSlot;
    if (o)
      hipLaunchKernelGGL((gemv_rows_batch_kernel<F, RR, RD, true>), grid,
                         dim3(kRowWaves * kWave), lds, stream, g.a);
    else
      hipLaunchKernelGGL((gemv_rows_batch_kernel<F, RR, RD, false>), grid,
                         dim3(kRowWaves * kWave), lds, stream, g.a);
    g.n = 0;
    g.tiles = 0;
    return hipGetLastError();
  };
  auto add = [](Group& g, const GemvJob& jb, int64_t tiles) {
    const int k = g.n++;
    g.a.B[k] = static_cast<const uint8_t*>(jb.blocks);
    g.a.x[k] = jb.x;
    g.a.y[k] = jb.y;
    g.a.M[k] = jb.M;
    g.a.K[k] = (int)jb.K;
    g.tiles = tiles > g.tiles ? tiles : g.tiles;
  };
  for (int64_t i = 0; i < count; ++i) {
    const GemvJob& jb = jobs[i];
    if (jb.M == 0) continue;
    const int64_t ns = jb.K / 32;
    if (QMAT_GEMV_ROWS && ns >= kBatchRowsMinSlices && ns <= kRowMaxSlices) {
      const int o = ((F::row_bytes(jb.K) & 2) != 0 && jb.M > 1) ? 1 : 0;  // rows start 2 mod 4
      const int st = (int)((ns + kWave - 1) / kWave);
      Group& g = rgrp[o][st];
      add(g, jb, (jb.M + kRowWaves * RR - 1) / (kRowWaves * RR));
      if (g.n == rper[o][st]) {
        const hipError_t e = flush_rows(o, st);
        if (e != hipSuccess) return e;
      }
      continue;
    }
    const StripShape sh = strip_shape<F>(jb.M, jb.K);
    const int o = sh.odd ? 1 : 0;
    const int w = sh.pair ? 0 : sh.waves;
    Group& g = grp[o][w];
    add(g, jb, (jb.M + sh.rows(RG) - 1) / sh.rows(RG));
    if (g.n == per[o][w]) {
      const hipError_t e = flush(o, w);
      if (e != hipSuccess) return e;
    }
  }
  for (int o = 0; o < 2; ++o) {
    for (int st = 0; st < kRowShapes; ++st) {
      const hipError_t e = flush_rows(o, st);
      if (e != hipSuccess) return e;
    }
    for (int w = 0; w < kShapes; ++w) {
      const hipError_t e = flush(o, w);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// ------------------------------------------------ small-N decode GEMM --
// Y[n][m] = sum_k W[m][k] X[n][k] for a few tokens at once, X given as Q8_0
// blocks. As in the GEMV every weight block is read from memory once, but it
// is applied to NT tokens: the codes are unpacked to int8 once per block and
// multiplied with each token's int8 block by v_dot4_i32_i8 (exact), then
// scaled by the two fp16 block scales in fp32.
//
// A workgroup owns G waves x R rows and all of K; each wave walks K in strips
// of 64 slices (lane = slice). The activation records of a strip (NT tokens x
// 64 slices: 32 int8 codes, dx, and dx * sum(codes) for Q4_K-style) are
// unpacked once per workgroup into LDS and shared by its waves; the next
// strip's records and weight blocks are requested while the current strip is
// used, and its records go to the other LDS buffer afterwards.
#ifndef QMAT_SMALL_CFG
// rows per wave and waves per workgroup for 1-4, 8 and 16 tokens
#define QMAT_SMALL_R4 1
#define QMAT_SMALL_G4 16
#define QMAT_SMALL_R8 1
#define QMAT_SMALL_G8 16
#define QMAT_SMALL_R16 1
#define QMAT_SMALL_G16 16
#endif

// 32 int8 codes of a weight block in element order (word i = elements
// 4i..4i+3), its scale S and, for Q4_K-style, its offset O (weight = S q - O);
// for Q6_K-style S scales elements 0..15 and Sb elements 16..31.
struct WBlk {
  uint32_t w[8];
  float S, O, Sb;
};

__device__ __forceinline__ uint32_t nib_s8(uint32_t c, int sh) {
  return (((c >> sh) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;  // c - 8 per byte
}

__device__ __forceinline__ WBlk unpack_w(const FmtQ4_0::Raw& r, const BlockLane& L, int /*j*/) {
  WBlk b;
  const uint32_t c[4] = {perm_b32(r.v.y, r.v.x, L.sel), perm_b32(r.v.z, r.v.y, L.sel),
                         perm_b32(r.v.w, r.v.z, L.sel), perm_b32(r.s, r.v.w, L.sel)};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    b.w[i] = nib_s8(c[i], 0);      // elements 4i..4i+3 (low nibbles)
    b.w[4 + i] = nib_s8(c[i], 4);  // elements 16+4i.. (high nibbles)
  }
  b.S = f16_bits_to_f32(L.mis ? r.s : r.v.x);
  b.O = 0.0f;
  return b;
}

__device__ __forceinline__ WBlk unpack_w(const FmtQ8_0::Raw& r, const BlockLane& L, int /*j*/) {
  WBlk b;
  const uint32_t w[9] = {r.v0.x, r.v0.y, r.v0.z, r.v0.w, r.v1.x, r.v1.y, r.v1.z, r.v1.w, r.s};
#pragma unroll
  for (int i = 0; i < 8; ++i) b.w[i] = perm_b32(w[i + 1], w[i], L.sel);
  b.S = f16_bits_to_f32(L.mis ? r.s : r.v0.x);
  b.O = 0.0f;
  return b;
}

__device__ __forceinline__ WBlk unpack_w(const FmtQ6_K::Raw& r, const BlockLane& L, int /*j*/) {
  WBlk b;
  const uint32_t x[7] = {r.v.x, r.v.y, r.v.z, r.v.w, r.u0, r.u1, (uint32_t)r.s};
  const uint32_t H[2] = {perm_b32(x[5], x[4], L.sel), perm_b32(x[6], x[5], L.sel)};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t N = perm_b32(x[w + 1], x[w], L.sel);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // codes 0..63 of elements 16h+4w.., then c - 32 per byte (c + 96 has
      // no carry out of its byte; flipping bit 7 then gives c - 32 mod 256)
      const uint32_t lo = h ? (N >> 4) & 0x0F0F0F0Fu : N & 0x0F0F0F0Fu;
      const uint32_t c = lo | (((H[h] >> (2 * w)) & 0x03030303u) << 4);
      b.w[4 * h + w] = (c + 0x60606060u) ^ 0x80808080u;
    }
  }
  const uint32_t scw = L.mis ? (uint32_t)r.s : r.v.x;
  const float D = f16_bits_to_f32(r.d);
  b.S = D * (float)(int8_t)(scw & 0xFFu);
  b.Sb = D * (float)(int8_t)((scw >> 8) & 0xFFu);
  b.O = 0.0f;
  return b;
}

__device__ __forceinline__ WBlk unpack_w(const FmtQ4_K::Raw& r, const BlockLane& /*L*/, int j) {
  WBlk b;
  const uint32_t c[4] = {r.c.x, r.c.y, r.c.z, r.c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    b.w[i] = c[i] & 0x0F0F0F0Fu;
    b.w[4 + i] = (c[i] >> 4) & 0x0F0F0F0Fu;
  }
  const int sub = j & 7;
  const int ps = 6 * sub, pm = 48 + 6 * sub;
  const uint32_t slo = ps < 32 ? r.h.y : r.h.z, shi = ps < 32 ? r.h.z : r.h.w;
  const uint32_t mlo = pm < 64 ? r.h.z : r.h.w, mhi = pm < 64 ? r.h.w : 0u;
  const uint32_t sc = __builtin_amdgcn_alignbit(shi, slo, ps & 31) & 63u;
  const uint32_t mn = __builtin_amdgcn_alignbit(mhi, mlo, pm & 31) & 63u;
  b.S = f16_bits_to_f32(r.h.x) * (float)sc;
  b.O = f16_bits_to_f32(r.h.x >> 16) * (float)mn;
  return b;
}

// LDS image of one strip's activation records for NT tokens: the two
// 16-byte halves of the 32 codes, dx, and dx * sum(codes).
template <int NT>
struct XRecs {
  uint32_t q[NT][2][kWave][4];
  float dx[NT][kWave];
  float xs[NT][kWave];
};

template <class F, int R, int G, int NT, bool kOdd>
__global__ __launch_bounds__(G * kWave) void gemm_small_kernel(
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Xq, float* __restrict__ Y,
    int64_t M, int K, int64_t N, int64_t n0) {
  static_assert((R * NT & (R * NT - 1)) == 0 && R * NT <= kWave, "values per lane");
  constexpr bool kQ4K = F::kBytes == 144;
  constexpr bool kQ6K = F::kBytes == 210;
  constexpr int kT = G * kWave;
  constexpr int kRecs = (NT * kWave + kT - 1) / kT;  // records a thread stages per strip
  __shared__ __attribute__((aligned(16))) XRecs<NT> xr[2];
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int ns = K >> 5;
  const int nstrips = (ns + kWave - 1) / kWave;
  const int64_t rb = F::row_bytes(K);
  const int64_t xrb = (int64_t)ns * 34;
  const int64_t mw = (int64_t)blockIdx.x * (G * R) + wv * R;  // this wave's first row

  // activation records: raw loads of a strip, then unpack into LDS
  struct XRaw {
    u32x4 a, b;
    uint32_t s;
  };
  XRaw xraw[kRecs];
  auto load_x = [&](int strip) {
#pragma unroll
    for (int k = 0; k < kRecs; ++k) {
      const int rec = tid + k * kT;
      const int n = rec >> 6, jj = rec & 63;
      const int j = strip * kWave + jj;
      if (rec < NT * kWave && n0 + n < N && j < ns) {
        const uint8_t* row = Xq + (n0 + n) * xrb;
        const BlockLane L = block_lane((uint32_t)j * 34u, (uint32_t)((n0 + n) * xrb) & 2u, 34);
        xraw[k].a = *reinterpret_cast<const u32x4_a4*>(row + L.o16);
        xraw[k].b = *reinterpret_cast<const u32x4_a4*>(row + L.o16 + 16);
        xraw[k].s = *reinterpret_cast<const uint16_t*>(row + L.o2);
      }
    }
  };
  auto store_x = [&](int strip, XRecs<NT>& dst) {
#pragma unroll
    for (int k = 0; k < kRecs; ++k) {
      const int rec = tid + k * kT;
      if (rec >= NT * kWave) continue;
      const int n = rec >> 6, jj = rec & 63;
      const int j = strip * kWave + jj;
      uint32_t c[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
      float dx = 0.0f;
      if (n0 + n < N && j < ns) {
        const BlockLane L = block_lane((uint32_t)j * 34u, (uint32_t)((n0 + n) * xrb) & 2u, 34);
        const uint32_t w[9] = {xraw[k].a.x, xraw[k].a.y, xraw[k].a.z, xraw[k].a.w,
                               xraw[k].b.x, xraw[k].b.y, xraw[k].b.z, xraw[k].b.w, xraw[k].s};
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = perm_b32(w[i + 1], w[i], L.sel);
        dx = f16_bits_to_f32(L.mis ? xraw[k].s : xraw[k].a.x);
      }
      *reinterpret_cast<u32x4*>(dst.q[n][0][jj]) = u32x4{c[0], c[1], c[2], c[3]};
      *reinterpret_cast<u32x4*>(dst.q[n][1][jj]) = u32x4{c[4], c[5], c[6], c[7]};
      dst.dx[n][jj] = dx;
      if (kQ4K) {
        int qs = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) qs = sdot4(c[i], 0x01010101u, qs);
        dst.xs[n][jj] = dx * (float)qs;
      }
    }
  };

  // weight blocks of this wave's R rows, slice (strip * 64 + lane)
  // with an odd row stride, row m starts at 2 (m & 1) mod 4 (the lane's
  // offsets are computed for that parity directly: an array of both would
  // be indexed at run time and live in scratch memory)
  auto lane_of = [&](int strip, int r) {
    return F::lane(strip * kWave + lane, kOdd ? 2u * (uint32_t)((mw + r) & 1) : 0u);
  };
  typename F::Raw wraw[R];
  auto load_w = [&](int strip) {
    if (strip * kWave + lane < ns) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        // rows past M re-read the last row of the same parity (M >= 2 here)
        const int p = kOdd ? (int)((mw + r) & 1) : 0;
        int64_t m = mw + r;
        if (m >= M) m = kOdd ? M - 1 - ((M - 1 - p) & 1) : M - 1;
        F::load(B + m * rb, lane_of(strip, r), wraw[r]);
      }
    }
  };

  float acc[R * NT];
#pragma unroll
  for (int i = 0; i < R * NT; ++i) acc[i] = 0.0f;

  if (nstrips > 0) {
    load_x(0);
    load_w(0);
    store_x(0, xr[0]);
  }
  __syncthreads();
  for (int st = 0; st < nstrips; ++st) {
    const bool more = st + 1 < nstrips;
    if (more) load_x(st + 1);
    const int j = st * kWave + lane;
    const bool live = j < ns;
    WBlk wb[R];
    {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        wb[r] = unpack_w(wraw[r], lane_of(st, r), j);
        if (!live) {
#pragma unroll
          for (int i = 0; i < 8; ++i) wb[r].w[i] = 0u;
          wb[r].S = 0.0f;
          wb[r].O = 0.0f;
          wb[r].Sb = 0.0f;
        }
      }
    }
    if (more) load_w(st + 1);
    const XRecs<NT>& cur = xr[st & 1];
    // token records one ahead of their use (two in registers at a time)
    u32x4 qa[2], qb[2];
    float dxv[2], xsv[2];
    auto read_rec = [&](int n, int slot) {
      qa[slot] = *reinterpret_cast<const u32x4*>(cur.q[n][0][lane]);
      qb[slot] = *reinterpret_cast<const u32x4*>(cur.q[n][1][lane]);
      dxv[slot] = cur.dx[n][lane];
      if (kQ4K) xsv[slot] = cur.xs[n][lane];
    };
    read_rec(0, 0);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      if (n + 1 < NT) read_rec(n + 1, (n + 1) & 1);
      const u32x4 a = qa[n & 1], b = qb[n & 1];
      const uint32_t xq[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (kQ6K) {
          // two 16-element halves with their own scales
          int32_t Sa = 0, Sb = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            Sa = sdot4(wb[r].w[i], xq[i], Sa);
            Sb = sdot4(wb[r].w[4 + i], xq[4 + i], Sb);
          }
          acc[r * NT + n] = fmaf((float)Sb * dxv[n & 1], wb[r].Sb,
                                 fmaf((float)Sa * dxv[n & 1], wb[r].S, acc[r * NT + n]));
          continue;
        }
        int32_t S = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) S = sdot4(wb[r].w[i], xq[i], S);
        const float t = (float)S * dxv[n & 1];
        if (kQ4K)
          acc[r * NT + n] = fmaf(-wb[r].O, xsv[n & 1], fmaf(t, wb[r].S, acc[r * NT + n]));
        else
          acc[r * NT + n] = fmaf(t, wb[r].S, acc[r * NT + n]);
      }
      // Keep the reads one token ahead: token n's sums are complete before
      // the next record is requested. (Left alone, the compiler reads all NT
      // records up front and holds them in registers.)
#pragma unroll
      for (int r = 0; r < R; ++r) asm volatile("" : "+v"(acc[r * NT + n])::"memory");
    }
    if (more) store_x(st + 1, xr[(st + 1) & 1]);
    __syncthreads();
  }

  // value v = r * NT + n, summed over the wave's 64 slices
  constexpr int RN = R * NT;
  constexpr int kShift = 6 - log2i<RN>();
  const int v = (lane >> kShift) & (RN - 1);
  const float sum = wave_reduce_rows<RN>(acc, lane);
  if ((lane & ((1 << kShift) - 1)) == 0) {
    const int r = v / NT, n = v % NT;
    const int64_t m = mw + r;
    if (m < M && n0 + n < N) Y[(n0 + n) * M + m] = sum;
  }
}

// ------------------------------------- few tokens, a row per wave (NT <= 8) --
// The row-per-wave GEMV's structure for up to eight tokens, X given as Q8_0
// blocks. A workgroup owns kRowWaves rows and all of K (at most 8 strips of
// 64 slices): 16 waves of one row each, or from four tokens 8 waves of two
// rows each, which halves the LDS reads per row. LDS holds one slot per 64-slice
// strip with the strip's records for NT tokens: the 32 codes of each block
// as two 16-byte halves ([token][half][slice]), dx, and for Q4_K-style
// dx * sum(codes). At the start, wave w loads strip w's blocks of every token
// (ahead of any weight load), requests its row's first kD strips of weight
// blocks, writes the strip's records and raises its ready flag. Each wave
// then streams its row strip by strip (lane = slice), waiting only for the
// flag of the strip it uses next; each weight block is unpacked to int8 once
// and multiplied with every token's block by v_dot4_i32_i8 (exact), then
// scaled by the two block scales in fp32, as in gemm_small_kernel.
template <int NT>
struct DecRows {
  static constexpr int kSlot = NT * (2 * kWave * 16 + 2 * kWave * 4);  // bytes per strip
  __device__ static u32x4* q(uint8_t* slot, int n, int h, int l) {
    return reinterpret_cast<u32x4*>(slot + (n * 2 + h) * (kWave * 16) + 16 * l);
  }
  __device__ static float* dx(uint8_t* slot, int n) {
    return reinterpret_cast<float*>(slot + NT * 2 * kWave * 16 + n * kWave * 4);
  }
  __device__ static float* xs(uint8_t* slot, int n) {
    return reinterpret_cast<float*>(slot + NT * 2 * kWave * 16 + (NT + n) * kWave * 4);
  }
};

template <class F, int NT, int R, int kWaves, int kD, bool kOdd>
__global__ __launch_bounds__(kWaves * kWave) void decode_rows_kernel(
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Xq, float* __restrict__ Y,
    int64_t M, int K, int64_t N, int64_t n0) {
  extern __shared__ __attribute__((aligned(16))) uint8_t slots[];
  __shared__ int ready[8];
  typedef DecRows<NT> L;
  constexpr bool kQ4K = F::kBytes == 144;
  constexpr bool kQ6K = F::kBytes == 210;
  constexpr uint32_t kOut = 0x80000000u;  // an offset past the end of any row
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int ns = K >> 5;
  const int nstrips = (ns + kWave - 1) / kWave;
  const int64_t rb = F::row_bytes(K);
  const int64_t xrb = (int64_t)ns * 34;
  static_assert(kWaves >= 8, "wave w converts strip w");
  const int64_t m0 = ((int64_t)blockIdx.x * kWaves + wv) * R;  // this wave's first row
  // with an odd row stride, row m starts at 2 (m & 1) mod 4; a row past M
  // re-reads the last row of the same parity (M >= 2 then)
  __amdgpu_buffer_rsrc_t rrs[R];
  uint32_t par[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t m = m0 + r;
    par[r] = kOdd ? (uint32_t)(m & 1) : 0u;
    const int64_t mr = m < M ? m : (kOdd ? M - 1 - ((M - 1 - (int64_t)par[r]) & 1) : M - 1);
    rrs[r] = make_rsrc(B + mr * rb, rb);
  }

  // LDS holds whatever the last workgroup left: clear the flags first
  if (threadIdx.x < 8) flag_set(&ready[threadIdx.x], 0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // strip wv of every token's blocks, first among this wave's loads
  const bool conv = wv < nstrips;
  const int jc = wv * kWave + lane;  // the slice this lane converts
  u32x4 xa[NT], xb[NT];
  uint32_t xsc[NT];
  BlockLane XL[NT];
  if (conv) {
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int64_t t = n0 + n < N ? n0 + n : N - 1;  // tokens past N: re-read, scaled by 0
      const uint8_t* row = Xq + t * xrb;
      XL[n] = block_lane((uint32_t)(jc < ns ? jc : ns - 1) * 34u, (uint32_t)(t * xrb) & 2u, 34);
      xa[n] = *reinterpret_cast<const u32x4_a4*>(row + XL[n].o16);
      xb[n] = *reinterpret_cast<const u32x4_a4*>(row + XL[n].o16 + 16);
      xsc[n] = *reinterpret_cast<const uint16_t*>(row + XL[n].o2);
    }
  }
  // every wave's weight loads queue behind all of the activation loads
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  auto lane_of = [&](int st, uint32_t p) { return F::lane(st * kWave + lane, 2u * p); };
  typename F::Raw wb[kD][R];
  auto load_w = [&](int st, typename F::Raw (&dst)[R]) {
    const bool ok = st < nstrips && st * kWave + lane < ns;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      BlockLane W = lane_of(st, par[r]);
      if (!ok) W.o16 = W.o2 = W.o8 = W.od = kOut;
      F::load(rrs[r], W, dst[r]);
    }
  };
#pragma unroll
  for (int u = 0; u < kD; ++u) {
    load_w(u, wb[u]);
    __builtin_amdgcn_sched_barrier(0);
  }

  if (conv) {
    uint8_t* const own = slots + wv * L::kSlot;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const uint32_t w[9] = {xa[n].x, xa[n].y, xa[n].z, xa[n].w,
                             xb[n].x, xb[n].y, xb[n].z, xb[n].w, xsc[n]};
      uint32_t c[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = perm_b32(w[i + 1], w[i], XL[n].sel);
      const uint32_t dbits = XL[n].mis ? xsc[n] : xa[n].x;
      const bool live = jc < ns && n0 + n < N;
      const float dx = live ? f16_bits_to_f32(dbits) : 0.0f;
      *L::q(own, n, 0, lane) = u32x4{c[0], c[1], c[2], c[3]};
      *L::q(own, n, 1, lane) = u32x4{c[4], c[5], c[6], c[7]};
      L::dx(own, n)[lane] = dx;
      if (kQ4K) {
        int qs = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) qs = sdot4(c[i], 0x01010101u, qs);
        L::xs(own, n)[lane] = dx * (float)qs;
      }
    }
    // records first (LDS completes a wave's accesses in order once waited
    // for), then the flag
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (lane == 0) flag_set(&ready[wv], 1);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_setprio(0);
  }

  float acc[R * NT];  // value r * NT + t
#pragma unroll
  for (int i = 0; i < R * NT; ++i) acc[i] = 0.0f;
  bool lost = false;  // a flag wait gave up
  // strip st from buffer w, then (if `next`) strip st + kD into w
  auto step = [&](int st, typename F::Raw (&w)[R], bool next) {
    const int j = st * kWave + lane;
    int n = 0;
    for (; flag_get(&ready[st]) == 0 && n < kRowSpinLimit; ++n) __builtin_amdgcn_s_sleep(1);
    lost |= n == kRowSpinLimit;
    asm volatile("" ::: "memory");
    uint8_t* const slot = slots + st * L::kSlot;
    WBlk b[R];
#pragma unroll
    for (int r = 0; r < R; ++r) b[r] = unpack_w(w[r], lane_of(st, par[r]), j);
    if (next) load_w(st + kD, w);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const u32x4 qa = *L::q(slot, t, 0, lane), qb = *L::q(slot, t, 1, lane);
      const uint32_t xq[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
      const float dx = L::dx(slot, t)[lane];
      const float xsv = kQ4K ? L::xs(slot, t)[lane] : 0.0f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float& a = acc[r * NT + t];
        if (kQ6K) {
          int32_t Sa = 0, Sb = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            Sa = sdot4(b[r].w[i], xq[i], Sa);
            Sb = sdot4(b[r].w[4 + i], xq[4 + i], Sb);
          }
          a = fmaf((float)Sb * dx, b[r].Sb, fmaf((float)Sa * dx, b[r].S, a));
          continue;
        }
        int32_t S = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) S = sdot4(b[r].w[i], xq[i], S);
        const float tt = (float)S * dx;
        if (kQ4K)
          a = fmaf(-b[r].O, xsv, fmaf(tt, b[r].S, a));
        else
          a = fmaf(tt, b[r].S, a);
      }
    }
    // the next strip's arithmetic must not move above these loads
    __builtin_amdgcn_sched_barrier(0);
  };
  int s0 = 0;
  for (; s0 + 2 * kD <= nstrips; s0 += kD) {
#pragma unroll
    for (int u = 0; u < kD; ++u) step(s0 + u, wb[u], true);
  }
#pragma unroll
  for (int u = 0; u < kD; ++u)
    if (s0 + u < nstrips) step(s0 + u, wb[u], s0 + u + kD < nstrips);
#pragma unroll
  for (int u = 0; u + 1 < kD; ++u)
    if (s0 + kD + u < nstrips) step(s0 + kD + u, wb[u], false);
  // value v = r * NT + t summed over the wave's 64 slices
  constexpr int RN = R * NT;
  constexpr int kShift = 6 - log2i<RN>();
  const int v = (lane >> kShift) & (RN - 1);
  const float sum = wave_reduce_rows<RN>(acc, lane);
  const int r = v / NT, t = v % NT;
  if ((lane & ((1 << kShift) - 1)) == 0 && m0 + r < M && n0 + t < N)
    Y[(n0 + t) * M + m0 + r] = lost ? __builtin_nanf("") : sum;
}

#ifndef QMAT_DECODE_ROWS
#define QMAT_DECODE_ROWS 1
#endif
// Chunks of up to 8 tokens take the row-per-wave kernel when K fits its LDS
// slots, except where another kernel measured faster. Against
// gemm_small_kernel (4096 x 11008 and 11008 x 4096): 1 and 2 tokens are
// faster in every format (Q4_0 4096 x 11008: 7.4 / 7.7 against 9.8 / 8.4
// us), and 3 and 4 tokens with two rows per wave (each token's records then
// read from LDS once per two rows) in every format but Q4_K-style at 4096 x
// 11008, which ties (Q4_0: 8.9 against 9.6 us; 11008 x 4096: 9.8 against
// 12.6; Q4_K-style 9.3 against 9.2 and 11.4 against 12.2; one row per wave:
// Q4_0 10.0-10.1, Q4_K-style 10.6 us). At 5 to 8 tokens, against the
// matrix-core kernel (Q4_0, Q8_0) or gemm_small_kernel: Q8_0 13.0 against
// 13.1 us and 13.0 against 17.3; Q6_K-style 15.3 against 15.6 and 14.6
// against 19.0; Q4_0 11.5 against 14.3 at 11008 x 4096 but 12.4 against
// 11.3 at 4096 x 11008 (the matrix cores win on long rows); Q4_K-style 12.8
// against 12.6-12.9 and 17.1 against 15.7 (left to gemm_small_kernel).
#ifndef QMAT_DECODE_ROWS_LDS
#define QMAT_DECODE_ROWS_LDS 160768
#endif
constexpr int64_t kDecodeRowsMaxLds = QMAT_DECODE_ROWS_LDS;  // dynamic LDS of a launch
constexpr int64_t kDecodeRowsLongK = 8192;  // Q4_0 rows from here: 5-8 tokens on the matrix cores

// the most tokens per chunk the row-per-wave kernel takes, by format and K
inline int64_t decode_rows_max_tokens(int fmt, int64_t K) {
  if (fmt == kFmtQ4_K) return 4;
  if (fmt == kFmtQ4_0) return K < kDecodeRowsLongK ? 8 : 4;
  return 8;
}

#ifndef QMAT_DECODE_ROWS_R4
#define QMAT_DECODE_ROWS_R4 2  // rows per wave from 3 tokens (16 / R waves per workgroup)
#endif

template <class F, int NT, int kD>
hipError_t launch_decode_rows(const void* blocks, const void* Xq8, float* Y, int64_t M,
                              int64_t K, int64_t N, int64_t n0, hipStream_t stream) {
  constexpr int R = NT >= 4 ? QMAT_DECODE_ROWS_R4 : 1, kWaves = kRowWaves / R;
  const int64_t ns = K / 32;
  const int64_t nstrips = (ns + kWave - 1) / kWave;
  const int64_t grid = (M + kWaves * R - 1) / (kWaves * R);
  const size_t lds = (size_t)nstrips * DecRows<NT>::kSlot;
  const bool odd = (F::row_bytes(K) & 2) != 0 && M > 1;  // rows start 2 mod 4
  const uint8_t* Bp = static_cast<const uint8_t*>(blocks);
  const uint8_t* Xp = static_cast<const uint8_t*>(Xq8);
  if (odd)
    hipLaunchKernelGGL((decode_rows_kernel<F, NT, R, kWaves, kD, true>), dim3((unsigned)grid),
                       dim3(kWaves * kWave), lds, stream, Bp, Xp, Y, M, (int)K, N, n0);
  else
    hipLaunchKernelGGL((decode_rows_kernel<F, NT, R, kWaves, kD, false>), dim3((unsigned)grid),
                       dim3(kWaves * kWave), lds, stream, Bp, Xp, Y, M, (int)K, N, n0);
  return hipGetLastError();
}

template <class F, int NT>
hipError_t launch_small_fmt(const void* blocks, const void* Xq8, float* Y, int64_t M, int64_t K,
                            int64_t N, int64_t n0, hipStream_t stream) {
  constexpr int R = NT <= 4 ? QMAT_SMALL_R4 : NT <= 8 ? QMAT_SMALL_R8 : QMAT_SMALL_R16;
  constexpr int G = NT <= 4 ? QMAT_SMALL_G4 : NT <= 8 ? QMAT_SMALL_G8 : QMAT_SMALL_G16;
  const int64_t ns = K / 32;
  const int64_t grid = (M + R * G - 1) / (R * G);
  const bool odd = (F::row_bytes(K) & 2) != 0 && M > 1;  // rows start 2 mod 4
  if (odd)
    hipLaunchKernelGGL((gemm_small_kernel<F, R, G, NT, true>), dim3((unsigned)grid),
                       dim3(G * kWave), 0, stream, static_cast<const uint8_t*>(blocks),
                       static_cast<const uint8_t*>(Xq8), Y, M, (int)K, N, n0);
  else
    hipLaunchKernelGGL((gemm_small_kernel<F, R, G, NT, false>), dim3((unsigned)grid),
                       dim3(G * kWave), 0, stream, static_cast<const uint8_t*>(blocks),
                       static_cast<const uint8_t*>(Xq8), Y, M, (int)K, N, n0);
  return hipGetLastError();
}

// whether a chunk of nt tokens goes to the row-per-wave kernel: its LDS
// slots (one per 64-slice strip, at most 8) must fit
inline bool decode_rows_takes(int fmt, int64_t K, int64_t nt) {
  const int64_t nstrips = (K / 32 + kWave - 1) / kWave;
  const int64_t slot = nt <= 1 ? DecRows<1>::kSlot
                       : nt <= 2 ? DecRows<2>::kSlot
                       : nt <= 4 ? DecRows<4>::kSlot
                                 : DecRows<8>::kSlot;
  return QMAT_DECODE_ROWS && K >= 32 && nt <= decode_rows_max_tokens(fmt, K) && nstrips <= 8 &&
         nstrips * slot <= kDecodeRowsMaxLds;
}

template <class F, int RD>
hipError_t launch_small_chunk(int fmt, const void* blocks, const void* Xq8, float* Y, int64_t M,
                              int64_t K, int64_t N, int64_t n0, hipStream_t stream) {
  const int64_t nt = N - n0 < 16 ? N - n0 : 16;
  if (decode_rows_takes(fmt, K, nt)) {
    if (nt <= 1) return launch_decode_rows<F, 1, RD>(blocks, Xq8, Y, M, K, N, n0, stream);
    if (nt <= 2) return launch_decode_rows<F, 2, RD>(blocks, Xq8, Y, M, K, N, n0, stream);
    if (nt <= 4) return launch_decode_rows<F, 4, RD>(blocks, Xq8, Y, M, K, N, n0, stream);
    return launch_decode_rows<F, 8, RD>(blocks, Xq8, Y, M, K, N, n0, stream);
  }
  if (nt <= 1) return launch_small_fmt<F, 1>(blocks, Xq8, Y, M, K, N, n0, stream);
  if (nt <= 2) return launch_small_fmt<F, 2>(blocks, Xq8, Y, M, K, N, n0, stream);
  if (nt <= 4) return launch_small_fmt<F, 4>(blocks, Xq8, Y, M, K, N, n0, stream);
  if (nt <= 8) return launch_small_fmt<F, 8>(blocks, Xq8, Y, M, K, N, n0, stream);
  return launch_small_fmt<F, 16>(blocks, Xq8, Y, M, K, N, n0, stream);
}

}  // namespace

hipError_t launch_gemv_batch(int fmt, const GemvJob* jobs, int64_t count, hipStream_t stream) {
  switch (fmt) {
    case kFmtQ4_0:
      return launch_batch_fmt<FmtQ4_0, QMAT_BATCH_R_Q4_0, QMAT_BATCH_G_Q4_0, QMAT_BATCH_D_Q4_0,
                              QMAT_GEMV_ROW_DEPTH_Q4_0>(jobs, count, stream);
    case kFmtQ8_0:
      return launch_batch_fmt<FmtQ8_0, QMAT_BATCH_R_Q8_0, QMAT_BATCH_G_Q8_0, QMAT_BATCH_D_Q8_0,
                              QMAT_GEMV_ROW_DEPTH_Q8_0>(jobs, count, stream);
    case kFmtQ4_K:
      return launch_batch_fmt<FmtQ4_K, QMAT_BATCH_R_Q4_K, QMAT_BATCH_G_Q4_K, QMAT_BATCH_D_Q4_K,
                              QMAT_GEMV_ROW_DEPTH_Q4_K>(jobs, count, stream);
    default:
      return launch_batch_fmt<FmtQ6_K, QMAT_BATCH_R_Q6_K, QMAT_BATCH_G_Q6_K, QMAT_BATCH_D_Q6_K,
                              QMAT_GEMV_ROW_DEPTH_Q6_K>(jobs, count, stream);
  }
}

hipError_t launch_gemv(int fmt, const void* blocks, const float* x, float* y, int64_t M,
                       int64_t K, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  switch (fmt) {
    case kFmtQ4_0:
      return launch_fmt<FmtQ4_0, QMAT_GEMV_R_Q4_0, QMAT_GEMV_G_Q4_0, QMAT_GEMV_D_Q4_0,
                        QMAT_GEMV_ROW_DEPTH_Q4_0>(
          blocks, x, y, M, K, stream);
    case kFmtQ8_0:
      return launch_fmt<FmtQ8_0, QMAT_GEMV_R_Q8_0, QMAT_GEMV_G_Q8_0, QMAT_GEMV_D_Q8_0,
                        QMAT_GEMV_ROW_DEPTH_Q8_0>(
          blocks, x, y, M, K, stream);
    case kFmtQ4_K:
      return launch_fmt<FmtQ4_K, QMAT_GEMV_R_Q4_K, QMAT_GEMV_G_Q4_K, QMAT_GEMV_D_Q4_K,
                        QMAT_GEMV_ROW_DEPTH_Q4_K>(
          blocks, x, y, M, K, stream);
    default:
      return launch_fmt<FmtQ6_K, QMAT_GEMV_R_Q6_K, QMAT_GEMV_G_Q6_K, QMAT_GEMV_D_Q6_K,
                        QMAT_GEMV_ROW_DEPTH_Q6_K>(
          blocks, x, y, M, K, stream);
  }
}

}  // namespace qmat

namespace qmat {

#ifndef QMAT_DECODE_MFMA
#define QMAT_DECODE_MFMA 1
#endif
// Chunks of at least this many tokens go to the matrix-core kernel when it
// takes the format and K (and the row-per-wave kernel does not). Measured
// at 4096 x 11008 against gemm_small_kernel: Q4_0 / Q8_0 from 5 tokens (8
// tokens: 11.4 / 13.3 us against 12.8 / 13.7; 16: 12.8 / 15.3 against 20.7
// / 21.4); Q4_K-style from 9 (8 tokens: 13.8 against 13.0 us; 12: 15.0
// against 20.5; 16: 15.2 against 22.1, and 19.6 against 24.8 at 11008 x
// 4096), its two matrix-core products per block (codes, and the block sums
// of the tokens for the offset term) costing more arithmetic. Q6_K-style
// (two products per block, one per half) also from 9: 4096 x 11008 at 9 / 16
// tokens 19.3 / 19.9 us against 23.8 / 25.6; at 5-8 tokens on rows too long
// for the row-per-wave kernel it loses (4096 x 20480, 8 tokens: 30.6 against
// 24.5). On tall matrices (the kernel's shape with several workgroups per
// CU) Q4_K-style takes it from 5 tokens too: 11008 x 4096 at 5 / 8 tokens
// 13.1 / 13.4 us against the strip kernel's 15.6 / 16.0.
inline int64_t decode_mfma_min_tokens(int fmt, int64_t M) {
  if (fmt == kFmtQ4_K) return decode_mfma_tall(M) ? 5 : 9;
  return fmt == kFmtQ6_K ? 9 : 5;
}

hipError_t launch_gemm_small(int fmt, const void* blocks, const void* Xq8, float* Y, int64_t M,
                             int64_t K, int64_t N, hipStream_t stream) {
  for (int64_t n0 = 0; n0 < N; n0 += 16) {
    hipError_t e;
    const int64_t nt = N - n0 < 16 ? N - n0 : 16;
    if (QMAT_DECODE_MFMA && nt >= decode_mfma_min_tokens(fmt, M) && !decode_rows_takes(fmt, K, nt) &&
        decode_mfma_fits(fmt, K)) {
      e = launch_decode_mfma(fmt, blocks, Xq8, Y, M, K, N, n0, stream);
      if (e != hipSuccess) return e;
      continue;
    }
    switch (fmt) {
      case kFmtQ4_0:
        e = launch_small_chunk<FmtQ4_0, QMAT_GEMV_ROW_DEPTH_Q4_0>(fmt, blocks, Xq8, Y, M, K, N, n0,
                                                                stream);
        break;
      case kFmtQ8_0:
        e = launch_small_chunk<FmtQ8_0, QMAT_GEMV_ROW_DEPTH_Q8_0>(fmt, blocks, Xq8, Y, M, K, N, n0,
                                                                stream);
        break;
      case kFmtQ4_K:
        e = launch_small_chunk<FmtQ4_K, QMAT_GEMV_ROW_DEPTH_Q4_K>(fmt, blocks, Xq8, Y, M, K, N, n0,
                                                                stream);
        break;
      default:
        e = launch_small_chunk<FmtQ6_K, QMAT_GEMV_ROW_DEPTH_Q6_K>(fmt, blocks, Xq8, Y, M, K, N, n0,
                                                                stream);
        break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qmat
