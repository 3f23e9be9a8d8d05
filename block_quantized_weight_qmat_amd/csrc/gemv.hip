// gemv.hip — decode-time y = dequant(W) x for Q4_0 / Q8_0 / Q4_K-style W.
//
// Source: "05. llama.cpp：从 GGUF 文件到本地推理服务", section "性能直觉：带宽
// 决定 Decode，算力决定 Prefill": single-token decode reads every weight once,
// so its speed limit is memory bandwidth divided by weight bytes. The kernel
// is therefore built around the HBM stream of packed blocks.
//
// Work split
//   * A workgroup owns R consecutive rows and all of K. Its waves split K
//     into 64-slice strips; lane l of a strip owns one 32-element K-slice
//     (one Q4_0/Q8_0 block, or one sub-block of a Q4_K superblock) of every
//     one of the R rows, so neighbouring lanes read neighbouring blocks and
//     a wave's loads cover a contiguous span of each row.
//   * The R rows' loads are issued first; the activation slice is prepared
//     while they are in flight and reused from registers for all R rows.
//   * Per-lane partial sums of the R rows are reduced with a butterfly that
//     halves the live values at each exchange, then across waves in LDS in a
//     fixed order (deterministic).
//
// Arithmetic
//   * Activation prescale: the lane's 32 values are multiplied by 2^s with
//     s = 15 - exponent(amax), so the largest is in [2^14, 2^15), then
//     rounded to fp16. Relative rounding error <= 2^-11 per value.
//   * Nibble unpack without conversions: a code c placed in the mantissa of
//     the fp16 pattern 0x6400 is exactly 1024 + c; the high nibble of a byte,
//     masked in place, gives 1024 + 16c. v_dot2_f32_f16 multiplies these by
//     fp16 activation pairs exactly and accumulates in fp32; the 1024 offsets
//     are removed once per slice with the slice's activation sums.
//   * Q8_0 bytes are made unsigned by flipping the sign bit (q + 128) and go
//     through the same 0x6400 pattern (1152 + q).
#include "qmat_device.hpp"
#include "qmat_launch.hpp"

namespace qmat {
namespace {

constexpr int kMaxWaves = 8;

// The fp16 pair (1024, 1024). Materialised in a VGPR so that
// (w & mask) | magic is a single v_and_or_b32 (mask in an SGPR, magic in a
// VGPR): a gfx9 VOP3 cannot take two literal or SGPR constants.
__device__ __forceinline__ uint32_t magic_1024() {
  uint32_t m;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
  return m;
}

struct XPrep {
  half2_t p[16];
  float c0, c1, c2;  // per-format constants derived from the fp16 values
  float inv;         // 2^-s
};

__device__ __forceinline__ void load_x32(const float* __restrict__ x, float (&v)[32]) {
  const f32x4* p = reinterpret_cast<const f32x4*>(x);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const f32x4 t = p[i];
    v[4 * i + 0] = t.x;
    v[4 * i + 1] = t.y;
    v[4 * i + 2] = t.z;
    v[4 * i + 3] = t.w;
  }
}

// s such that amax * 2^s lies in [2^14, 2^15).
__device__ __forceinline__ int prescale_exp(const float (&v)[32]) {
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(v[i]));
  int e;
  frexpf(am, &e);
  return 15 - e;
}

__device__ __forceinline__ half2_t hpair(float a, float b, int s) {
  half2_t r;
  r.x = (_Float16)ldexpf(a, s);
  r.y = (_Float16)ldexpf(b, s);
  return r;
}

// Activation pairs for nibble formats. For code dword i (code bytes
// 4i..4i+3; byte t = element t low nibble, element t+16 high nibble):
//   p[4i+0] = (x[4i],    x[4i+2])          low nibbles of bytes 0, 2
//   p[4i+1] = (x[4i+16], x[4i+18]) / 16    high nibbles of bytes 0, 2
//   p[4i+2] = (x[4i+1],  x[4i+3])          low nibbles of bytes 1, 3
//   p[4i+3] = (x[4i+17], x[4i+19]) / 16    high nibbles of bytes 1, 3
// H = sum of the fp16 low-half values, G = sum of the fp16 high-half values
// (the latter already divided by 16).
__device__ __forceinline__ void prep_nibble(const float (&v)[32], XPrep& xp, float& H, float& G) {
  const int s = prescale_exp(v);
  const half2_t one = {(_Float16)1.0f, (_Float16)1.0f};
  H = 0.0f;
  G = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xp.p[4 * i + 0] = hpair(v[4 * i], v[4 * i + 2], s);
    xp.p[4 * i + 1] = hpair(v[4 * i + 16], v[4 * i + 18], s - 4);
    xp.p[4 * i + 2] = hpair(v[4 * i + 1], v[4 * i + 3], s);
    xp.p[4 * i + 3] = hpair(v[4 * i + 17], v[4 * i + 19], s - 4);
    H = __builtin_amdgcn_fdot2(xp.p[4 * i + 0], one, H, false);
    H = __builtin_amdgcn_fdot2(xp.p[4 * i + 2], one, H, false);
    G = __builtin_amdgcn_fdot2(xp.p[4 * i + 1], one, G, false);
    G = __builtin_amdgcn_fdot2(xp.p[4 * i + 3], one, G, false);
  }
  xp.inv = ldexpf(1.0f, -s);
}

// Low-nibble and high-nibble sums over the 16 code bytes c[0..3]:
//   lo = sum (1024 + c) x_lo,  hi = sum (1024 + 16c) (x_hi / 16).
__device__ __forceinline__ void nib_dot(const uint32_t (&c)[4], const XPrep& xp, float& lo,
                                        float& hi) {
  lo = 0.0f;
  hi = 0.0f;
  const uint32_t kMagic = magic_1024();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = c[i], t = w >> 8;
    lo = dot2((w & 0x000F000Fu) | kMagic, xp.p[4 * i + 0], lo);
    hi = dot2((w & 0x00F000F0u) | kMagic, xp.p[4 * i + 1], hi);
    lo = dot2((t & 0x000F000Fu) | kMagic, xp.p[4 * i + 2], lo);
    hi = dot2((t & 0x00F000F0u) | kMagic, xp.p[4 * i + 3], hi);
  }
}

// ------------------------------------------------------------------ Q4_0 --
// 18-byte blocks: fp16 scale, 16 code bytes; weight = d * (c - 8).
struct FmtQ4_0 {
  static constexpr int kRows = 16;
  struct Raw {
    u32x4 v;
    uint32_t s;
  };
  __device__ static int64_t row_bytes(int K) { return (int64_t)(K >> 5) * 18; }
  // A block at byte offset o (even). If o = 0 mod 4 the scale and the first
  // 14 code bytes are the 16 bytes at o and the last 2 code bytes follow;
  // if o = 2 mod 4 the scale is the 2 bytes at o and the 16 code bytes are
  // the 4-aligned 16 bytes at o+2. Both cases: one 16-byte and one 2-byte
  // load, nothing read outside the block.
  __device__ static void load(const uint8_t* __restrict__ row, int j, Raw& r) {
    const uint8_t* b = row + (int64_t)j * 18;
    const uint32_t a = (uint32_t)(reinterpret_cast<uintptr_t>(b) & 2u);
    r.v = *reinterpret_cast<const u32x4_a4*>(b + a);
    r.s = *reinterpret_cast<const uint16_t*>(b + (a ? 0 : 16));
    r.s |= a << 30;  // remember the alignment case in an unused bit
  }
  __device__ static void prep(const float (&v)[32], XPrep& xp) {
    float H, G;
    prep_nibble(v, xp, H, G);
    // sum (c-8) x = lo - 1032 H + hi - 1152 G   (hi pairs are x/16)
    xp.c0 = 1032.0f * H;
    xp.c1 = 1152.0f * G;
  }
  __device__ static float apply(const Raw& r, const XPrep& xp, int /*sub*/) {
    const bool mis = (r.s >> 30) != 0;  // block at o = 2 mod 4
    const uint32_t s16 = r.s & 0xFFFFu;
    const uint32_t sel = mis ? 0x03020100u : 0x05040302u;
    uint32_t c[4];
    c[0] = perm_b32(r.v.y, r.v.x, sel);
    c[1] = perm_b32(r.v.z, r.v.y, sel);
    c[2] = perm_b32(r.v.w, r.v.z, sel);
    c[3] = perm_b32(s16, r.v.w, sel);
    const float D = f16_bits_to_f32(mis ? s16 : r.v.x);
    float lo, hi;
    nib_dot(c, xp, lo, hi);
    return (D * xp.inv) * ((lo - xp.c0) + (hi - xp.c1));
  }
};

// ------------------------------------------------------------------ Q8_0 --
// 34-byte blocks: fp16 scale, 32 int8; weight = d * q.
struct FmtQ8_0 {
  static constexpr int kRows = 8;
  struct Raw {
    u32x4 v0, v1;
    uint32_t s;
  };
  __device__ static int64_t row_bytes(int K) { return (int64_t)(K >> 5) * 34; }
  __device__ static void load(const uint8_t* __restrict__ row, int j, Raw& r) {
    const uint8_t* b = row + (int64_t)j * 34;
    const uint32_t a = (uint32_t)(reinterpret_cast<uintptr_t>(b) & 2u);
    r.v0 = *reinterpret_cast<const u32x4_a4*>(b + a);
    r.v1 = *reinterpret_cast<const u32x4_a4*>(b + a + 16);
    r.s = *reinterpret_cast<const uint16_t*>(b + (a ? 0 : 32));
    r.s |= a << 30;
  }
  // pairs: for code dword i (elements 4i..4i+3): p[2i] = (x[4i], x[4i+2]),
  // p[2i+1] = (x[4i+1], x[4i+3]).
  __device__ static void prep(const float (&v)[32], XPrep& xp) {
    const int s = prescale_exp(v);
    const half2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    float H = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      xp.p[2 * i] = hpair(v[4 * i], v[4 * i + 2], s);
      xp.p[2 * i + 1] = hpair(v[4 * i + 1], v[4 * i + 3], s);
      H = __builtin_amdgcn_fdot2(xp.p[2 * i], one, H, false);
      H = __builtin_amdgcn_fdot2(xp.p[2 * i + 1], one, H, false);
    }
    xp.inv = ldexpf(1.0f, -s);
    xp.c0 = 1152.0f * H;  // sum q x = sum (1152 + q) x - 1152 H
  }
  __device__ static float apply(const Raw& r, const XPrep& xp, int /*sub*/) {
    const bool mis = (r.s >> 30) != 0;
    const uint32_t s16 = r.s & 0xFFFFu;
    const uint32_t sel = mis ? 0x03020100u : 0x05040302u;
    const uint32_t w[9] = {r.v0.x, r.v0.y, r.v0.z, r.v0.w, r.v1.x, r.v1.y, r.v1.z, r.v1.w, s16};
    const uint32_t kMagic = magic_1024();
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t u = perm_b32(w[i + 1], w[i], sel) ^ 0x80808080u;  // q + 128
      a0 = dot2((u & 0x00FF00FFu) | kMagic, xp.p[2 * i], a0);
      a1 = dot2(((u >> 8) & 0x00FF00FFu) | kMagic, xp.p[2 * i + 1], a1);
    }
    const float D = f16_bits_to_f32(mis ? s16 : r.v0.x);
    return (D * xp.inv) * ((a0 + a1) - xp.c0);
  }
};

// ------------------------------------------------------------------ Q4_K --
// 144-byte superblocks (16-byte aligned whenever the buffer is): header
// (d, dmin, 96-bit field word) then 8 x 16 code bytes. Slice j is sub-block
// j % 8 of superblock j / 8; weight = (d sc) q - (dmin mn).
struct FmtQ4_K {
  static constexpr int kRows = 8;
  struct Raw {
    u32x4 h, c;
  };
  __device__ static int64_t row_bytes(int K) { return (int64_t)(K >> 8) * 144; }
  __device__ static void load(const uint8_t* __restrict__ row, int j, Raw& r) {
    const uint8_t* b = row + (int64_t)(j >> 3) * 144;
    r.h = *reinterpret_cast<const u32x4*>(b);
    r.c = *reinterpret_cast<const u32x4*>(b + 16 + 16 * (j & 7));
  }
  __device__ static void prep(const float (&v)[32], XPrep& xp) {
    float H, G;
    prep_nibble(v, xp, H, G);
    // sum (S q - O) x = S (lo - 1024 H + hi - 1024 G) - O (H + 16 G)
    xp.c0 = 1024.0f * H;
    xp.c1 = 1024.0f * G;
    xp.c2 = H + 16.0f * G;
  }
  __device__ static float apply(const Raw& r, const XPrep& xp, int sub) {
    // 6-bit fields: sc at bit 6*sub, mn at bit 48 + 6*sub of {w, z, y}
    const int ps = 6 * sub, pm = 48 + 6 * sub;
    const uint32_t slo = ps < 32 ? r.h.y : r.h.z, shi = ps < 32 ? r.h.z : r.h.w;
    const uint32_t mlo = pm < 64 ? r.h.z : r.h.w, mhi = pm < 64 ? r.h.w : 0u;
    const uint32_t sc = __builtin_amdgcn_alignbit(shi, slo, ps & 31) & 63u;
    const uint32_t mn = __builtin_amdgcn_alignbit(mhi, mlo, pm & 31) & 63u;
    const float S = f16_bits_to_f32(r.h.x) * (float)sc;
    const float O = f16_bits_to_f32(r.h.x >> 16) * (float)mn;
    const uint32_t c[4] = {r.c.x, r.c.y, r.c.z, r.c.w};
    float lo, hi;
    nib_dot(c, xp, lo, hi);
    return xp.inv * fmaf(S, (lo - xp.c0) + (hi - xp.c1), -O * xp.c2);
  }
};

// Butterfly reduction of R per-lane values: every exchange sends the half of
// the live values that the partner keeps, so R values need
// R/2 + R/4 + ... + 1 shuffles plus log2(64/R) full ones. On return lane l
// holds the wave sum of row (l >> (6 - log2 R)) & (R - 1).
template <int R>
__device__ __forceinline__ float wave_reduce_rows(float (&v)[R], int lane) {
  int mask = 32;
#pragma unroll
  for (int half = R / 2; half >= 1; half >>= 1) {
    // all-ones in the upper lanes of this exchange; a bitwise select keeps
    // the compiler from turning the choice into register-array indexing
    const uint32_t up = (lane & mask) ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const uint32_t a = __builtin_bit_cast(uint32_t, v[i]);
      const uint32_t b = __builtin_bit_cast(uint32_t, v[i + half]);
      const float keep = __builtin_bit_cast(float, (b & up) | (a & ~up));
      const float send = __builtin_bit_cast(float, (a & up) | (b & ~up));
      v[i] = keep + shfl_xor_f(send, mask);
    }
    mask >>= 1;
  }
#pragma unroll
  for (int m = 32 / R; m >= 1; m >>= 1) v[0] += shfl_xor_f(v[0], m);
  return v[0];
}

template <int R>
constexpr int log2i() {
  return R <= 1 ? 0 : 1 + log2i<R / 2>();
}

template <class F>
__global__ __launch_bounds__(kMaxWaves * kWave) void gemv_kernel(const uint8_t* __restrict__ B,
                                                                 const float* __restrict__ x,
                                                                 float* __restrict__ y,
                                                                 int64_t M, int K) {
  constexpr int R = F::kRows;
  __shared__ float red[kMaxWaves][R];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int ns = K >> 5;
  const int64_t rb = F::row_bytes(K);
  const int64_t m0 = (int64_t)blockIdx.x * R;

  float part[R];
#pragma unroll
  for (int r = 0; r < R; ++r) part[r] = 0.0f;

  for (int base = wv * kWave; base < ns; base += nw * kWave) {
    const int j = base + lane;
    if (j < ns) {
      // x first: its loads hit L2 and return first (loads complete in
      // order), so the activation prep overlaps the HBM weight stream
      float xv[32];
      load_x32(x + (int64_t)j * 32, xv);
      typename F::Raw raw[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t m = (m0 + r < M) ? m0 + r : M - 1;
        F::load(B + m * rb, j, raw[r]);
      }
      // keep every load above this point: all R rows are in flight before
      // any of them is consumed
      __builtin_amdgcn_sched_barrier(0);
      XPrep xp;
      F::prep(xv, xp);
#pragma unroll
      for (int r = 0; r < R; ++r) part[r] += F::apply(raw[r], xp, lane & 7);
    }
  }

  const float s = wave_reduce_rows<R>(part, lane);
  constexpr int kShift = 6 - log2i<R>();
  const int row = (lane >> kShift) & (R - 1);
  if ((lane & ((1 << kShift) - 1)) == 0) red[wv][row] = s;
  __syncthreads();
  if ((int)threadIdx.x < R) {
    float t = 0.0f;
    for (int w = 0; w < nw; ++w) t += red[w][threadIdx.x];
    if (m0 + threadIdx.x < M) y[m0 + threadIdx.x] = t;
  }
}

template <class F>
hipError_t launch_fmt(const void* blocks, const float* x, float* y, int64_t M, int64_t K,
                      hipStream_t stream) {
  const int64_t ns = K / 32;
  int waves = (int)((ns + kWave - 1) / kWave);
  if (waves < 1) waves = 1;
  if (waves > kMaxWaves) waves = kMaxWaves;
  const int64_t grid = (M + F::kRows - 1) / F::kRows;
  hipLaunchKernelGGL(gemv_kernel<F>, dim3((unsigned)grid), dim3(waves * kWave), 0, stream,
                     static_cast<const uint8_t*>(blocks), x, y, M, (int)K);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(int fmt, const void* blocks, const float* x, float* y, int64_t M,
                       int64_t K, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  switch (fmt) {
    case kFmtQ4_0: return launch_fmt<FmtQ4_0>(blocks, x, y, M, K, stream);
    case kFmtQ8_0: return launch_fmt<FmtQ8_0>(blocks, x, y, M, K, stream);
    default: return launch_fmt<FmtQ4_K>(blocks, x, y, M, K, stream);
  }
}

}  // namespace qmat
