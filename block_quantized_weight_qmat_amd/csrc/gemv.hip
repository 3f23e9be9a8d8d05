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
// Arithmetic: exact integer products
//   * Each lane turns its 32 activations into 16-bit fixed point with a
//     power-of-two scale: X = rint(x * 2^s) with s = 15 - exponent(amax)
//     (s one lower if the largest value would round to 2^15), so
//     |X| <= 32767 and the step is at most 2^-14 of the slice's largest
//     value. X is split into two int8 digits, X = 256 Xh + Xl (Xl in
//     [0,255], Xh in [-128,127]).
//   * The rounding needs no integer conversion: fma(x, 2^s, 1.5*2^23) is a
//     float whose bit pattern is 0x4B400000 + X, so its bytes 0 and 1 are
//     Xl and Xh directly; four lanes' bytes are gathered with v_perm.
//   * Codes are multiplied by the digits with v_dot4 (four 8-bit products
//     into an int32, exact): nibble codes c in [0,15] are valid as both u8
//     and i8, so sum c Xl uses v_dot4_u32_u8 and sum c Xh v_dot4_i32_i8;
//     Q8_0 bytes q use (q + 128) for the unsigned digit and subtract
//     128 * sum Xl once per slice.
//   * Per (row, slice) the exact integer sum_i (c_i - 8) X_i (Q4_0),
//     sum_i q_i X_i (Q8_0) or S sum q X - O sum X (Q4_K) is converted to
//     fp32, scaled by 2^-s and the block scale, and accumulated in fp32.
#include "qmat_device.hpp"
#include "qmat_launch.hpp"

namespace qmat {
namespace {

constexpr int kMaxWaves = 8;
constexpr float kMagicF = 12582912.0f;  // 1.5 * 2^23

// One lane's 32 activations in 16-bit fixed point, as int8 digit bytes:
// xl[i] / xh[i] hold the low / high digits of elements 4i..4i+3.
struct XPrep {
  uint32_t xl[8], xh[8];
  int32_t sx;   // sum of X
  int32_t sxl;  // sum of the low digits (0..255 each)
  int s;        // X = rint(x * 2^s)
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

__device__ __forceinline__ uint32_t udot4(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_udot4(a, b, c, false);
}

__device__ __forceinline__ int32_t sdot4(uint32_t a, uint32_t b, int32_t c) {
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

__device__ __forceinline__ void prep_x(float (&v)[32], XPrep& xp) {
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(v[i]));
  int e;
  frexpf(am, &e);  // am = m 2^e, m in [0.5, 1) (e = 0 for am = 0)
  int s = 15 - e;  // am 2^s in [2^14, 2^15)
  if (ldexpf(am, s) >= 32767.5f) s -= 1;  // would round to 2^15
  xp.s = s;
  int sa = s;
  if (sa > 120) {  // tiny activations: pre-scale exactly so 2^sa stays finite
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = ldexpf(v[i], 64);
    sa -= 64;
  }
  const float scale = ldexpf(1.0f, sa);
  uint32_t t[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) t[i] = __builtin_bit_cast(uint32_t, fmaf(v[i], scale, kMagicF));
  int32_t sl = 0, sh = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t a = perm_b32(t[4 * i + 1], t[4 * i], 0x05010400u);
    const uint32_t b = perm_b32(t[4 * i + 3], t[4 * i + 2], 0x05010400u);
    xp.xl[i] = perm_b32(b, a, 0x05040100u);
    xp.xh[i] = perm_b32(b, a, 0x07060302u);
    sl = (int32_t)udot4(xp.xl[i], 0x01010101u, (uint32_t)sl);
    sh = sdot4(xp.xh[i], 0x01010101u, sh);
  }
  xp.sxl = sl;
  xp.sx = sh * 256 + sl;
}

// sum_e c_e X_e over the 32 nibble codes in c[0..3] (byte t: element t low
// nibble, element t+16 high nibble), as the pair (sum c Xl, sum c Xh).
__device__ __forceinline__ int32_t nib_dot(const uint32_t (&c)[4], const XPrep& xp) {
  uint32_t accL = 0;
  int32_t accH = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = c[i] & 0x0F0F0F0Fu;         // elements 4i..4i+3
    const uint32_t hi = (c[i] >> 4) & 0x0F0F0F0Fu;  // elements 16+4i..16+4i+3
    accL = udot4(lo, xp.xl[i], accL);
    accH = sdot4(lo, xp.xh[i], accH);
    accL = udot4(hi, xp.xl[4 + i], accL);
    accH = sdot4(hi, xp.xh[4 + i], accH);
  }
  return accH * 256 + (int32_t)accL;
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
    const int32_t S = nib_dot(c, xp) - 8 * xp.sx;  // sum (c - 8) X, exact
    return D * ldexpf((float)S, -xp.s);
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
  __device__ static float apply(const Raw& r, const XPrep& xp, int /*sub*/) {
    const bool mis = (r.s >> 30) != 0;
    const uint32_t s16 = r.s & 0xFFFFu;
    const uint32_t sel = mis ? 0x03020100u : 0x05040302u;
    const uint32_t w[9] = {r.v0.x, r.v0.y, r.v0.z, r.v0.w, r.v1.x, r.v1.y, r.v1.z, r.v1.w, s16};
    uint32_t accL = 0;
    int32_t accH = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t q = perm_b32(w[i + 1], w[i], sel);   // q[4i..4i+3], int8
      accL = udot4(q ^ 0x80808080u, xp.xl[i], accL);      // sum (q + 128) Xl
      accH = sdot4(q, xp.xh[i], accH);                    // sum q Xh
    }
    const int32_t S = accH * 256 + ((int32_t)accL - 128 * xp.sxl);  // sum q X
    const float D = f16_bits_to_f32(mis ? s16 : r.v0.x);
    return D * ldexpf((float)S, -xp.s);
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
    const int32_t Q = nib_dot(c, xp);  // sum q X, exact
    return ldexpf(fmaf(S, (float)Q, -O * (float)xp.sx), -xp.s);
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
      prep_x(xv, xp);
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
