// gemv.hip — decode-time y = dequant(W) x for Q4_0 / Q8_0 / Q4_K-style W.
//
// Source: "05. llama.cpp：从 GGUF 文件到本地推理服务", section "性能直觉：带宽
// 决定 Decode，算力决定 Prefill": single-token decode reads every weight once,
// so its speed limit is memory bandwidth divided by weight bytes. The kernel
// is therefore built around the HBM stream of packed blocks.
//
// Work split
//   * A workgroup owns R consecutive rows (R = 8) and all of K. Its waves
//     split K into strips of 64 slices; lane l of a strip owns one 32-element
//     slice (one Q4_0/Q8_0 block, or one sub-block of a Q4_K superblock) of
//     each of the R rows, so neighbouring lanes read neighbouring blocks.
//   * Each lane issues its activation loads, then all R rows' weight loads,
//     before consuming anything; the activation slice is converted while the
//     weights stream in, and reused from registers for all R rows. Two
//     workgroups per CU (three waves per SIMD) keep enough loads in flight.
//   * Row base addresses are wave-uniform (scalar registers); each lane
//     keeps 32-bit offsets and its block-alignment case, fixed per pass (per
//     row parity when the row stride is 2 mod 4).
//   * Per-lane partial sums of the R rows are reduced with a butterfly that
//     halves the live values at each exchange, then across the strips in LDS
//     in a fixed order (deterministic).
//
// Arithmetic: exact integer products
//   * Each lane turns its 32 activations into 16-bit fixed point with a
//     power-of-two scale: X = rint(x * 2^s) with s = 15 - exponent(amax)
//     (s one lower if the largest value would round above 32639), so
//     |X| <= 32639 and the step is at most 2^-14 of the slice's largest
//     value. X is split into two signed int8 digits, X = 256 Xh + Xl with
//     Xl, Xh in [-128, 127] (balanced: Xh = (X + 128) >> 8).
//   * The rounding needs no integer conversion: fma(x, 2^s, 1.5*2^23) is a
//     float whose bit pattern is 0x4B400000 + X, so its low 16 bits are X;
//     byte 0 is Xl and byte 1 of X + 128 (a packed 16-bit add) is Xh.
//   * Codes are multiplied by the digits with v_dot4_i32_i8 (four 8-bit
//     products into an int32, exact); nibble codes c in [0,15] are valid
//     signed bytes once masked, Q8_0 bytes are signed already. The Q4_0
//     offset -8 sum X is folded into the accumulator's initial value.
//   * Per (row, slice) the exact integer sum_i (c_i - 8) X_i (Q4_0),
//     sum_i q_i X_i (Q8_0) or S sum q X - O sum X (Q4_K) is converted to
//     fp32, scaled by 2^-s and the block scale, and accumulated in fp32.
#include "qmat_device.hpp"
#include "qmat_launch.hpp"

namespace qmat {
namespace {

constexpr int kMaxStrips = 8;  // waves per workgroup
constexpr float kMagicF = 12582912.0f;  // 1.5 * 2^23

// One lane's 32 activations in 16-bit fixed point, as signed int8 digit
// bytes: xl[i] / xh[i] hold the low / high digits of elements 4i..4i+3.
struct XPrep {
  uint32_t xl[8], xh[8];
  int32_t sx;   // sum of X
  float inv;    // 2^-s, X = rint(x * 2^s)
};

__device__ __forceinline__ int32_t sdot4(uint32_t a, uint32_t b, int32_t c) {
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// Packed 16-bit add (two lanes of 16 bits, no carry between them).
__device__ __forceinline__ uint32_t add_u16x2(uint32_t a, uint32_t b) {
  typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, a) + __builtin_bit_cast(u16x2, b));
}

__device__ __forceinline__ void load_x32(const float* __restrict__ x, f32x4 (&v)[8]) {
  const f32x4* p = reinterpret_cast<const f32x4*>(x);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = p[i];
}

__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_fmaxf(__builtin_fmaxf(a, b), c);  // v_max3_f32
}

__device__ __forceinline__ void prep_x(f32x4 (&v)[8], XPrep& xp) {
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    am = max3f(am, fabsf(v[i].x), fabsf(v[i].y));
    am = max3f(am, fabsf(v[i].z), fabsf(v[i].w));
  }
  int e;
  frexpf(am, &e);  // am = m 2^e, m in [0.5, 1) (e = 0 for am = 0)
  int s = 15 - e;  // am 2^s in [2^14, 2^15)
  // balanced digits need X + 128 < 2^15, i.e. X <= 32639
  if (ldexpf(am, s) >= 32639.5f) s -= 1;
  xp.inv = ldexpf(1.0f, -s);
  int sa = s;
  if (__builtin_expect(s > 120, 0)) {
    // tiny activations: pre-scale exactly by 2^64 so that 2^sa stays finite
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i].x = ldexpf(v[i].x, 64);
      v[i].y = ldexpf(v[i].y, 64);
      v[i].z = ldexpf(v[i].z, 64);
      v[i].w = ldexpf(v[i].w, 64);
    }
    sa -= 64;
  }
  const float scale = ldexpf(1.0f, sa);
  int32_t sl = 0, sh = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t t[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      t[k] = __builtin_bit_cast(uint32_t, fmaf(v[i][k], scale, kMagicF));
    const uint32_t w01 = perm_b32(t[1], t[0], 0x05040100u);  // {X0, X1} as 16-bit
    const uint32_t w23 = perm_b32(t[3], t[2], 0x05040100u);  // {X2, X3}
    const uint32_t u01 = add_u16x2(w01, 0x00800080u);       // {X0+128, X1+128}
    const uint32_t u23 = add_u16x2(w23, 0x00800080u);
    xp.xl[i] = perm_b32(w23, w01, 0x06040200u);  // low bytes of X0..X3
    xp.xh[i] = perm_b32(u23, u01, 0x07050301u);  // byte 1 of X0+128 .. X3+128
    sl = sdot4(xp.xl[i], 0x01010101u, sl);
    sh = sdot4(xp.xh[i], 0x01010101u, sh);
  }
  xp.sx = sh * 256 + sl;
}

// sum_e c_e X_e over the 32 nibble codes in c[0..3] (byte t: element t low
// nibble, element t+16 high nibble), starting from `init`.
__device__ __forceinline__ int32_t nib_dot(const uint32_t (&c)[4], const XPrep& xp, int32_t init) {
  int32_t accL = init, accH = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = c[i] & 0x0F0F0F0Fu;         // elements 4i..4i+3
    const uint32_t hi = (c[i] >> 4) & 0x0F0F0F0Fu;  // elements 16+4i..16+4i+3
    accL = sdot4(lo, xp.xl[i], accL);
    accH = sdot4(lo, xp.xh[i], accH);
    accL = sdot4(hi, xp.xl[4 + i], accL);
    accH = sdot4(hi, xp.xh[4 + i], accH);
  }
  return accH * 256 + accL;
}

// A lane's fixed load offsets and alignment case for one 18- or 34-byte
// block at byte offset o of a row whose base has alignment parity p:
// if (base + o) = 0 mod 4 the 16-byte load at o holds the scale and the first
// code bytes and the 2-byte load at o+B-2 the last two code bytes; if it is
// 2 mod 4 the 2-byte load at o is the scale and the 16-byte load(s) at o+2
// hold the codes. Both cases read exactly the block.
struct BlockLane {
  uint32_t o16;  // offset of the (first) 16-byte load
  uint32_t o2;   // offset of the 2-byte load
  uint32_t sel;  // v_perm selector realigning the codes to 4-byte words
  bool mis;      // block starts at 2 mod 4
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
  struct Raw {
    u32x4 v;
    uint32_t s;
  };
  __device__ static int64_t row_bytes(int K) { return (int64_t)(K >> 5) * 18; }
  __device__ static void load(const uint8_t* __restrict__ row, const BlockLane& L, Raw& r) {
    r.v = *reinterpret_cast<const u32x4_a4*>(row + L.o16);
    r.s = *reinterpret_cast<const uint16_t*>(row + L.o2);
  }
  // D * sum_i (c_i - 8) X_i (still to be scaled by 2^-s)
  __device__ static float apply(const Raw& r, const BlockLane& L, const XPrep& xp, int /*sub*/) {
    uint32_t c[4];
    c[0] = perm_b32(r.v.y, r.v.x, L.sel);
    c[1] = perm_b32(r.v.z, r.v.y, L.sel);
    c[2] = perm_b32(r.v.w, r.v.z, L.sel);
    c[3] = perm_b32(r.s, r.v.w, L.sel);
    const float D = f16_bits_to_f32(L.mis ? r.s : r.v.x);
    const int32_t S = nib_dot(c, xp, -8 * xp.sx);  // sum (c - 8) X, exact
    return D * (float)S;
  }
};

// ------------------------------------------------------------------ Q8_0 --
// 34-byte blocks: fp16 scale, 32 int8; weight = d * q.
struct FmtQ8_0 {
  static constexpr int kBytes = 34;
  struct Raw {
    u32x4 v0, v1;
    uint32_t s;
  };
  __device__ static int64_t row_bytes(int K) { return (int64_t)(K >> 5) * 34; }
  __device__ static void load(const uint8_t* __restrict__ row, const BlockLane& L, Raw& r) {
    r.v0 = *reinterpret_cast<const u32x4_a4*>(row + L.o16);
    r.v1 = *reinterpret_cast<const u32x4_a4*>(row + L.o16 + 16);
    r.s = *reinterpret_cast<const uint16_t*>(row + L.o2);
  }
  __device__ static float apply(const Raw& r, const BlockLane& L, const XPrep& xp, int /*sub*/) {
    const uint32_t w[9] = {r.v0.x, r.v0.y, r.v0.z, r.v0.w, r.v1.x, r.v1.y, r.v1.z, r.v1.w, r.s};
    int32_t accL = 0, accH = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t q = perm_b32(w[i + 1], w[i], L.sel);  // q[4i..4i+3], int8
      accL = sdot4(q, xp.xl[i], accL);
      accH = sdot4(q, xp.xh[i], accH);
    }
    const float D = f16_bits_to_f32(L.mis ? r.s : r.v0.x);
    return D * (float)(accH * 256 + accL);  // D * sum q X
  }
};

// ------------------------------------------------------------------ Q4_K --
// 144-byte superblocks (16-byte aligned whenever the buffer is): header
// (d, dmin, 96-bit field word) then 8 x 16 code bytes. Slice j is sub-block
// j % 8 of superblock j / 8; weight = (d sc) q - (dmin mn).
struct FmtQ4_K {
  static constexpr int kBytes = 144;
  struct Raw {
    u32x4 h, c;
  };
  __device__ static int64_t row_bytes(int K) { return (int64_t)(K >> 8) * 144; }
  __device__ static void load(const uint8_t* __restrict__ row, const BlockLane& L, Raw& r) {
    r.h = *reinterpret_cast<const u32x4*>(row + L.o16);
    r.c = *reinterpret_cast<const u32x4*>(row + L.o2);
  }
  __device__ static float apply(const Raw& r, const BlockLane& /*L*/, const XPrep& xp, int sub) {
    // 6-bit fields: sc at bit 6*sub, mn at bit 48 + 6*sub of {w, z, y}
    const int ps = 6 * sub, pm = 48 + 6 * sub;
    const uint32_t slo = ps < 32 ? r.h.y : r.h.z, shi = ps < 32 ? r.h.z : r.h.w;
    const uint32_t mlo = pm < 64 ? r.h.z : r.h.w, mhi = pm < 64 ? r.h.w : 0u;
    const uint32_t sc = __builtin_amdgcn_alignbit(shi, slo, ps & 31) & 63u;
    const uint32_t mn = __builtin_amdgcn_alignbit(mhi, mlo, pm & 31) & 63u;
    const float S = f16_bits_to_f32(r.h.x) * (float)sc;
    const float O = f16_bits_to_f32(r.h.x >> 16) * (float)mn;
    const uint32_t c[4] = {r.c.x, r.c.y, r.c.z, r.c.w};
    const int32_t Q = nib_dot(c, xp, 0);  // sum q X, exact
    return fmaf(S, (float)Q, -O * (float)xp.sx);
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

constexpr int kRows = 8;  // rows per workgroup

// kOdd: the row stride is 2 mod 4 (K/32 odd for Q4_0/Q8_0), so even and odd
// rows have different block alignments; row m0 + r has parity r & 1 since
// m0 is a multiple of kRows (even).
template <class F, bool kOdd>
__global__ __launch_bounds__(kMaxStrips * kWave) void gemv_kernel(const uint8_t* __restrict__ B,
                                                                  const float* __restrict__ x,
                                                                  float* __restrict__ y,
                                                                  int64_t M, int K) {
  constexpr int R = kRows;
  __shared__ float red[kMaxStrips][R];
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
      BlockLane L[2];
      if (F::kBytes == 144) {  // Q4_K: header and the sub-block's 16 code bytes
        const uint32_t o = (uint32_t)(j >> 3) * 144u;
        L[0].o16 = o;
        L[0].o2 = o + 16u + 16u * (uint32_t)(j & 7);
        L[0].sel = 0;
        L[0].mis = false;
        L[1] = L[0];
      } else {
        const uint32_t o = (uint32_t)j * (uint32_t)F::kBytes;
        L[0] = block_lane(o, 0u, F::kBytes);
        L[1] = block_lane(o, kOdd ? 2u : 0u, F::kBytes);
      }
      f32x4 xv[8];
      load_x32(x + (int64_t)j * 32, xv);
      typename F::Raw raw[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        // rows past M re-read the last row of the same parity (their sums
        // are discarded); with an odd stride M >= 2 here
        int64_t m = m0 + r;
        if (m >= M) m = kOdd ? M - 1 - ((M - 1 - r) & 1) : M - 1;
        F::load(B + m * rb, L[kOdd ? (r & 1) : 0], raw[r]);
      }
      // every load above is issued before any is consumed
      __builtin_amdgcn_sched_barrier(0);
      XPrep xp;
      prep_x(xv, xp);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float t = F::apply(raw[r], L[kOdd ? (r & 1) : 0], xp, lane & 7);
        part[r] = fmaf(t, xp.inv, part[r]);
      }
    }
  }

  const float sum = wave_reduce_rows<R>(part, lane);
  constexpr int kShift = 6 - log2i<R>();
  const int row = (lane >> kShift) & (R - 1);
  if ((lane & ((1 << kShift) - 1)) == 0) red[wv][row] = sum;
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
  if (waves > kMaxStrips) waves = kMaxStrips;
  const int64_t grid = (M + kRows - 1) / kRows;
  // a single row has only the even parity: the aligned variant covers it
  const bool odd = F::kBytes != 144 && (ns & 1) != 0 && M > 1;
  if (odd)
    hipLaunchKernelGGL((gemv_kernel<F, true>), dim3((unsigned)grid), dim3(waves * kWave), 0,
                       stream, static_cast<const uint8_t*>(blocks), x, y, M, (int)K);
  else
    hipLaunchKernelGGL((gemv_kernel<F, false>), dim3((unsigned)grid), dim3(waves * kWave), 0,
                       stream, static_cast<const uint8_t*>(blocks), x, y, M, (int)K);
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
