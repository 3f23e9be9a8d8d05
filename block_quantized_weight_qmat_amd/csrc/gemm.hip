// gemm.hip — prefill Y[n][m] = sum_k dequant(W)[m][k] * dequant(Xq8)[n][k].
//
// Source: "05. llama.cpp：从 GGUF 文件到本地推理服务", section "性能直觉：带宽
// 决定 Decode，算力决定 Prefill": a prompt of hundreds of tokens reuses every
// weight read many times, so prefill is bound by arithmetic, not bandwidth.
// Here the arithmetic is an int8 matrix-core product per 32-element block.
//
// Per K-block b (32 elements) and output (m, n):
//   S[m,n,b] = sum_{i<32} wq[m,32b+i] * xq[n,32b+i]        (exact int32, MFMA)
//   Y[n][m] += dw[m,b] * dx[n,b] * S[m,n,b]                 (fp32, VALU)
// wq is the signed code (c - 8) for Q4_0, q for Q8_0, and the unsigned code q
// for Q4_K-style, whose per-sub-block offset adds -O[m,b] * dx[n,b] * sum(xq).
//
// Scale step in two fp32 FMAs per element: the MFMA accumulates onto the
// integer constant 0x4B400000, the bit pattern of 1.5 * 2^23, so its int32
// result 0x4B400000 + S (|S| < 2^22) is, read as a float, exactly
// 12582912 + S. Then t = fma(F, dx, -12582912 * dx) = dx * S with one
// rounding (12582912 * dx is exact for an fp16 dx), and acc = fma(t, dw, acc).
//
// Tiling: a 256-thread workgroup computes a 128 (m) x 64 (n) tile; wave w owns
// rows 32w..32w+31 and both 32-column halves (two MFMA tiles). Each stage
// brings 4 K-blocks of W and X into LDS, unpacked to int8 rows of 32 bytes
// plus fp32 scales, so every MFMA operand is one 16-byte LDS read.
#include "qmat_device.hpp"
#include "qmat_launch.hpp"

namespace qmat {
namespace {

constexpr int kBM = 128;
constexpr int kBN = 64;
constexpr int kKB = 4;  // K-blocks per stage
constexpr int kThreads = 256;
constexpr uint32_t kMagicI = 0x4B400000u;  // 1.5 * 2^23 as fp32 bits
constexpr float kMagicF = 12582912.0f;

struct Stage {
  int8_t wq[kKB][kBM][32];
  float wd[kKB][kBM];
  float wo[kKB][kBM];
  int8_t xq[kKB][kBN][32];
  float xd[kKB][kBN];
  float xs[kKB][kBN];
};

// Nibbles of 4 code bytes -> 4 signed bytes (c - 8), for the low or high
// nibble: ((c | 0x80) - 8) ^ 0x80 per byte, with no borrow between bytes.
__device__ __forceinline__ uint32_t nib_signed(uint32_t w, int shift) {
  const uint32_t c = (w >> shift) & 0x0F0F0F0Fu;
  return ((c | 0x80808080u) - 0x08080808u) ^ 0x80808080u;
}

__device__ __forceinline__ uint32_t nib_unsigned(uint32_t w, int shift) {
  return (w >> shift) & 0x0F0F0F0Fu;
}

// Load a 32-element block of 18 (Q4_0) or 34 (Q8_0) bytes at an even
// address: returns the fp16 scale bits and the code bytes realigned to
// 4-byte words (see the same loads in the GEMV).
__device__ __forceinline__ void load_q4_0(const uint8_t* b, uint32_t& h, uint32_t (&c)[4]) {
  const uint32_t a = (uint32_t)(reinterpret_cast<uintptr_t>(b) & 2u);
  const u32x4 v = *reinterpret_cast<const u32x4_a4*>(b + a);
  const uint32_t s16 = *reinterpret_cast<const uint16_t*>(b + (a ? 0 : 16));
  const uint32_t sel = a ? 0x03020100u : 0x05040302u;
  c[0] = perm_b32(v.y, v.x, sel);
  c[1] = perm_b32(v.z, v.y, sel);
  c[2] = perm_b32(v.w, v.z, sel);
  c[3] = perm_b32(s16, v.w, sel);
  h = a ? s16 : (v.x & 0xFFFFu);
}

__device__ __forceinline__ void load_q8_0(const uint8_t* b, uint32_t& h, uint32_t (&c)[8]) {
  const uint32_t a = (uint32_t)(reinterpret_cast<uintptr_t>(b) & 2u);
  const u32x4 v0 = *reinterpret_cast<const u32x4_a4*>(b + a);
  const u32x4 v1 = *reinterpret_cast<const u32x4_a4*>(b + a + 16);
  const uint32_t s16 = *reinterpret_cast<const uint16_t*>(b + (a ? 0 : 32));
  const uint32_t sel = a ? 0x03020100u : 0x05040302u;
  const uint32_t w[9] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w, s16};
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = perm_b32(w[i + 1], w[i], sel);
  h = a ? s16 : (v0.x & 0xFFFFu);
}

__device__ __forceinline__ void store16(int8_t* dst, uint32_t a, uint32_t b, uint32_t c,
                                        uint32_t d) {
  u32x4 v = {a, b, c, d};
  *reinterpret_cast<u32x4*>(dst) = v;
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const uint8_t* __restrict__ Wb,
                                                        const uint8_t* __restrict__ Xb,
                                                        float* __restrict__ Y, int64_t M,
                                                        int K, int64_t N, int64_t tiles_n,
                                                        int64_t ntiles) {
  __shared__ __attribute__((aligned(16))) Stage st;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int nb = K >> 5;  // 32-element blocks along K
  const int64_t wrb = FMT == kFmtQ4_0 ? (int64_t)nb * 18
                      : FMT == kFmtQ8_0 ? (int64_t)nb * 34
                                        : (int64_t)(K >> 8) * 144;
  const int64_t xrb = (int64_t)nb * 34;
  i32x16 cmagic;
#pragma unroll
  for (int i = 0; i < 16; ++i) cmagic[i] = (int)kMagicI;

  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t tm = tile / tiles_n, tn = tile - tm * tiles_n;
    const int64_t m0 = tm * kBM, n0 = tn * kBN;

    float acc[2][16];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][i] = 0.0f;

    for (int kb = 0; kb < nb; kb += kKB) {
      // ---- stage W: 128 rows x 4 blocks, two (row, block) items per thread
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int item = tid + it * kThreads;
        const int rr = item >> 2, bb = item & 3;
        const int b = kb + bb;
        if (b < nb) {
          const int64_t m = (m0 + rr < M) ? m0 + rr : M - 1;
          const uint8_t* row = Wb + m * wrb;
          if (FMT == kFmtQ4_0) {
            uint32_t h, c[4];
            load_q4_0(row + (int64_t)b * 18, h, c);
            store16(&st.wq[bb][rr][0], nib_signed(c[0], 0), nib_signed(c[1], 0),
                    nib_signed(c[2], 0), nib_signed(c[3], 0));
            store16(&st.wq[bb][rr][16], nib_signed(c[0], 4), nib_signed(c[1], 4),
                    nib_signed(c[2], 4), nib_signed(c[3], 4));
            st.wd[bb][rr] = f16_bits_to_f32(h);
          } else if (FMT == kFmtQ8_0) {
            uint32_t h, c[8];
            load_q8_0(row + (int64_t)b * 34, h, c);
            store16(&st.wq[bb][rr][0], c[0], c[1], c[2], c[3]);
            store16(&st.wq[bb][rr][16], c[4], c[5], c[6], c[7]);
            st.wd[bb][rr] = f16_bits_to_f32(h);
          } else {
            const uint8_t* sb = row + (int64_t)(b >> 3) * 144;
            const int sub = b & 7;
            const u32x4 hd = *reinterpret_cast<const u32x4*>(sb);
            const u32x4 cv = *reinterpret_cast<const u32x4*>(sb + 16 + 16 * sub);
            const int ps = 6 * sub, pm = 48 + 6 * sub;
            const uint32_t slo = ps < 32 ? hd.y : hd.z, shi = ps < 32 ? hd.z : hd.w;
            const uint32_t mlo = pm < 64 ? hd.z : hd.w, mhi = pm < 64 ? hd.w : 0u;
            const uint32_t sc = __builtin_amdgcn_alignbit(shi, slo, ps & 31) & 63u;
            const uint32_t mn = __builtin_amdgcn_alignbit(mhi, mlo, pm & 31) & 63u;
            store16(&st.wq[bb][rr][0], nib_unsigned(cv.x, 0), nib_unsigned(cv.y, 0),
                    nib_unsigned(cv.z, 0), nib_unsigned(cv.w, 0));
            store16(&st.wq[bb][rr][16], nib_unsigned(cv.x, 4), nib_unsigned(cv.y, 4),
                    nib_unsigned(cv.z, 4), nib_unsigned(cv.w, 4));
            st.wd[bb][rr] = f16_bits_to_f32(hd.x) * (float)sc;
            st.wo[bb][rr] = f16_bits_to_f32(hd.x >> 16) * (float)mn;
          }
        }
      }
      // ---- stage X: 64 columns x 4 blocks, one item per thread
      {
        const int cc = tid >> 2, bb = tid & 3;
        const int b = kb + bb;
        if (b < nb) {
          const int64_t n = (n0 + cc < N) ? n0 + cc : N - 1;
          uint32_t h, c[8];
          load_q8_0(Xb + n * xrb + (int64_t)b * 34, h, c);
          store16(&st.xq[bb][cc][0], c[0], c[1], c[2], c[3]);
          store16(&st.xq[bb][cc][16], c[4], c[5], c[6], c[7]);
          const float dx = f16_bits_to_f32(h);
          st.xd[bb][cc] = dx;
          if (FMT == kFmtQ4_K) {
            int qs = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) qs = __builtin_amdgcn_sdot4((int)c[i], 0x01010101, qs, false);
            st.xs[bb][cc] = dx * (float)qs;
          }
        }
      }
      __syncthreads();

      // ---- compute
#pragma unroll
      for (int bb = 0; bb < kKB; ++bb) {
        if (kb + bb < nb) {
          const i32x4 a = *reinterpret_cast<const i32x4*>(&st.wq[bb][wv * 32 + l32][16 * half]);
          float dw[16], wo[16];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(&st.wd[bb][wv * 32 + 8 * q + 4 * half]);
            dw[4 * q + 0] = t.x;
            dw[4 * q + 1] = t.y;
            dw[4 * q + 2] = t.z;
            dw[4 * q + 3] = t.w;
            if (FMT == kFmtQ4_K) {
              const f32x4 o = *reinterpret_cast<const f32x4*>(&st.wo[bb][wv * 32 + 8 * q + 4 * half]);
              wo[4 * q + 0] = o.x;
              wo[4 * q + 1] = o.y;
              wo[4 * q + 2] = o.z;
              wo[4 * q + 3] = o.w;
            }
          }
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const i32x4 bv = *reinterpret_cast<const i32x4*>(&st.xq[bb][t * 32 + l32][16 * half]);
            const float dx = st.xd[bb][t * 32 + l32];
            const i32x16 d = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bv, cmagic, 0, 0, 0);
            const f32x16 df = __builtin_bit_cast(f32x16, d);
            const float c1 = -kMagicF * dx;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const float f = df[i];
              const float s = fmaf(f, dx, c1);
              acc[t][i] = fmaf(s, dw[i], acc[t][i]);
            }
            if (FMT == kFmtQ4_K) {
              const float xs = st.xs[bb][t * 32 + l32];
#pragma unroll
              for (int i = 0; i < 16; ++i) acc[t][i] = fmaf(-wo[i], xs, acc[t][i]);
            }
          }
        }
      }
      __syncthreads();
    }

    // ---- store: lane holds column n = n0 + 32t + l32, rows
    //      m = m0 + 32 wv + 8q + 4 half + r  (q, r in 0..3)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t n = n0 + 32 * t + l32;
      if (n >= N) continue;
      float* yrow = Y + n * M;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t mb = m0 + wv * 32 + 8 * q + 4 * half;
        if (mb + 3 < M && (M & 3) == 0) {
          f32x4 v = {acc[t][4 * q], acc[t][4 * q + 1], acc[t][4 * q + 2], acc[t][4 * q + 3]};
          *reinterpret_cast<f32x4*>(yrow + mb) = v;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (mb + r < M) yrow[mb + r] = acc[t][4 * q + r];
        }
      }
    }
  }
}

constexpr int64_t kMaxGrid = 1 << 24;

}  // namespace

hipError_t launch_gemm(int fmt, const void* blocks, const void* Xq8, float* Y, int64_t M,
                       int64_t K, int64_t N, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
  const int64_t ntiles = tiles_m * tiles_n;
  const unsigned grid = (unsigned)(ntiles < kMaxGrid ? ntiles : kMaxGrid);
  const uint8_t* W = static_cast<const uint8_t*>(blocks);
  const uint8_t* X = static_cast<const uint8_t*>(Xq8);
  switch (fmt) {
    case kFmtQ4_0:
      hipLaunchKernelGGL(gemm_kernel<kFmtQ4_0>, dim3(grid), dim3(kThreads), 0, stream, W, X, Y,
                         M, (int)K, N, tiles_n, ntiles);
      break;
    case kFmtQ8_0:
      hipLaunchKernelGGL(gemm_kernel<kFmtQ8_0>, dim3(grid), dim3(kThreads), 0, stream, W, X, Y,
                         M, (int)K, N, tiles_n, ntiles);
      break;
    default:
      hipLaunchKernelGGL(gemm_kernel<kFmtQ4_K>, dim3(grid), dim3(kThreads), 0, stream, W, X, Y,
                         M, (int)K, N, tiles_n, ntiles);
      break;
  }
  return hipGetLastError();
}

}  // namespace qmat
