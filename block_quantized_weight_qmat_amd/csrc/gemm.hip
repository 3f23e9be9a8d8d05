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
// Tiling: a workgroup computes a 128 (m) x 64 (n) tile; each of its eight
// compute waves owns one 32 x 32 MFMA tile of it (two compute waves per SIMD:
// a single wave issues dependent-free fp32 FMAs at only half the rate). A stage holds 8
// K-blocks of W and X in LDS, unpacked to int8 rows of 32 bytes plus fp32
// scales, so every MFMA operand is one 16-byte LDS read.
//
// Pipeline: a workgroup has eight compute waves and four loader waves. Loader
// waves hold kDepth stages of raw blocks in registers (stage s+1+kDepth is
// requested while stage s is computed), unpack stage s+1 into the free half of a
// two-stage LDS buffer, and meet the compute waves at one barrier per stage.
// Keeping several stages in flight per CU is what the memory latency needs;
// compute waves keep only accumulators and operands.
//
// Tile order: consecutive workgroup ids land on different XCDs (round
// robin), so ids are remapped to give each XCD a contiguous band of m-tiles
// with all their n-tiles: W rows are then read by one XCD's L2 only, and the
// smaller X is what every XCD re-reads.
#include "qmat_device.hpp"
#include "qmat_launch.hpp"

namespace qmat {
namespace {

#ifndef QMAT_GEMM_DEPTH
#define QMAT_GEMM_DEPTH 1
#endif
constexpr int kBM = 128;
constexpr int kBN = 64;
constexpr int kKB = 8;  // K-blocks per stage
#ifndef QMAT_GEMM_NT
#define QMAT_GEMM_NT 2
#endif
// each compute wave owns 32 rows x (32 * kNT) columns of the 128 x 64 tile
constexpr int kNT = QMAT_GEMM_NT;  // 32-column MFMA tiles per compute wave
constexpr int kThreads = 512 / kNT;  // compute threads
constexpr int kLoadThreads = 256; // loader threads (4 waves)
constexpr int kDepth = QMAT_GEMM_DEPTH;  // stages a loader thread holds in registers
constexpr uint32_t kMagicI = 0x4B400000u;  // 1.5 * 2^23 as fp32 bits
constexpr float kMagicF = 12582912.0f;

// One K-stage in LDS. Code bytes are stored per block as [half][row][16 B]
// (the two 16-byte halves of a row's 32 int8 codes in separate planes), so
// the lanes of an MFMA operand read consecutive 16-byte chunks. Each block's
// plane (and each scale row) is padded by 16 bytes: the eight threads that
// write eight blocks of one row then hit eight different bank groups.
struct Stage {
  static constexpr int kWPlane = 2 * kBM * 16 + 16;
  static constexpr int kXPlane = 2 * kBN * 16 + 16;
  int8_t wq[kKB][kWPlane];
  int8_t xq[kKB][kXPlane];
  float wd[kKB][kBM + 4];
  float wo[kKB][kBM + 4];
  float xd[kKB][kBN + 4];
  float xs[kKB][kBN + 4];
  __device__ int8_t* w(int bb, int half, int row) { return &wq[bb][(half * kBM + row) * 16]; }
  __device__ int8_t* x(int bb, int half, int col) { return &xq[bb][(half * kBN + col) * 16]; }
  __device__ const int8_t* w(int bb, int half, int row) const {
    return &wq[bb][(half * kBM + row) * 16];
  }
  __device__ const int8_t* x(int bb, int half, int col) const {
    return &xq[bb][(half * kBN + col) * 16];
  }
};

// Nibbles of 4 code bytes -> 4 signed bytes (c - 8), for the low or high
// nibble: per byte, c + 0x78 stays below 0x88 (no carry between bytes) and
// flipping its top bit gives c - 8 as a signed byte.
__device__ __forceinline__ uint32_t nib_signed(uint32_t w, int shift) {
  const uint32_t c = (w >> shift) & 0x0F0F0F0Fu;
  return (c + 0x78787878u) ^ 0x80808080u;
}

__device__ __forceinline__ uint32_t nib_unsigned(uint32_t w, int shift) {
  return (w >> shift) & 0x0F0F0F0Fu;
}

__device__ __forceinline__ void store16(int8_t* dst, uint32_t a, uint32_t b, uint32_t c,
                                        uint32_t d) {
  u32x4 v = {a, b, c, d};
  *reinterpret_cast<u32x4*>(dst) = v;
}

// Global data of one stage held in registers between its load and its LDS
// write: four W items (row, block) and two X items per thread.
template <int FMT>
struct StageRegs {
  static constexpr int kWItems = kBM * kKB / kLoadThreads;  // 4
  static constexpr int kXItems = kBN * kKB / kLoadThreads;  // 2
  u32x4 wa[kWItems], wb[kWItems];  // Q8_0: 2 x 16 B; Q4_0: 16 B; Q4_K: header, codes
  uint32_t ws[kWItems];            // 2-byte piece (Q4_0/Q8_0)
  u32x4 xa[kXItems], xb[kXItems];
  uint32_t xs[kXItems];
};

// Byte address parity: blocks of 18 or 34 bytes start at 0 or 2 mod 4.
__device__ __forceinline__ void load_blk(const uint8_t* b, int bytes, u32x4& va, u32x4& vb,
                                         uint32_t& s2) {
  const uint32_t a = (uint32_t)(reinterpret_cast<uintptr_t>(b) & 2u);
  va = *reinterpret_cast<const u32x4_a4*>(b + a);
  if (bytes == 34) vb = *reinterpret_cast<const u32x4_a4*>(b + a + 16);
  s2 = *reinterpret_cast<const uint16_t*>(b + (a ? 0 : bytes - 2));
}

// Realign the code words of a block loaded by load_blk; h = fp16 scale bits.
__device__ __forceinline__ void realign(const uint8_t* b, int bytes, const u32x4& va,
                                        const u32x4& vb, uint32_t s2, uint32_t& h,
                                        uint32_t (&c)[8]) {
  const uint32_t a = (uint32_t)(reinterpret_cast<uintptr_t>(b) & 2u);
  const uint32_t sel = a ? 0x03020100u : 0x05040302u;
  if (bytes == 18) {
    c[0] = perm_b32(va.y, va.x, sel);
    c[1] = perm_b32(va.z, va.y, sel);
    c[2] = perm_b32(va.w, va.z, sel);
    c[3] = perm_b32(s2, va.w, sel);
  } else {
    const uint32_t w[9] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w, s2};
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = perm_b32(w[i + 1], w[i], sel);
  }
  h = a ? s2 : (va.x & 0xFFFFu);
}

// The MFMA tile of one K-block: rows 32wm..32wm+31 against columns
// 32wn..32wn+31 of the stage; the accumulator input is the magic constant.
__device__ __forceinline__ void mfma_block(const Stage& cur, int bb, int wm, int wn, int l32,
                                           int half, const i32x16& cmagic, i32x16& d) {
  const i32x4 a = *reinterpret_cast<const i32x4*>(cur.w(bb, half, wm * 32 + l32));
  const i32x4 bv = *reinterpret_cast<const i32x4*>(cur.x(bb, half, wn * 32 + l32));
  d = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bv, cmagic, 0, 0, 0);
}

// acc += dw * dx * S for the 16 values per lane (lane l holds column l % 32
// and rows 8q + 4(l / 32) + r of the tile); Q4_K-style also subtracts
// O * dx * sum(xq).
template <int FMT, int NT>
__device__ __forceinline__ void epilogue(const Stage& cur, int bb, int wm, int wn0, int l32,
                                         int half, const i32x16 (&d)[NT], float (&acc)[NT][16]) {
  float dw[16], wo[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(&cur.wd[bb][wm * 32 + 8 * q + 4 * half]);
    dw[4 * q + 0] = t.x;
    dw[4 * q + 1] = t.y;
    dw[4 * q + 2] = t.z;
    dw[4 * q + 3] = t.w;
    if (FMT == kFmtQ4_K) {
      const f32x4 o = *reinterpret_cast<const f32x4*>(&cur.wo[bb][wm * 32 + 8 * q + 4 * half]);
      wo[4 * q + 0] = o.x;
      wo[4 * q + 1] = o.y;
      wo[4 * q + 2] = o.z;
      wo[4 * q + 3] = o.w;
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int col = (wn0 + t) * 32 + l32;
    const float dx = cur.xd[bb][col];
    const f32x16 df = __builtin_bit_cast(f32x16, d[t]);
    const float c1 = -kMagicF * dx;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float sdx = fmaf(df[i], dx, c1);
      acc[t][i] = fmaf(sdx, dw[i], acc[t][i]);
    }
    if (FMT == kFmtQ4_K) {
      const float xs = cur.xs[bb][col];
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][i] = fmaf(-wo[i], xs, acc[t][i]);
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(kThreads + kLoadThreads) void gemm_kernel(const uint8_t* __restrict__ Wb,
                                                            const uint8_t* __restrict__ Xb,
                                                            float* __restrict__ Y, int64_t M,
                                                            int K, int64_t N, int64_t tiles_n,
                                                            int64_t ntiles) {
  __shared__ __attribute__((aligned(16))) Stage st[2];
  typedef StageRegs<FMT> R;
  const bool loader = threadIdx.x >= kThreads;
  const int tid = loader ? threadIdx.x - kThreads : threadIdx.x;  // index within its group
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int nb = K >> 5;  // 32-element blocks along K
  const int nstage = (nb + kKB - 1) / kKB;
  constexpr int wbytes = FMT == kFmtQ4_0 ? 18 : FMT == kFmtQ8_0 ? 34 : 144;
  const int64_t wrb = FMT == kFmtQ4_K ? (int64_t)(K >> 8) * 144 : (int64_t)nb * wbytes;
  const int64_t xrb = (int64_t)nb * 34;

  // XCD-aware order: XCD x = id % 8 takes linear tiles [x * per, (x+1) * per)
  int64_t lin = blockIdx.x;
  if ((ntiles & 7) == 0 && (int64_t)gridDim.x == ntiles) {
    const int64_t per = ntiles >> 3;
    lin = (int64_t)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
  }

  for (int64_t tile = lin; tile < ntiles; tile += gridDim.x) {
    const int64_t tm = tile / tiles_n, tn = tile - tm * tiles_n;
    const int64_t m0 = tm * kBM, n0 = tn * kBN;

    if (loader) {
      // item -> (row, block): 8 consecutive threads cover one row's 8 blocks.
      // Rows are addressed from the tile's first row (a wave-uniform base)
      // with 32-bit offsets; rows past M re-read the last row.
      const uint8_t* wtile = Wb + m0 * wrb;
      const uint8_t* xtile = Xb + n0 * xrb;
      const uint32_t wlast = (uint32_t)min<int64_t>(kBM - 1, M - 1 - m0);
      const uint32_t xlast = (uint32_t)min<int64_t>(kBN - 1, N - 1 - n0);
      auto w_row = [&](int it) -> const uint8_t* {
        const uint32_t r = min((uint32_t)((tid + it * kLoadThreads) >> 3), wlast);
        return wtile + r * (uint32_t)wrb;
      };
      auto x_row = [&](int it) -> const uint8_t* {
        const uint32_t r = min((uint32_t)((tid + it * kLoadThreads) >> 3), xlast);
        return xtile + r * (uint32_t)xrb;
      };
      // global -> registers for stage s (blocks past nb are not loaded)
      auto load_stage = [&](int s, R& r) {
#pragma unroll
        for (int it = 0; it < R::kWItems; ++it) {
          const int b = s * kKB + ((tid + it * kLoadThreads) & 7);
          if (b < nb) {
            const uint8_t* row = w_row(it);
            if (FMT == kFmtQ4_K) {
              const uint8_t* sb = row + (int64_t)(b >> 3) * 144;
              r.wa[it] = *reinterpret_cast<const u32x4*>(sb);
              r.wb[it] = *reinterpret_cast<const u32x4*>(sb + 16 + 16 * (b & 7));
            } else {
              load_blk(row + (int64_t)b * wbytes, wbytes, r.wa[it], r.wb[it], r.ws[it]);
            }
          }
        }
#pragma unroll
        for (int it = 0; it < R::kXItems; ++it) {
          const int b = s * kKB + ((tid + it * kLoadThreads) & 7);
          if (b < nb) load_blk(x_row(it) + (int64_t)b * 34, 34, r.xa[it], r.xb[it], r.xs[it]);
        }
      };
      // registers -> LDS buffer for stage s
      auto write_stage = [&](int s, const R& r, Stage& dst) {
#pragma unroll
        for (int it = 0; it < R::kWItems; ++it) {
          const int item = tid + it * kLoadThreads;
          const int rr = item >> 3, bb = item & 7;
          const int b = s * kKB + bb;
          if (b < nb) {
            if (FMT == kFmtQ4_0) {
              uint32_t h, c[8];
              realign(w_row(it) + (int64_t)b * 18, 18, r.wa[it], r.wb[it], r.ws[it], h, c);
              store16(dst.w(bb, 0, rr), nib_signed(c[0], 0), nib_signed(c[1], 0),
                      nib_signed(c[2], 0), nib_signed(c[3], 0));
              store16(dst.w(bb, 1, rr), nib_signed(c[0], 4), nib_signed(c[1], 4),
                      nib_signed(c[2], 4), nib_signed(c[3], 4));
              dst.wd[bb][rr] = f16_bits_to_f32(h);
            } else if (FMT == kFmtQ8_0) {
              uint32_t h, c[8];
              realign(w_row(it) + (int64_t)b * 34, 34, r.wa[it], r.wb[it], r.ws[it], h, c);
              store16(dst.w(bb, 0, rr), c[0], c[1], c[2], c[3]);
              store16(dst.w(bb, 1, rr), c[4], c[5], c[6], c[7]);
              dst.wd[bb][rr] = f16_bits_to_f32(h);
            } else {
              const u32x4 hd = r.wa[it], cv = r.wb[it];
              const int sub = b & 7;
              const int ps = 6 * sub, pm = 48 + 6 * sub;
              const uint32_t slo = ps < 32 ? hd.y : hd.z, shi = ps < 32 ? hd.z : hd.w;
              const uint32_t mlo = pm < 64 ? hd.z : hd.w, mhi = pm < 64 ? hd.w : 0u;
              const uint32_t sc = __builtin_amdgcn_alignbit(shi, slo, ps & 31) & 63u;
              const uint32_t mn = __builtin_amdgcn_alignbit(mhi, mlo, pm & 31) & 63u;
              store16(dst.w(bb, 0, rr), nib_unsigned(cv.x, 0), nib_unsigned(cv.y, 0),
                      nib_unsigned(cv.z, 0), nib_unsigned(cv.w, 0));
              store16(dst.w(bb, 1, rr), nib_unsigned(cv.x, 4), nib_unsigned(cv.y, 4),
                      nib_unsigned(cv.z, 4), nib_unsigned(cv.w, 4));
              dst.wd[bb][rr] = f16_bits_to_f32(hd.x) * (float)sc;
              dst.wo[bb][rr] = f16_bits_to_f32(hd.x >> 16) * (float)mn;
            }
          }
        }
#pragma unroll
        for (int it = 0; it < R::kXItems; ++it) {
          const int item = tid + it * kLoadThreads;
          const int cc = item >> 3, bb = item & 7;
          const int b = s * kKB + bb;
          if (b < nb) {
            uint32_t h, c[8];
            realign(x_row(it) + (int64_t)b * 34, 34, r.xa[it], r.xb[it], r.xs[it], h, c);
            store16(dst.x(bb, 0, cc), c[0], c[1], c[2], c[3]);
            store16(dst.x(bb, 1, cc), c[4], c[5], c[6], c[7]);
            const float dx = f16_bits_to_f32(h);
            dst.xd[bb][cc] = dx;
            if (FMT == kFmtQ4_K) {
              int qs = 0;
#pragma unroll
              for (int i = 0; i < 8; ++i)
                qs = __builtin_amdgcn_sdot4((int)c[i], 0x01010101, qs, false);
              dst.xs[bb][cc] = dx * (float)qs;
            }
          }
        }
      };

      // Register set k holds stages k, k + kDepth, ...: set indices stay
      // compile-time constants by stepping kDepth stages per iteration.
      R regs[kDepth];
#pragma unroll
      for (int k = 0; k < kDepth; ++k)
        if (k < nstage) load_stage(k, regs[k]);
      if (nstage > 0) {
        write_stage(0, regs[0], st[0]);
        if (kDepth < nstage) load_stage(kDepth, regs[0]);
      }
      __syncthreads();
      // step s: write stage s+1 (set (s+1) % kDepth), refill it with stage
      // s+1+kDepth
      auto step = [&](int s, R& r) {
        if (s + 1 < nstage) {
          write_stage(s + 1, r, st[(s + 1) & 1]);
          if (s + 1 + kDepth < nstage) load_stage(s + 1 + kDepth, r);
        }
        __syncthreads();
      };
      int s = 0;
      for (; s + kDepth <= nstage; s += kDepth) {
#pragma unroll
        for (int k = 0; k < kDepth; ++k) step(s + k, regs[(k + 1) % kDepth]);
      }
#pragma unroll
      for (int k = 0; k + 1 < kDepth; ++k)
        if (s + k < nstage) step(s + k, regs[(k + 1) % kDepth]);
    } else {
      i32x16 cmagic;
#pragma unroll
      for (int i = 0; i < 16; ++i) cmagic[i] = (int)kMagicI;
      const int wm = wv & 3, wn0 = (wv >> 2) * kNT;  // rows 32wm.., column tiles wn0..
      float acc[kNT][16];
#pragma unroll
      for (int t = 0; t < kNT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][i] = 0.0f;

      __syncthreads();  // stage 0 is in LDS
      for (int s = 0; s < nstage; ++s) {
        const Stage& cur = st[s & 1];
        const int nbs = min(kKB, nb - s * kKB);
        if (nbs == kKB) {
          // full stage: the MFMAs of block bb+1 are issued before the scale
          // epilogue of block bb, so the matrix core and the VALU overlap
          i32x16 d[2][kNT];
#pragma unroll
          for (int t = 0; t < kNT; ++t) mfma_block(cur, 0, wm, wn0 + t, l32, half, cmagic, d[0][t]);
#pragma unroll
          for (int bb = 0; bb < kKB; ++bb) {
            if (bb + 1 < kKB)
#pragma unroll
              for (int t = 0; t < kNT; ++t)
                mfma_block(cur, bb + 1, wm, wn0 + t, l32, half, cmagic, d[(bb + 1) & 1][t]);
            epilogue<FMT, kNT>(cur, bb, wm, wn0, l32, half, d[bb & 1], acc);
          }
        } else {
          for (int bb = 0; bb < nbs; ++bb) {
            i32x16 d[kNT];
#pragma unroll
            for (int t = 0; t < kNT; ++t) mfma_block(cur, bb, wm, wn0 + t, l32, half, cmagic, d[t]);
            epilogue<FMT, kNT>(cur, bb, wm, wn0, l32, half, d, acc);
          }
        }
        __syncthreads();
      }

      // ---- store: lane holds column n = n0 + 32(wn0 + t) + l32, rows
      //      m = m0 + 32 wm + 8q + 4 half + r  (q, r in 0..3)
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
        const int64_t n = n0 + 32 * (wn0 + t) + l32;
        if (n >= N) continue;
        float* yrow = Y + n * M;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t mb = m0 + wm * 32 + 8 * q + 4 * half;
          if (mb + 3 < M && (M & 3) == 0) {
            f32x4 v = {acc[t][4 * q], acc[t][4 * q + 1], acc[t][4 * q + 2], acc[t][4 * q + 3]};
            *reinterpret_cast<f32x4*>(yrow + mb) = v;
          } else {
#pragma unroll
            for (int r2 = 0; r2 < 4; ++r2)
              if (mb + r2 < M) yrow[mb + r2] = acc[t][4 * q + r2];
          }
        }
      }
    }
    // the next tile reuses both LDS stages
    __syncthreads();
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
      hipLaunchKernelGGL(gemm_kernel<kFmtQ4_0>, dim3(grid), dim3(kThreads + kLoadThreads), 0, stream, W, X, Y,
                         M, (int)K, N, tiles_n, ntiles);
      break;
    case kFmtQ8_0:
      hipLaunchKernelGGL(gemm_kernel<kFmtQ8_0>, dim3(grid), dim3(kThreads + kLoadThreads), 0, stream, W, X, Y,
                         M, (int)K, N, tiles_n, ntiles);
      break;
    default:
      hipLaunchKernelGGL(gemm_kernel<kFmtQ4_K>, dim3(grid), dim3(kThreads + kLoadThreads), 0, stream, W, X, Y,
                         M, (int)K, N, tiles_n, ntiles);
      break;
  }
  return hipGetLastError();
}

}  // namespace qmat
