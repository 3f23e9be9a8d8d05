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
// wq is 16 (c - 8) for Q4_0 (its dw is stored divided by 16, exactly), q for
// Q8_0, and the unsigned code q for Q4_K-style, whose per-sub-block offset
// adds -O[m,b] * dx[n,b] * sum(xq).
// Q6_K-style blocks (wq = c - 32) have a scale per 16-element half: each half
// is its own MFMA (the other half's operand lanes zeroed) and scaled alone.
//
// Scale step in two fp32 FMAs per element: the MFMA accumulates onto the
// integer constant 0x4B400000, the bit pattern of 1.5 * 2^23, so its int32
// result 0x4B400000 + S (|S| < 2^22) is, read as a float, exactly
// 12582912 + S. Then t = fma(F, dx, -12582912 * dx) = dx * S with one
// rounding (12582912 * dx is exact for an fp16 dx), and acc = fma(t, dw, acc).
//
// Tiling: a workgroup computes a 128 (m) x 64 (n) tile: four 32 x 64 wave
// tiles (two 32 x 32 MFMA tiles each). Each wave tile is shared by two
// compute waves on the same SIMD, which take the first and the second half
// of every stage's K-blocks and add their accumulators through LDS at the
// end of the tile.
// The scale step is fp32 VALU work and a single wave issues independent
// fp32 FMAs at only about half the SIMD's rate, so two waves per SIMD split
// it; every operand and scale is still read from LDS once. A stage holds 8
// K-blocks of W and X in LDS, unpacked to int8 rows of 32 bytes plus fp32
// scales, so every MFMA operand is one 16-byte LDS read.
//
// Pipeline: a workgroup has eight compute waves and eight loader waves.
// Loader waves hold kDepth stages of raw blocks
// in registers (stage s+1+kDepth is requested while stage s is computed),
// unpack stage s+1 into the free half of a two-stage LDS buffer, and meet the
// compute waves at one barrier per stage. Compute waves keep only
// accumulators and operands.
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
#ifndef QMAT_GEMM_BM
#define QMAT_GEMM_BM 128
#define QMAT_GEMM_BN 64
#endif
constexpr int kBM = QMAT_GEMM_BM;  // tile rows (weights)
constexpr int kBN = QMAT_GEMM_BN;  // tile columns (tokens)
constexpr int kRT = kBM / 32, kCT = kBN / 32;  // 32 x 32 MFMA tiles per tile
constexpr int kKB = 8;  // K-blocks per stage
#ifndef QMAT_GEMM_NT
#define QMAT_GEMM_NT 2
#endif
// each compute wave owns 32 rows x (32 * kNT) columns of the tile
constexpr int kNT = QMAT_GEMM_NT;  // 32-column MFMA tiles per compute wave
constexpr int kTileWaves = kRT * kCT / kNT;  // wave tiles per workgroup tile
// Compute waves per wave tile (each takes kKB / ks_of(FMT) blocks of every
// stage).
constexpr int ks_of(int) { return 2; }
constexpr int threads_of(int fmt) { return kWave * kTileWaves * ks_of(fmt); }  // compute threads
// Loader waves: eight, two per SIMD, each with half the items of a stage
// (with four, their unpacking and LDS writes ran behind the compute waves and
// set the stage length), at four waves per SIMD and 128 registers.
constexpr int loaders_of(int) { return 8; }
constexpr int load_threads_of(int fmt) { return kWave * loaders_of(fmt); }
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

// Nibbles of 4 Q4_0 code bytes -> 4 signed bytes 16 (c - 8), given
// x = codes ^ 0x88888888: a nibble c ^ 8 in the top half of a byte is, read
// as a signed byte, 16 (c - 8). The high nibbles are x & 0xF0F0F0F0, the low
// ones (x << 4) & 0xF0F0F0F0: two or one operations per word after the
// shared XOR (the unscaled c - 8 takes four per nibble set).
__device__ __forceinline__ uint32_t nib16_hi(uint32_t x) { return x & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t nib16_lo(uint32_t x) { return (x << 4) & 0xF0F0F0F0u; }

__device__ __forceinline__ uint32_t nib_unsigned(uint32_t w, int shift) {
  return (w >> shift) & 0x0F0F0F0Fu;
}

__device__ __forceinline__ void store16(int8_t* dst, uint32_t a, uint32_t b, uint32_t c,
                                        uint32_t d) {
  u32x4 v = {a, b, c, d};
  *reinterpret_cast<u32x4*>(dst) = v;
}

// One loader item's fixed offsets from the stage base: an 18- or 34-byte
// block at byte offset o starts at 0 or 2 mod 4. If 0, the 16-byte load(s)
// at o hold the scale and the first code bytes and the 2-byte load at
// o + bytes - 2 the last two code bytes; if 2, the 2-byte load at o is the
// scale and the 16-byte load(s) at o + 2 hold the codes. sel realigns the
// code words with v_perm; hsel picks the scale's two bytes.
struct BlkLane {
  uint32_t o16, o2, sel, hsel;
};

__device__ __forceinline__ BlkLane blk_lane(uint32_t o, uint32_t par, int bytes) {
  const bool mis = ((o + par) & 2u) != 0;
  BlkLane l;
  l.o16 = o + (mis ? 2u : 0u);
  l.o2 = o + (mis ? 0u : (uint32_t)bytes - 2u);
  l.sel = mis ? 0x03020100u : 0x05040302u;
  l.hsel = mis ? 0x0c0c0504u : 0x0c0c0100u;  // s2's or the first word's low half
  return l;
}

__device__ __forceinline__ void load_lane(__amdgpu_buffer_rsrc_t rs, uint32_t soff,
                                          const BlkLane& l, int bytes, u32x4& va, u32x4& vb,
                                          uint32_t& s2) {
  va = __builtin_amdgcn_raw_buffer_load_b128(rs, l.o16, soff, 0);
  if (bytes == 34) vb = __builtin_amdgcn_raw_buffer_load_b128(rs, l.o16 + 16u, soff, 0);
  s2 = __builtin_amdgcn_raw_buffer_load_b16(rs, l.o2, soff, 0);
}

// Realign the code words of a block loaded by load_lane; h = fp16 scale bits.
__device__ __forceinline__ void realign_lane(const BlkLane& l, int bytes, const u32x4& va,
                                             const u32x4& vb, uint32_t s2, uint32_t& h,
                                             uint32_t (&c)[8]) {
  if (bytes == 18) {
    c[0] = perm_b32(va.y, va.x, l.sel);
    c[1] = perm_b32(va.z, va.y, l.sel);
    c[2] = perm_b32(va.w, va.z, l.sel);
    c[3] = perm_b32(s2, va.w, l.sel);
  } else {
    const uint32_t w[9] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w, s2};
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = perm_b32(w[i + 1], w[i], l.sel);
  }
  h = perm_b32(s2, va.x, l.hsel);
}

// The MFMA tile of one K-block: rows 32wm..32wm+31 against columns
// 32wn..32wn+31 of the stage; the accumulator input is the magic constant.
__device__ __forceinline__ void mfma_block(const Stage& cur, int bb, int wm, int wn, int l32,
                                           int half, const i32x16& cmagic, i32x16& d) {
  const i32x4 a = *reinterpret_cast<const i32x4*>(cur.w(bb, half, wm * 32 + l32));
  const i32x4 bv = *reinterpret_cast<const i32x4*>(cur.x(bb, half, wn * 32 + l32));
  d = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bv, cmagic, 0, 0, 0);
}

// MFMA operands of one K-block for a wave's NT tiles: its 32 weight rows
// and the NT x 32 token columns (16 bytes per lane each).
template <int NT>
struct Ops {
  i32x4 a;
  i32x4 b[NT];
};

template <int NT>
__device__ __forceinline__ void load_ops(const Stage& cur, int bb, int wm, int wn0, int l32,
                                         int half, Ops<NT>& op) {
  op.a = *reinterpret_cast<const i32x4*>(cur.w(bb, half, wm * 32 + l32));
#pragma unroll
  for (int t = 0; t < NT; ++t)
    op.b[t] = *reinterpret_cast<const i32x4*>(cur.x(bb, half, (wn0 + t) * 32 + l32));
}

// Per-block scales a lane needs: dw of its 16 rows and dx of its column in
// each of the NT tiles.
template <int NT>
struct Scales {
  float dw[16];
  float dx[NT];
};

template <int NT>
__device__ __forceinline__ void load_scales(const Stage& cur, int bb, int wm, int wn0, int l32,
                                            int half, Scales<NT>& sc) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(&cur.wd[bb][wm * 32 + 8 * q + 4 * half]);
    sc.dw[4 * q + 0] = t.x;
    sc.dw[4 * q + 1] = t.y;
    sc.dw[4 * q + 2] = t.z;
    sc.dw[4 * q + 3] = t.w;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) sc.dx[t] = cur.xd[bb][(wn0 + t) * 32 + l32];
}

// acc += dw * dx * S for the 16 values per lane (lane l holds column l % 32
// and rows 8q + 4(l / 32) + r of the tile). The MFMA accumulated S onto
// 1.5 * 2^23, so its result read as a float is 1.5 * 2^23 + S and
// S * dx = fma(F, dx, -1.5 * 2^23 * dx) exactly (dx is an fp16 value).
template <int NT>
__device__ __forceinline__ void apply_scales(const Scales<NT>& sc, const i32x16 (&d)[NT],
                                             float (&acc)[NT][16]) {
  // Two passes of independent instructions: first every S * dx (in place of
  // the MFMA results), then every accumulation, so that no instruction waits
  // on the one just before it.
  f32x16 df[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float c1 = -kMagicF * sc.dx[t];
    df[t] = __builtin_bit_cast(f32x16, d[t]);
#pragma unroll
    for (int i = 0; i < 16; ++i) df[t][i] = fmaf(df[t][i], sc.dx[t], c1);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = fmaf(df[t][i], sc.dw[i], acc[t][i]);
}

// Q4_K-style min term of blocks b0 and b0 + 1 (b0 + 1 < nbs, else only b0):
// acc -= O[m, b] * xs[n, b] summed over the two blocks, as one fp32 MFMA
// (32 x 32 x 2) whose output layout is that of the int8 MFMA. Lane l gives
// A[row l % 32][block l / 32] = -O and B[block l / 32][column l % 32] = xs.
// kGuard = false where both blocks are known to exist: the guarded reads
// become branches whose registers made the split kernel spill.
template <int NT, bool kGuard = true>
__device__ __forceinline__ void min_term(const Stage& cur, int b0, int nbs, int wm, int wn0,
                                         int l32, int half, float (&acc)[NT][16]) {
  const int b = b0 + half;
  const bool ok = !kGuard || b < nbs;
  const float a = ok ? cur.wo[b][wm * 32 + l32] : 0.0f;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float x = ok ? cur.xs[b][(wn0 + t) * 32 + l32] : 0.0f;
    f32x16 c;
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = acc[t][i];
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a, x, c, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = c[i];
  }
}

// Loader side of a tile: kLT threads move the 128 x 8 W items and 64 x 8
// X items (row, block) of each stage from memory into registers and then,
// unpacked, into an LDS stage. 8 consecutive threads cover one row's 8
// blocks of a stage. A stage is the same 8 blocks of every row, so an item
// keeps its byte offsets from the stage's (wave-uniform) base, and its
// alignment case, for the whole tile. Rows past M (N) re-read the last row.
template <int FMT, int kLT>
struct TileLoader {
  static constexpr int kWItems = kBM * kKB / kLT;
  static constexpr int kXItems = kBN * kKB / kLT;
  static constexpr bool kQ6K = FMT == kFmtQ6_K;
  static constexpr int wbytes = FMT == kFmtQ4_0 ? 18 : FMT == kFmtQ8_0 ? 34 : FMT == kFmtQ4_K ? 144 : 210;
  // a stage is 8 blocks: one superblock for Q4_K/Q6_K
  static constexpr int stage_wbytes = FMT == kFmtQ4_K || kQ6K ? wbytes : kKB * wbytes;
  struct Regs {
    u32x4 wa[kWItems], wb[kWItems];  // Q8_0: 2 x 16 B; Q4_0: 16 B; Q4_K: header, codes;
                                     // Q6_K: 16 B and (in wb.x, wb.y) 8 B of the group
    uint32_t ws[kWItems];            // 2-byte piece (Q4_0/Q8_0/Q6_K)
    uint32_t wdd[kWItems];           // Q6_K: the superblock's fp16 d
    u32x4 xa[kXItems], xb[kXItems];
    uint32_t xs[kXItems];
  };
  BlkLane wl[kWItems], xl[kXItems];
  int tid, nb;
  // Q6_K group of an item: its 26 bytes start at wl.o16 (relative to the
  // stage base) and are 2 mod 4 in even stages when wl.sel is 1; a stage is
  // 210 bytes, so odd stages flip that
  __device__ __forceinline__ static bool q6_mis(const BlkLane& l, int s) {
    return (l.sel ^ (uint32_t)(s & 1)) != 0;
  }

  __device__ __forceinline__ void setup(int64_t M, int64_t N, int64_t m0, int64_t n0,
                                        int64_t wrb, int64_t xrb, int tid_, int nb_) {
    tid = tid_;
    nb = nb_;
    const uint32_t wlast = (uint32_t)min<int64_t>(kBM - 1, M - 1 - m0);
    const uint32_t xlast = (uint32_t)min<int64_t>(kBN - 1, N - 1 - n0);
    // tile bases mod 4 (the buffers are 16-byte aligned, stage strides are
    // multiples of 4)
    const uint32_t wpar = (uint32_t)(m0 * wrb) & 3u, xpar = (uint32_t)(n0 * xrb) & 3u;
#pragma unroll
    for (int it = 0; it < kWItems; ++it) {
      const int item = tid + it * kLT;
      const uint32_t ro = min((uint32_t)(item >> 3), wlast) * (uint32_t)wrb;
      if (FMT == kFmtQ4_K) {
        wl[it].o16 = ro;                                    // superblock header
        wl[it].o2 = ro + 16u + 16u * (uint32_t)(item & 7);  // sub-block codes
        wl[it].sel = 0u;
        wl[it].hsel = 0u;
      } else if (kQ6K) {
        wl[it].o16 = ro + 2u + 26u * (uint32_t)(item & 7);  // the group's bytes
        wl[it].o2 = ro;                                     // d
        wl[it].sel = ((wl[it].o16 + wpar) & 2u) != 0 ? 1u : 0u;
        wl[it].hsel = 0u;
      } else {
        wl[it] = blk_lane(ro + (uint32_t)(item & 7) * (uint32_t)wbytes, wpar, wbytes);
      }
    }
#pragma unroll
    for (int it = 0; it < kXItems; ++it) {
      const int item = tid + it * kLT;
      const uint32_t ro = min((uint32_t)(item >> 3), xlast) * (uint32_t)xrb;
      xl[it] = blk_lane(ro + (uint32_t)(item & 7) * 34u, xpar, 34);
    }
  }

  // global -> registers for stage s (blocks past nb are not loaded); wrs and
  // xrs cover the W and X bytes from the tile's first rows to the end
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t wrs, __amdgpu_buffer_rsrc_t xrs,
                                       int s, Regs& r) const {
    const uint32_t wso = (uint32_t)s * (uint32_t)stage_wbytes;
    const uint32_t xso = (uint32_t)s * (uint32_t)(kKB * 34);
    const int left = nb - s * kKB;  // blocks of this stage that exist
#pragma unroll
    for (int it = 0; it < kWItems; ++it) {
      if (((tid + it * kLT) & 7) < left) {
        if (FMT == kFmtQ4_K) {
          r.wa[it] = __builtin_amdgcn_raw_buffer_load_b128(wrs, wl[it].o16, wso, 0);
          r.wb[it] = __builtin_amdgcn_raw_buffer_load_b128(wrs, wl[it].o2, wso, 0);
        } else if (kQ6K) {
          // group bytes [G, G + 26): aligned: 16 at G, 8 at G + 16, 2 at
          // G + 24; else 2 at G, 16 at G + 2, 8 at G + 18
          const uint32_t G = wl[it].o16;
          const bool mis = q6_mis(wl[it], s);
          r.wa[it] = __builtin_amdgcn_raw_buffer_load_b128(wrs, mis ? G + 2u : G, wso, 0);
          const uint2 u = __builtin_bit_cast(
              uint2, __builtin_amdgcn_raw_buffer_load_b64(wrs, mis ? G + 18u : G + 16u, wso, 0));
          r.wb[it].x = u.x;
          r.wb[it].y = u.y;
          r.ws[it] = __builtin_amdgcn_raw_buffer_load_b16(wrs, mis ? G : G + 24u, wso, 0);
          r.wdd[it] = __builtin_amdgcn_raw_buffer_load_b16(wrs, wl[it].o2, wso, 0);
        } else {
          load_lane(wrs, wso, wl[it], wbytes, r.wa[it], r.wb[it], r.ws[it]);
        }
      }
    }
#pragma unroll
    for (int it = 0; it < kXItems; ++it)
      if (((tid + it * kLT) & 7) < left) load_lane(xrs, xso, xl[it], 34, r.xa[it], r.xb[it], r.xs[it]);
  }

  // registers -> LDS buffer for stage s
  __device__ __forceinline__ void write(int s, const Regs& r, Stage& dst) const {
    const int left = nb - s * kKB;
#pragma unroll
    for (int it = 0; it < kWItems; ++it) {
      const int item = tid + it * kLT;
      const int rr = item >> 3, bb = item & 7;
      if (bb < left) {
        if (FMT == kFmtQ4_0) {
          uint32_t h, c[8];
          realign_lane(wl[it], 18, r.wa[it], r.wb[it], r.ws[it], h, c);
#pragma unroll
          for (int k = 0; k < 4; ++k) c[k] ^= 0x88888888u;
          store16(dst.w(bb, 0, rr), nib16_lo(c[0]), nib16_lo(c[1]), nib16_lo(c[2]), nib16_lo(c[3]));
          store16(dst.w(bb, 1, rr), nib16_hi(c[0]), nib16_hi(c[1]), nib16_hi(c[2]), nib16_hi(c[3]));
          dst.wd[bb][rr] = f16_bits_to_f32(h) * 0.0625f;  // the codes carry a factor 16
        } else if (FMT == kFmtQ8_0) {
          uint32_t h, c[8];
          realign_lane(wl[it], 34, r.wa[it], r.wb[it], r.ws[it], h, c);
          store16(dst.w(bb, 0, rr), c[0], c[1], c[2], c[3]);
          store16(dst.w(bb, 1, rr), c[4], c[5], c[6], c[7]);
          dst.wd[bb][rr] = f16_bits_to_f32(h);
        } else if (kQ6K) {
          // realign the group: 16 nibble bytes N, then H0, H1; codes
          // c = lo | hi << 4 become c - 32 per byte (c + 96 has no carry
          // out of its byte; flipping bit 7 gives c - 32 mod 256)
          const bool mis = q6_mis(wl[it], s);
          const uint32_t sel = mis ? 0x03020100u : 0x05040302u;
          const uint32_t x[7] = {r.wa[it].x, r.wa[it].y, r.wa[it].z, r.wa[it].w,
                                 r.wb[it].x, r.wb[it].y, r.ws[it]};
          const uint32_t H0 = perm_b32(x[5], x[4], sel), H1 = perm_b32(x[6], x[5], sel);
          uint32_t qa[4], qb[4];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t N = perm_b32(x[w + 1], x[w], sel);
            const uint32_t ca = (N & 0x0F0F0F0Fu) | (((H0 >> (2 * w)) & 0x03030303u) << 4);
            const uint32_t cb = ((N >> 4) & 0x0F0F0F0Fu) | (((H1 >> (2 * w)) & 0x03030303u) << 4);
            qa[w] = (ca + 0x60606060u) ^ 0x80808080u;
            qb[w] = (cb + 0x60606060u) ^ 0x80808080u;
          }
          store16(dst.w(bb, 0, rr), qa[0], qa[1], qa[2], qa[3]);
          store16(dst.w(bb, 1, rr), qb[0], qb[1], qb[2], qb[3]);
          const uint32_t scw = mis ? r.ws[it] : r.wa[it].x;
          const float D = f16_bits_to_f32(r.wdd[it]);
          dst.wd[bb][rr] = D * (float)(int8_t)(scw & 0xFFu);          // elements 0..15
          dst.wo[bb][rr] = D * (float)(int8_t)((scw >> 8) & 0xFFu);   // elements 16..31
        } else {
          const u32x4 hd = r.wa[it], cv = r.wb[it];
          const int sub = bb;  // a stage is one superblock
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
          dst.wo[bb][rr] = -(f16_bits_to_f32(hd.x >> 16) * (float)mn);  // -O
        }
      }
    }
#pragma unroll
    for (int it = 0; it < kXItems; ++it) {
      const int item = tid + it * kLT;
      const int cc = item >> 3, bb = item & 7;
      if (bb < left) {
        uint32_t h, c[8];
        realign_lane(xl[it], 34, r.xa[it], r.xb[it], r.xs[it], h, c);
        store16(dst.x(bb, 0, cc), c[0], c[1], c[2], c[3]);
        store16(dst.x(bb, 1, cc), c[4], c[5], c[6], c[7]);
        const float dx = f16_bits_to_f32(h);
        dst.xd[bb][cc] = dx;
        if (FMT == kFmtQ4_K) {
          int qs = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) qs = __builtin_amdgcn_sdot4((int)c[i], 0x01010101, qs, false);
          dst.xs[bb][cc] = dx * (float)qs;
        }
      }
    }
  }
};

// Blocks [b0, b1) of a K-stage for a wave's NT 32 x 32 tiles (rows 32 wm..,
// column tiles wn0..), from LDS into the fp32 accumulators.
// Q6_K-style stage: per block, the MFMA of each 16-element half (lanes of
// the other half give zero weight operands: the products pair operand bytes
// of the same lane half, which hold the same elements on both sides), each
// scaled by its own row scale.
template <int NT>
__device__ __forceinline__ void compute_range_q6(const Stage& cur, int b0, int b1, int wm,
                                                 int wn0, int l32, int half,
                                                 const i32x16& cmagic, float (&acc)[NT][16]) {
  for (int bb = b0; bb < b1; ++bb) {
    Ops<NT> op;
    load_ops(cur, bb, wm, wn0, l32, half, op);
    const i32x4 z = {0, 0, 0, 0};
    const i32x4 a0 = half == 0 ? op.a : z, a1 = half == 0 ? z : op.a;
    // one half at a time, so that a single set of MFMA results is live
    i32x16 d[NT];
    Scales<NT> sc;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      d[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, op.b[t], cmagic, 0, 0, 0);
    load_scales(cur, bb, wm, wn0, l32, half, sc);
    apply_scales(sc, d, acc);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      d[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, op.b[t], cmagic, 0, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(&cur.wo[bb][wm * 32 + 8 * q + 4 * half]);
      sc.dw[4 * q + 0] = t.x;
      sc.dw[4 * q + 1] = t.y;
      sc.dw[4 * q + 2] = t.z;
      sc.dw[4 * q + 3] = t.w;
    }
    apply_scales(sc, d, acc);
  }
}

template <int FMT, int NT, int PER>
__device__ __forceinline__ void compute_range(const Stage& cur, int b0, int b1, int wm,
                                              int wn0, int l32, int half, const i32x16& cmagic,
                                              float (&acc)[NT][16]) {
  if (FMT == kFmtQ6_K) {
    compute_range_q6<NT>(cur, b0, b1, wm, wn0, l32, half, cmagic, acc);
  } else if (b1 - b0 == PER) {
    // A full share, unrolled. The other compute wave of the SIMD covers
    // this wave's waits for the LDS and the matrix core (reading block j+1's
    // operands ahead of block j's scaling measured slower).
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      Ops<NT> op;
      Scales<NT> sc;
      load_ops(cur, b0 + j, wm, wn0, l32, half, op);
      i32x16 d[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t)
        d[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(op.a, op.b[t], cmagic, 0, 0, 0);
      load_scales(cur, b0 + j, wm, wn0, l32, half, sc);
      apply_scales(sc, d, acc);
      if (FMT == kFmtQ4_K && (j & 1))
        min_term<NT, false>(cur, b0 + j - 1, b1, wm, wn0, l32, half, acc);
    }
  } else {
    for (int bb = b0; bb < b1; ++bb) {
      i32x16 d[NT];
      Scales<NT> sc;
#pragma unroll
      for (int t = 0; t < NT; ++t) mfma_block(cur, bb, wm, wn0 + t, l32, half, cmagic, d[t]);
      load_scales(cur, bb, wm, wn0, l32, half, sc);
      apply_scales(sc, d, acc);
      if (FMT == kFmtQ4_K && (((bb - b0) & 1) || bb + 1 == b1))
        min_term(cur, bb - ((bb - b0) & 1), b1, wm, wn0, l32, half, acc);
    }
  }
}

// Store: lane holds column n = n0 + 32(wn0 + t) + l32, rows
// m = m0 + 32 wm + 8q + 4 half + r (q, r in 0..3).
template <int NT>
__device__ __forceinline__ void store_tile(float* __restrict__ Y, int64_t M, int64_t N,
                                           int64_t m0, int64_t n0, int wm, int wn0, int l32,
                                           int half, const float (&acc)[NT][16]) {
#pragma unroll
  for (int t = 0; t < NT; ++t) {
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

// XCD-aware order: XCD x = id % 8 takes linear tiles [x * per, (x+1) * per)
__device__ __forceinline__ int64_t first_tile(int64_t ntiles) {
  int64_t lin = blockIdx.x;
  if ((ntiles & 7) == 0 && (int64_t)gridDim.x == ntiles) {
    const int64_t per = ntiles >> 3;
    lin = (int64_t)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
  }
  return lin;
}

__device__ __forceinline__ i32x16 magic_vec() {
  i32x16 c;
#pragma unroll
  for (int i = 0; i < 16; ++i) c[i] = (int)kMagicI;
  return c;
}

// K split. A product whose tiles cannot fill the GPU is also divided along
// K into nsplit ranges of whole stages (pairs of stages for Q6_K-style, so
// that a range starts at an even stage and keeps the stage parity its
// 210-byte alignment cases follow). Linear tile index = (split, m-tile,
// n-tile); each range's partial product is written whole (range 0 into Y),
// and a second kernel adds the others into Y in range order.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint64_t u = (uint64_t)v;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

struct SplitTile {
  int64_t tm, tn;
  int split, stage0, nb, nstage;
};
template <int FMT>
__device__ __forceinline__ SplitTile split_tile(int64_t tile, int64_t tiles_n, int64_t tps,
                                                int nsplit, int nbk) {
  // every value is wave-uniform: readfirstlane keeps them in scalar
  // registers (the divisions themselves are expanded into vector code)
  SplitTile t;
  // (a split product has at most 2^24 tiles in all)
  t.split = nsplit > 1 ? __builtin_amdgcn_readfirstlane((int)((uint32_t)tile / (uint32_t)tps)) : 0;
  const int64_t r = tile - (int64_t)t.split * tps;
  t.tm = uniform64(r / tiles_n);
  t.tn = r - t.tm * tiles_n;
  constexpr int kUnit = FMT == kFmtQ6_K ? 2 : 1;  // stages per unit of a range
  const int nst = (nbk + kKB - 1) / kKB;
  const int units = (nst + kUnit - 1) / kUnit;  // < 2^16: K <= 2^24
  const int u0 = t.split * units / nsplit;
  const int u1 = (t.split + 1) * units / nsplit;
  t.stage0 = __builtin_amdgcn_readfirstlane(u0 * kUnit);
  const int b0 = t.stage0 * kKB, b1 = min(nbk, u1 * kUnit * kKB);
  t.nb = __builtin_amdgcn_readfirstlane(b1 - b0);
  t.nstage = (t.nb + kKB - 1) / kKB;
  return t;
}

// Warp-specialized kernel: load_threads_of(FMT) loader threads fill the LDS stages,
// threads_of(FMT) compute threads share 32 x (32 kNT) wave tiles ks_of(FMT)
// to a tile.
template <int FMT>
__global__ __launch_bounds__(threads_of(FMT) + load_threads_of(FMT)) void gemm_kernel(
    const uint8_t* __restrict__ Wb, const uint8_t* __restrict__ Xb, float* __restrict__ Y,
    float* __restrict__ part, int64_t M, int K, int64_t N, int64_t tiles_n, int64_t tps,
    int nsplit) {
  __shared__ __attribute__((aligned(16))) Stage st[2];
  typedef TileLoader<FMT, load_threads_of(FMT)> TL;
  constexpr int kKS = ks_of(FMT), kPer = kKB / kKS, kThreads = threads_of(FMT);
  static_assert((kKS - 1) * kTileWaves * kNT * 16 * kWave * 4 <= 2 * (int)sizeof(Stage),
                "reduction buffer exceeds the LDS stages");
  static_assert(kKB % kKS == 0 && (kPer % 2 == 0 || kKS == 1), "K split must keep block pairs");
  // role per wave, in a scalar register so that the branch is uniform
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const bool loader = wave >= kThreads / kWave;
  const int tid = (int)threadIdx.x - (loader ? kThreads : 0);  // index within its group
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int nbk = K >> 5;  // 32-element blocks along K
  const int64_t wrb = FMT == kFmtQ4_K || FMT == kFmtQ6_K ? (int64_t)(K >> 8) * TL::wbytes
                                                          : (int64_t)nbk * TL::wbytes;
  const int64_t xrb = (int64_t)nbk * 34;
  const int64_t ntiles = tps * nsplit;
  const int64_t lin = first_tile(ntiles);

  // Each role runs its own tile loop (so that neither keeps the other's
  // tile-invariant values live); both pass the same barriers per tile: one
  // before the first stage, one per stage and one after the last.
  if (loader) {
    for (int64_t tile = lin; tile < ntiles; tile += gridDim.x) {
      const SplitTile t = split_tile<FMT>(tile, tiles_n, tps, nsplit, nbk);
      const int64_t m0 = t.tm * kBM, n0 = t.tn * kBN;
      const int nb = t.nb, nstage = t.nstage;
      TL ld;
      ld.setup(M, N, m0, n0, wrb, xrb, tid, nb);
      const int64_t wo = (int64_t)t.stage0 * TL::stage_wbytes, xo = (int64_t)t.stage0 * (kKB * 34);
      const __amdgpu_buffer_rsrc_t wrs = make_rsrc(Wb + m0 * wrb + wo, (M - m0) * wrb - wo);
      const __amdgpu_buffer_rsrc_t xrs = make_rsrc(Xb + n0 * xrb + xo, (N - n0) * xrb - xo);
      // Register set k holds stages k, k + kDepth, ...: set indices stay
      // compile-time constants by stepping kDepth stages per iteration.
      typename TL::Regs regs[kDepth];
#pragma unroll
      for (int k = 0; k < kDepth; ++k)
        if (k < nstage) ld.load(wrs, xrs, k, regs[k]);
      if (nstage > 0) {
        ld.write(0, regs[0], st[0]);
        if (kDepth < nstage) ld.load(wrs, xrs, kDepth, regs[0]);
      }
      __syncthreads();
      // step s: write stage s+1 (set (s+1) % kDepth), refill it with stage
      // s+1+kDepth
      auto step = [&](int s, typename TL::Regs& r) {
        if (s + 1 < nstage) {
          ld.write(s + 1, r, st[(s + 1) & 1]);
          if (s + 1 + kDepth < nstage) ld.load(wrs, xrs, s + 1 + kDepth, r);
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
      if (kKS > 1) __syncthreads();  // the compute waves' reduction
      // the next tile reuses both LDS stages
      __syncthreads();
    }
  } else {
    const i32x16 cmagic = magic_vec();
    // waves tw and tw + kTileWaves share a SIMD and wave tile tw: rows
    // 32 wm.., column tiles wn0..; share ks takes blocks [ks kPer, (ks+1) kPer)
    // of every stage
    const int ks = wv / kTileWaves, tw = wv % kTileWaves;
    const int wm = tw % kRT, wn0 = (tw / kRT) * kNT;
    for (int64_t tile = lin; tile < ntiles; tile += gridDim.x) {
      const SplitTile t = split_tile<FMT>(tile, tiles_n, tps, nsplit, nbk);
      const int64_t m0 = t.tm * kBM, n0 = t.tn * kBN;
      const int nb = t.nb, nstage = t.nstage;
      // the first K range writes Y, range s > 0 its own partial product
      float* __restrict__ out = t.split == 0 ? Y : part + (int64_t)(t.split - 1) * N * M;
      float acc[kNT][16];
#pragma unroll
      for (int t = 0; t < kNT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][i] = 0.0f;
      __syncthreads();  // stage 0 is in LDS
      for (int s = 0; s < nstage; ++s) {
        const int nbs = min(kKB, nb - s * kKB);
        compute_range<FMT, kNT, kPer>(st[s & 1], min(nbs, ks * kPer), min(nbs, (ks + 1) * kPer), wm,
                                wn0, l32, half, cmagic, acc);
        __syncthreads();
      }
      if (kKS > 1) {
        // both LDS stages are free until the end-of-tile barrier: the other
        // shares park their sums there, and share 0 adds them in share order
        float* red = reinterpret_cast<float*>(&st[0]);
        // an opaque copy of the base, so that the 32 addresses below are
        // formed here and not hoisted out of the tile loop into registers
        int rbase = ((ks > 0 ? ks - 1 : 0) * kTileWaves + tw) * kNT * 16 * kWave + lane;
        asm volatile("" : "+v"(rbase));
        constexpr int kVals = kNT * 16;
        if (ks > 0) {
          float* p = red + rbase;
#pragma unroll
          for (int t = 0; t < kNT; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) p[(t * 16 + i) * kWave] = acc[t][i];
        }
        __syncthreads();
        if (ks == 0) {
#pragma unroll
          for (int k = 1; k < kKS; ++k) {
            const float* p = red + rbase + (k - 1) * kTileWaves * kVals * kWave;
#pragma unroll
            for (int t = 0; t < kNT; ++t)
#pragma unroll
              for (int i = 0; i < 16; ++i) acc[t][i] += p[(t * 16 + i) * kWave];
          }
          store_tile<kNT>(out, M, N, m0, n0, wm, wn0, l32, half, acc);
        }
      } else {
        store_tile<kNT>(out, M, N, m0, n0, wm, wn0, l32, half, acc);
      }
      __syncthreads();
    }
  }
}

constexpr int64_t kMaxGrid = 1 << 24;
static_assert(kBM == split::kTileM && kBN == split::kTileN && kKB == split::kStageBlocks,
              "the K-split policy assumes this kernel's tile and stage sizes");
#ifndef QMAT_GEMM_SMALL_N
#define QMAT_GEMM_SMALL_N 48
#endif
constexpr int64_t kSmallN = QMAT_GEMM_SMALL_N;
#ifndef QMAT_GEMM_DECODE_MODEL
#define QMAT_GEMM_DECODE_MODEL 1
#endif
// Y += part[0] + part[1] + ... + part[kParts - 1] (partial products of
// count values each), added in that order for every element. All loads of
// an element are issued before the first add.
template <int kParts>
__global__ __launch_bounds__(256) void splitk_add_kernel(float* __restrict__ Y,
                                                         const float* __restrict__ part,
                                                         int64_t count) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if ((count & 3) == 0) {
    const int64_t n4 = count >> 2;
    f32x4* y4 = reinterpret_cast<f32x4*>(Y);
    const f32x4* p4 = reinterpret_cast<const f32x4*>(part);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
      f32x4 a[kParts];
#pragma unroll
      for (int k = 0; k < kParts; ++k) a[k] = __builtin_nontemporal_load(p4 + k * n4 + i);
      f32x4 v = y4[i];
#pragma unroll
      for (int k = 0; k < kParts; ++k) {
        v[0] += a[k][0];
        v[1] += a[k][1];
        v[2] += a[k][2];
        v[3] += a[k][3];
      }
      y4[i] = v;
    }
  } else {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
      float a[kParts];
#pragma unroll
      for (int k = 0; k < kParts; ++k) a[k] = part[k * count + i];
      float v = Y[i];
#pragma unroll
      for (int k = 0; k < kParts; ++k) v += a[k];
      Y[i] = v;
    }
  }
}

template <int kParts>
hipError_t launch_add(float* Y, const float* part, int64_t count, int nparts, hipStream_t stream) {
  if constexpr (kParts > 1) {
    if (nparts < kParts) return launch_add<kParts - 1>(Y, part, count, nparts, stream);
  }
  const int64_t items = (count & 3) == 0 ? count >> 2 : count;
  int64_t nblk = (items + 255) / 256;
  nblk = nblk < 4096 ? nblk : 4096;
  hipLaunchKernelGGL(splitk_add_kernel<kParts>, dim3((unsigned)nblk), dim3(256), 0, stream, Y,
                     part, count);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int fmt, const void* blocks, const void* Xq8, float* Y, int64_t M,
                       int64_t K, int64_t N, float* part, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int nsplit = part != nullptr ? gemm_splits(fmt, M, K, N) : 1;
  // a few tokens and no K split: the weights are streamed once per 16
  // tokens instead (the MFMA tiles would leave most of the GPU idle)
  if (nsplit == 1 && (QMAT_GEMM_DECODE_MODEL ? gemm_uses_decode(fmt, M, K, N) : N <= kSmallN))
    return launch_gemm_small(fmt, blocks, Xq8, Y, M, K, N, stream);
  const int64_t tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
  const int64_t tps = tiles_m * tiles_n;
  const int64_t ntiles = tps * nsplit;
  const unsigned grid = (unsigned)(ntiles < kMaxGrid ? ntiles : kMaxGrid);
  const uint8_t* W = static_cast<const uint8_t*>(blocks);
  const uint8_t* X = static_cast<const uint8_t*>(Xq8);
#define QMAT_GEMM_LAUNCH(F)                                                                \
  hipLaunchKernelGGL(gemm_kernel<F>, dim3(grid), dim3(threads_of(F) + load_threads_of(F)), 0, stream, W, \
                     X, Y, part, M, (int)K, N, tiles_n, tps, nsplit)
  switch (fmt) {
    case kFmtQ4_0:
      QMAT_GEMM_LAUNCH(kFmtQ4_0);
      break;
    case kFmtQ8_0:
      QMAT_GEMM_LAUNCH(kFmtQ8_0);
      break;
    case kFmtQ4_K:
      QMAT_GEMM_LAUNCH(kFmtQ4_K);
      break;
    default:
      QMAT_GEMM_LAUNCH(kFmtQ6_K);
      break;
  }
#undef QMAT_GEMM_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  return launch_add<(int)split::kMaxSplit - 1>(Y, part, N * M, nsplit - 1, stream);
}

}  // namespace qmat
