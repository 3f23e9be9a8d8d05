// decode.hip — the decode batch on the int8 matrix cores: Y = W X^T for 5 to
// 16 tokens per launch, W in Q4_0, Q8_0, Q4_K-style or Q6_K-style blocks, X
// in Q8_0 blocks.
//
// Source: "05. llama.cpp：从 GGUF 文件到本地推理服务", sections "槽位、连续批处理与
// 上下文切分" (several requests decoded at once) and "性能直觉：带宽决定 Decode，
// 算力决定 Prefill" (decode is bound by reading the weights): a batch of tokens
// shares one read of W, so the weight stream stays the bound as long as the
// per-token arithmetic stays off the critical path.
//
// Work split. A workgroup owns 16 rows of W and all of K; its waves (16, 12
// or 8, as LDS allows; 4 with shallow rings when there are more workgroups
// than CUs, see DecRing) take contiguous shares of the rows' stages. A stage
// is 8 blocks of every row (144 or 272 bytes per row) and of every token
// (272 bytes): both are whole 16-byte pieces, so the copies go from memory
// straight into LDS (global_load_lds, 64 pieces per instruction). Each wave keeps its own ring
// of D stages and issues a stage's weight and token copies together, D - 1
// stages ahead; it waits for a stage by counting its outstanding copies
// (they complete in issue order), so the waves never synchronise until the
// final sum, and each stage is used as soon as it has landed.
//
// Arithmetic per block, exact in integers: one v_mfma_i32_16x16x32_i8 takes
// the 16 rows' 32 codes (A) and the 16 tokens' 32 codes (B). Lane l supplies
// row/token l % 16 and the elements 4q..4q+3 and 16+4q..16+4q+3 (q = l / 16)
// of the block: for Q4_0 these are the two nibbles of code bytes 4q..4q+3,
// read as one dword and turned into 16 (c - 8) with an XOR and two masks;
// for Q8_0 (and X) two dwords of codes, realigned when the block starts at
// 0 mod 4 (codes at 2 mod 4); for Q4_K-style the unsigned nibbles of the
// sub-block's code bytes 4q..4q+3, whose offset term (the sub-block's min
// times the token's block sum) takes a second MFMA with all-ones weights;
// for Q6_K-style the 6-bit codes c - 32 of the same elements, rebuilt from
// the low nibbles and the high-bit words, one MFMA per 16-element half
// (each half has its own scale; the other half's operand bytes are zero).
// A Q6_K-style superblock (210 bytes) is not 16-byte aligned in memory: a
// row's stage is the 14 aligned pieces that cover it, and the lanes read
// their words at the superblock's offset inside them. The MFMA accumulates onto 1.5 * 2^23, so each
// integer sum C comes out as the float 1.5 * 2^23 + C (|C| < 2^22) and
// fma(F, dx, -1.5 * 2^23 * dx) is C * dx rounded once (1.5 dx is exact for
// an fp16 dx); a second fma adds C * dx * dw to the lane's fp32 sums of rows
// 4q..4q+3 for token l % 16. Lane 16q + r reads the scale of row 4q + (r & 3),
// and a DPP row broadcast hands each lane the scales of its four rows.
// A wave reads every LDS word of a stage's 8 blocks before it uses any, so
// the reads overlap each other and the previous blocks' arithmetic.
// The waves' sums meet in LDS and are added in wave order (deterministic).
//
// What bounds it: the copies. Every workgroup copies all of X next to its
// 16 rows of W (at 16 tokens 187 KB of X per 99 KB of Q4_0 weights at
// K = 11008), and the copies alone take about as long as the whole kernel
// minus the arithmetic of its last stages.
#include "qmat_device.hpp"
#include "qmat_launch.hpp"

namespace qmat {
namespace {

constexpr uint32_t kDecMagicI = 0x4B400000u;  // 1.5 * 2^23 as fp32 bits
constexpr float kDecMagicF = 12582912.0f;
constexpr int kDecRows = 16;   // rows of W per workgroup: the MFMA's A rows
constexpr int kGroup = 8;      // blocks per stage
constexpr int kXRowBytes = kGroup * 34;

// Weight formats: Q4_0, Q8_0, Q4_K-style (a stage is one 144-byte
// superblock per row) or Q6_K-style (one 210-byte superblock per row, held
// in LDS as the 224 bytes of 16-byte pieces that cover it).
template <int kFmt>
struct DecW {
  static constexpr bool kQ6 = kFmt == kFmtQ6_K;
  static constexpr int kBytes = kFmt == kFmtQ8_0 ? 34 : 18;  // per block (Q4_K: on average)
  static constexpr int kGlobalRowBytes = kQ6 ? 210 : kGroup * kBytes;  // a row's stage in memory
  static constexpr int kRowBytes = kQ6 ? 224 : kGroup * kBytes;  // its LDS slot
  static constexpr int kPiecesPerRow = kRowBytes / 16;
  static constexpr int kPieces = kDecRows * kPiecesPerRow;
  static constexpr int kLoads = (kPieces + kWave - 1) / kWave;
  static constexpr int kStage = kDecRows * kRowBytes;
  static_assert(kRowBytes % 16 == 0, "whole pieces");
};

template <int NT>
struct DecX {
  static constexpr int kPiecesPerRow = kXRowBytes / 16;
  static constexpr int kPieces = NT * kPiecesPerRow;
  static constexpr int kLoads = (kPieces + kWave - 1) / kWave;
  static constexpr int kStage = NT * kXRowBytes;
};

// Per wave: a ring of kDepth stages (weights and tokens). Up to one
// workgroup per CU (at most 256 workgroups): as many waves as 160 KB of LDS
// allows with a ring of at least two stages (16, 12 or 8: the waves hide
// each other's LDS and matrix-core latency), each with the deepest ring
// that then fits. Taller matrices (kDecTall: more 16-row workgroups than CUs)
// take 4 waves with rings of 2 stages instead, 27-70 KB per workgroup, so
// that two or more workgroups share a CU and hide each other's copy
// latency; measured at 16 tokens, 11008 x 4096: Q4_0 17.7 -> 13.4 us, Q8_0
// 21.1 -> 16.6, Q4_K-style 19.4 -> 15.2, Q6_K-style 28.0 -> 23.9 (also
// 14336 and 28672 x 4096, 11008 x 2048, 8192 x 8192); with 4096 rows the
// one-workgroup shape stays ahead (Q4_0 4096 x 11008: 12.9 against 14.8).
// kDecLong: rows of at least 24 stages (K >= 6144) take 8 waves with 2-stage
// rings (3 or more stages per wave) where the one-round shape would run
// 12 or 16: 16 tokens at 4096 x 11008 Q4_0 13.3 -> 12.6 us, Q4_K-style
// 15.4 -> 14.6 (4096 x 6144 to 4096 x 14336 and 3072 x 11008 alike); 5-8
// tokens of Q4_0, 4096 x 14336: 14.3 -> 12.9; Q8_0 and Q6_K-style at 16
// tokens run 8 waves either way. At K = 4096 the 12 waves stay ahead (Q4_0
// 6.3 against 6.6 us).
enum DecShape { kDecOne = 0, kDecTall = 1, kDecLong = 2 };
template <int kFmt, int NT, int kShape>
struct DecRing {
  static constexpr bool kTall = kShape == kDecTall;
  static constexpr int kStage = DecW<kFmt>::kStage + DecX<NT>::kStage;
  static constexpr int depth_for(int waves) { return 163840 / waves / kStage; }
  static constexpr int kWaves = kTall ? 4
                                : kShape == kDecLong ? 8
                                : depth_for(16) >= 2 ? 16
                                : depth_for(12) >= 2 ? 12
                                                     : 8;
  static constexpr int kDepth0 = depth_for(kWaves);
  static constexpr int kDepth = kTall || kShape == kDecLong ? 2 : kDepth0 > 6 ? 6 : kDepth0;
  static constexpr int kLoads = DecW<kFmt>::kLoads + DecX<NT>::kLoads;
  static constexpr int kWaveLds = kDepth * kStage;
  static_assert(kDepth >= 2 && (kDepth - 1) * kLoads < 64, "ring");
  static_assert(kWaves * 4 * kWave * 4 <= kWaves * kWaveLds, "final sums fit");
};

// Wait until at most N copies are outstanding. The copies land in LDS behind
// the compiler's back, so no LDS access may move across the wait.
template <int N>
__device__ __forceinline__ void wait_copies() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm<N>());
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// Wait until at most n * kPer copies are outstanding, 0 <= n < kMax (n is
// wave-uniform; the immediate must be a constant).
template <int kPer, int kMax>
__device__ __forceinline__ void wait_stages(int n) {
  if constexpr (kMax > 1) {
    if (n >= kMax - 1) {
      wait_copies<(kMax - 1) * kPer>();
      return;
    }
    wait_stages<kPer, kMax - 1>(n);
  } else {
    wait_copies<0>();
  }
}

// The LDS words a lane needs from one block: codes of elements 4q..4q+3
// and 16+4q..16+4q+3 of its weight row and of its token, and the fp16 scales
// of its token and of the row it broadcasts. A block at 0 mod 4 has its
// codes at 2 mod 4, so each 4-byte run spans two words (w[0..1], w[2..3]);
// a block at 2 mod 4 has them aligned (w[0], w[1]). Q4_0 codes hold both
// element runs in the nibbles of one 4-byte run.
struct BlockWords {
  uint32_t w[4], x[4];
  uint32_t dxb, swb;
};

// The token's words (Q8_0, as for a Q8_0 weight block).
__device__ __forceinline__ void fetch_x(const uint8_t* xb, bool odd, int q, BlockWords& o) {
  if (!odd) {
    const uint32_t* px = reinterpret_cast<const uint32_t*>(xb + 4 * q);
    o.x[0] = px[0];
    o.x[1] = px[1];
    o.x[2] = px[4];
    o.x[3] = px[5];
  } else {
    const uint32_t* px = reinterpret_cast<const uint32_t*>(xb + 2 + 4 * q);
    o.x[0] = px[0];
    o.x[1] = px[4];
  }
  o.dxb = *reinterpret_cast<const uint16_t*>(xb);
}

// The weight row's words: Q4_0 / Q8_0 block wb (at 0 mod 4 when !odd);
// Q4_K-style: wb is the sub-block's 16 code bytes, always aligned.
template <int kFmt>
__device__ __forceinline__ void fetch_w(const uint8_t* wb, bool odd, int q, BlockWords& o) {
  if (kFmt == kFmtQ4_K) {
    o.w[0] = reinterpret_cast<const uint32_t*>(wb + 4 * q)[0];
  } else if (!odd) {
    const uint32_t* pw = reinterpret_cast<const uint32_t*>(wb + 4 * q);
    o.w[0] = pw[0];
    o.w[1] = pw[1];
    if (kFmt == kFmtQ8_0) {
      o.w[2] = pw[4];
      o.w[3] = pw[5];
    }
  } else {
    const uint32_t* pw = reinterpret_cast<const uint32_t*>(wb + 2 + 4 * q);
    o.w[0] = pw[0];
    if (kFmt == kFmtQ8_0) o.w[1] = pw[4];
  }
}

// Q8_0 codes of the lane's 8 elements as the MFMA operand (low dword:
// elements 4q..4q+3, high dword: 16+4q..16+4q+3).
__device__ __forceinline__ uint64_t q8_operand(const uint32_t (&w)[4], bool odd) {
  const uint32_t lo = odd ? w[0] : __builtin_amdgcn_alignbyte(w[1], w[0], 2);
  const uint32_t hi = odd ? w[1] : __builtin_amdgcn_alignbyte(w[3], w[2], 2);
  return (uint64_t)hi << 32 | lo;
}

// The same elements of a Q4_0 block as 16 (c - 8): code byte t holds element
// t in its low nibble and element t + 16 in its high nibble, and c ^ 8 read
// as the top nibble of a byte is 16 (c - 8).
__device__ __forceinline__ uint64_t q4_operand(const uint32_t (&w)[4], bool odd) {
  const uint32_t c = odd ? w[0] : __builtin_amdgcn_alignbyte(w[1], w[0], 2);
  const uint32_t v = c ^ 0x88888888u;
  const uint32_t lo = (v << 4) & 0xF0F0F0F0u;
  const uint32_t hi = v & 0xF0F0F0F0u;
  return (uint64_t)hi << 32 | lo;
}

// The same elements of a Q4_K-style sub-block as unsigned codes 0..15 (byte
// t of its 16 code bytes: element t low, element t + 16 high).
__device__ __forceinline__ uint64_t q4k_operand(uint32_t c) {
  const uint32_t lo = c & 0x0F0F0F0Fu;
  const uint32_t hi = (c >> 4) & 0x0F0F0F0Fu;
  return (uint64_t)hi << 32 | lo;
}

// 6-bit field f of a Q4_K-style superblock's 96-bit scale word (header
// words 1..3): bits 6f .. 6f + 5.
__device__ __forceinline__ uint32_t field6(uint32_t w1, uint32_t w2, uint32_t w3, int f) {
  const int p = 6 * f;
  const uint32_t lo = p < 32 ? w1 : p < 64 ? w2 : w3;
  const uint32_t hi = p < 32 ? w2 : p < 64 ? w3 : 0u;
  return __builtin_amdgcn_alignbit(hi, lo, (uint32_t)(p & 31)) & 63u;
}

// The value of s held by lane v of this lane's 16-lane row (DPP
// row_newbcast:v).
template <int v>
__device__ __forceinline__ float row_bcast(float s) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s),
                                                               0x150 + v, 0xF, 0xF, false));
}

template <int kFmt, int NT, int kShape>
__global__ __launch_bounds__((DecRing<kFmt, NT, kShape>::kWaves * kWave)) void decode_mfma_kernel(
    const uint8_t* __restrict__ Wb, const uint8_t* __restrict__ Xq, float* __restrict__ Y,
    int64_t M, int K, int64_t N, int64_t n0) {
  constexpr bool kQ4 = kFmt == kFmtQ4_0, kQ4K = kFmt == kFmtQ4_K;
  using WS = DecW<kFmt>;
  using XS = DecX<NT>;
  using RG = DecRing<kFmt, NT, kShape>;
  constexpr int kWaves = RG::kWaves;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kWaves * RG::kWaveLds];
  const int lane = (int)(threadIdx.x & 63);
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  uint8_t* ring = lds + wv * RG::kWaveLds;  // slot: weights, then tokens
  const int ns = K >> 5;
  const int ngroups = ns / kGroup;
  const int ga = (int)((int64_t)wv * ngroups / kWaves);
  const int gb = (int)((int64_t)(wv + 1) * ngroups / kWaves);
  const int64_t m0 = (int64_t)blockIdx.x * kDecRows;
  const int64_t rb = (int64_t)ngroups * WS::kGlobalRowBytes, xrb = (int64_t)ns * 34;

  // Copy sources: piece p = lane + 64 d of a stage is 16 bytes of row (or
  // token) p / pieces-per-row. Rows past M and tokens past N copy the last
  // valid one; their results are not stored.
  // (Q6_K-style: the row's start and the piece's offset inside the window
  // of aligned pieces that covers the stage's superblock)
  const uint8_t* wsrc[WS::kLoads];
  int64_t wrow[WS::kLoads];
  int wpiece[WS::kLoads];
#pragma unroll
  for (int d = 0; d < WS::kLoads; ++d) {
    const int p = lane + kWave * d;
    const int r = p / WS::kPiecesPerRow, u = p - r * WS::kPiecesPerRow;
    int64_t m = m0 + (r < kDecRows ? r : kDecRows - 1);
    if (m >= M) m = M - 1;
    wsrc[d] = Wb + m * rb + 16 * u;
    wrow[d] = m * rb;
    wpiece[d] = 16 * u;
  }
  const uint8_t* xsrc[XS::kLoads];
#pragma unroll
  for (int d = 0; d < XS::kLoads; ++d) {
    const int p = lane + kWave * d;
    const int t = p / XS::kPiecesPerRow, u = p - t * XS::kPiecesPerRow;
    int64_t n = n0 + (t < NT ? t : NT - 1);
    if (n >= N) n = N - 1;
    xsrc[d] = Xq + n * xrb + 16 * u;
  }
  // Stage g goes to ring slot g mod depth, its weight copies first. Lane 0
  // of every copy instruction is inside the stage, so each instruction is
  // issued and counted.
  auto issue = [&](int g) {
    uint8_t* dst = ring + (g % RG::kDepth) * RG::kStage;
    const int64_t woff = (int64_t)g * WS::kRowBytes, xoff = (int64_t)g * kXRowBytes;
#pragma unroll
    for (int d = 0; d < WS::kLoads; ++d)
      if (lane + kWave * d < WS::kPieces) {
        // Q6_K-style: the 14 pieces from the 16-byte boundary at or below
        // the superblock's start; the last one ends at most 14 bytes past
        // the superblock, inside the 16-byte granule of its last byte
        const uint8_t* src =
            WS::kQ6 ? Wb + ((wrow[d] + (int64_t)g * WS::kGlobalRowBytes) & ~(int64_t)15) + wpiece[d]
                    : wsrc[d] + woff;
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr_t)(dst + 1024 * d), 16, 0, 0);
      }
#pragma unroll
    for (int d = 0; d < XS::kLoads; ++d)
      if (lane + kWave * d < XS::kPieces)
        __builtin_amdgcn_global_load_lds((const void*)(xsrc[d] + xoff),
                                         (lds_ptr_t)(dst + WS::kStage + 1024 * d), 16, 0, 0);
  };

  const int i16 = lane & 15, q = lane >> 4;
  const int tj = i16 < NT ? i16 : NT - 1;  // the token this lane supplies to B
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};

  // Lane 16 q + r also reads the scale of row 4 q + (r & 3); a row broadcast
  // (DPP row_newbcast:v) then gives every lane of DPP row q the scale of row
  // 4 q + v, the row of its v-th sum.
  const int srow = 4 * q + (lane & 3);
  const i32x4 cmagic = {(int)kDecMagicI, (int)kDecMagicI, (int)kDecMagicI, (int)kDecMagicI};

  // Q6_K-style: where the rows of this lane's A operand and of its scales
  // start (mod 16, all a superblock's offset inside its window depends on)
  const uint32_t rowA16 = (uint32_t)(((m0 + i16 < M ? m0 + i16 : M - 1) * rb) & 15);
  const uint32_t rowS16 = (uint32_t)(((m0 + srow < M ? m0 + srow : M - 1) * rb) & 15);

  auto compute = [&](int g) {
    if constexpr (WS::kQ6) {
      // byte offsets into lds (kept as integers so that the accesses stay
      // LDS accesses): the lane's A row's superblock and its scale row's
      const int slot = (int)(ring - lds) + (g % RG::kDepth) * RG::kStage;
      const int offA = slot + i16 * WS::kRowBytes + (int)((rowA16 + 210u * (uint32_t)g) & 15u);
      const int offS = slot + srow * WS::kRowBytes + (int)((rowS16 + 210u * (uint32_t)g) & 15u);
      const uint8_t* xr = lds + slot + WS::kStage + tj * kXRowBytes;
      const uint32_t* L = reinterpret_cast<const uint32_t*>(lds);
      // the 4 bytes at an even offset o
      auto rd = [&](int o) {
        const int w = o >> 2;
        return __builtin_amdgcn_alignbyte(L[w + 1], L[w], (uint32_t)(o & 3));
      };
      BlockWords bw[kGroup];
      uint32_t nib[kGroup], h0[kGroup], h1[kGroup], scw[kGroup];
#pragma unroll
      for (int k = 0; k < kGroup; ++k) {
        const int ga = offA + 2 + 26 * k;  // group k of the A row
        nib[k] = rd(ga + 2 + 4 * q);
        const int hb = ga + 18, hw = hb >> 2;
        const uint32_t s3 = (uint32_t)(hb & 3);
        const uint32_t t0 = L[hw], t1 = L[hw + 1], t2 = L[hw + 2];
        h0[k] = __builtin_amdgcn_alignbyte(t1, t0, s3);
        h1[k] = __builtin_amdgcn_alignbyte(t2, t1, s3);
        scw[k] = *reinterpret_cast<const uint16_t*>(lds + offS + 2 + 26 * k);
        fetch_x(xr + 34 * k, (k & 1) != 0, q, bw[k]);
      }
      const float d = f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(lds + offS));
#pragma unroll
      for (int k = 0; k < kGroup; ++k) {
        // codes 0..63 of elements 4q..4q+3 (low nibbles and H0) and
        // 16+4q..16+4q+3 (high nibbles and H1), then c - 32 per byte (c + 96
        // has no carry out of its byte; flipping bit 7 gives c - 32 mod 256)
        const uint32_t sh = 2u * (uint32_t)q;
        const uint32_t lo = (nib[k] & 0x0F0F0F0Fu) | (((h0[k] >> sh) & 0x03030303u) << 4);
        const uint32_t hi = ((nib[k] >> 4) & 0x0F0F0F0Fu) | (((h1[k] >> sh) & 0x03030303u) << 4);
        const uint64_t a0 = (uint64_t)((lo + 0x60606060u) ^ 0x80808080u);
        const uint64_t a1 = (uint64_t)((hi + 0x60606060u) ^ 0x80808080u) << 32;
        const uint64_t b = q8_operand(bw[k].x, (k & 1) != 0);
        const i32x4 c0 = __builtin_amdgcn_mfma_i32_16x16x32_i8((long)a0, (long)b, cmagic, 0, 0, 0);
        const i32x4 c1 = __builtin_amdgcn_mfma_i32_16x16x32_i8((long)a1, (long)b, cmagic, 0, 0, 0);
        const float dx = f16_bits_to_f32(bw[k].dxb);
        const float mdx = -kDecMagicF * dx;
        const float S0 = d * (float)(int8_t)(scw[k] & 0xFFu);
        const float S1 = d * (float)(int8_t)(scw[k] >> 8);
        const f32x4 F0 = __builtin_bit_cast(f32x4, c0), F1 = __builtin_bit_cast(f32x4, c1);
        acc[0] = fmaf(fmaf(F1.x, dx, mdx), row_bcast<0>(S1), fmaf(fmaf(F0.x, dx, mdx), row_bcast<0>(S0), acc[0]));
        acc[1] = fmaf(fmaf(F1.y, dx, mdx), row_bcast<1>(S1), fmaf(fmaf(F0.y, dx, mdx), row_bcast<1>(S0), acc[1]));
        acc[2] = fmaf(fmaf(F1.z, dx, mdx), row_bcast<2>(S1), fmaf(fmaf(F0.z, dx, mdx), row_bcast<2>(S0), acc[2]));
        acc[3] = fmaf(fmaf(F1.w, dx, mdx), row_bcast<3>(S1), fmaf(fmaf(F0.w, dx, mdx), row_bcast<3>(S0), acc[3]));
      }
      return;
    }
    const uint8_t* ws = ring + (g % RG::kDepth) * RG::kStage;
    const uint8_t* xs = ws + WS::kStage;
    const uint8_t* wr = ws + i16 * WS::kRowBytes;
    const uint8_t* xr = xs + tj * kXRowBytes;
    const uint8_t* sr = ws + srow * WS::kRowBytes;
    // every LDS word of the stage's 8 blocks first, so the reads overlap
    BlockWords bw[kGroup];
    u32x4 hd = {0u, 0u, 0u, 0u};  // Q4_K-style: the scale row's header
    if (kQ4K) hd = *reinterpret_cast<const u32x4*>(sr);
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      fetch_w<kFmt>(kQ4K ? wr + 16 + 16 * k : wr + k * WS::kBytes, (k & 1) != 0, q, bw[k]);
      fetch_x(xr + 34 * k, (k & 1) != 0, q, bw[k]);
      if (!kQ4K) bw[k].swb = *reinterpret_cast<const uint16_t*>(sr + k * WS::kBytes);
    }
    if (kQ4K) {
      // sub-block k of the scale row: weight = (d sc_k) c - dmin mn_k;
      // sum_i w_i x_i = S_k sum c x - O_k sum x, and sum x comes from a
      // second MFMA with all-ones weights
      const float d = f16_bits_to_f32(hd.x), dmin = f16_bits_to_f32(hd.x >> 16);
      constexpr long kOnes = 0x0101010101010101L;
#pragma unroll
      for (int k = 0; k < kGroup; ++k) {
        const float S = d * (float)field6(hd.y, hd.z, hd.w, k);
        const float O = dmin * (float)field6(hd.y, hd.z, hd.w, 8 + k);
        const bool odd = (k & 1) != 0;
        const uint64_t b = q8_operand(bw[k].x, odd);
        const i32x4 c =
            __builtin_amdgcn_mfma_i32_16x16x32_i8((long)q4k_operand(bw[k].w[0]), (long)b, cmagic, 0, 0, 0);
        const i32x4 cs = __builtin_amdgcn_mfma_i32_16x16x32_i8(kOnes, (long)b, cmagic, 0, 0, 0);
        const float dx = f16_bits_to_f32(bw[k].dxb);
        const float mdx = -kDecMagicF * dx;
        const f32x4 F = __builtin_bit_cast(f32x4, c);
        const float u = fmaf(__builtin_bit_cast(float, cs[0]), dx, mdx);  // dx * sum(xq)
        acc[0] = fmaf(-row_bcast<0>(O), u, fmaf(fmaf(F.x, dx, mdx), row_bcast<0>(S), acc[0]));
        acc[1] = fmaf(-row_bcast<1>(O), u, fmaf(fmaf(F.y, dx, mdx), row_bcast<1>(S), acc[1]));
        acc[2] = fmaf(-row_bcast<2>(O), u, fmaf(fmaf(F.z, dx, mdx), row_bcast<2>(S), acc[2]));
        acc[3] = fmaf(-row_bcast<3>(O), u, fmaf(fmaf(F.w, dx, mdx), row_bcast<3>(S), acc[3]));
      }
      return;
    }
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      const bool odd = (k & 1) != 0;
      const uint64_t a = kQ4 ? q4_operand(bw[k].w, odd) : q8_operand(bw[k].w, odd);
      const uint64_t b = q8_operand(bw[k].x, odd);
      const i32x4 c = __builtin_amdgcn_mfma_i32_16x16x32_i8((long)a, (long)b, cmagic, 0, 0, 0);
      const float dx = f16_bits_to_f32(bw[k].dxb);
      const float mdx = -kDecMagicF * dx;
      const float S = f16_bits_to_f32(bw[k].swb);
      const f32x4 F = __builtin_bit_cast(f32x4, c);
      acc[0] = fmaf(fmaf(F.x, dx, mdx), row_bcast<0>(S), acc[0]);
      acc[1] = fmaf(fmaf(F.y, dx, mdx), row_bcast<1>(S), acc[1]);
      acc[2] = fmaf(fmaf(F.z, dx, mdx), row_bcast<2>(S), acc[2]);
      acc[3] = fmaf(fmaf(F.w, dx, mdx), row_bcast<3>(S), acc[3]);
    }
  };

  for (int i = 0; i < RG::kDepth - 1; ++i)
    if (ga + i < gb) issue(ga + i);
  for (int g = ga; g < gb; ++g) {
    // copies issued after stage g's: stages g + 1 .. min(g + depth - 2, gb - 1)
    const int after = gb - 1 - g < RG::kDepth - 2 ? gb - 1 - g : RG::kDepth - 2;
    wait_stages<RG::kLoads, RG::kDepth - 1>(after);
    // stage g + depth - 1 reuses the slot of stage g - 1, read last iteration
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (g + RG::kDepth - 1 < gb) issue(g + RG::kDepth - 1);
    compute(g);
  }

  // the waves' sums, added in wave order
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);  // [wave][4][64]
#pragma unroll
  for (int v = 0; v < 4; ++v) red[(wv * 4 + v) * kWave + lane] = acc[v];
  __syncthreads();
  if (wv == 0) {
    const int64_t n = n0 + i16;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float s = 0.0f;
      for (int w = 0; w < kWaves; ++w) s += red[(w * 4 + v) * kWave + lane];
      const int64_t m = m0 + 4 * q + v;
      if (m < M && n < N && i16 < NT) Y[n * M + m] = kQ4 ? s * 0.0625f : s;
    }
  }
}

constexpr int64_t kDecOneRound = 256;  // workgroups of one round (the CUs of an MI355X)

constexpr int64_t kDecLongK = 6144;

template <int kFmt, int NT, int kShape>
hipError_t launch_dec_shape(const void* blocks, const void* Xq8, float* Y, int64_t M, int64_t K,
                            int64_t N, int64_t n0, int64_t grid, hipStream_t stream) {
  hipLaunchKernelGGL((decode_mfma_kernel<kFmt, NT, kShape>), dim3((unsigned)grid),
                     dim3(DecRing<kFmt, NT, kShape>::kWaves * kWave), 0, stream,
                     static_cast<const uint8_t*>(blocks), static_cast<const uint8_t*>(Xq8), Y, M,
                     (int)K, N, n0);
  return hipGetLastError();
}

template <int kFmt, int NT>
hipError_t launch_dec(const void* blocks, const void* Xq8, float* Y, int64_t M, int64_t K,
                      int64_t N, int64_t n0, hipStream_t stream) {
  const int64_t grid = (M + kDecRows - 1) / kDecRows;
  if (decode_mfma_tall(M))
    return launch_dec_shape<kFmt, NT, kDecTall>(blocks, Xq8, Y, M, K, N, n0, grid, stream);
  if (K >= kDecLongK)
    return launch_dec_shape<kFmt, NT, kDecLong>(blocks, Xq8, Y, M, K, N, n0, grid, stream);
  return launch_dec_shape<kFmt, NT, kDecOne>(blocks, Xq8, Y, M, K, N, n0, grid, stream);
}

template <int kFmt>
hipError_t launch_dec_fmt(const void* blocks, const void* Xq8, float* Y, int64_t M, int64_t K,
                          int64_t N, int64_t n0, hipStream_t stream) {
  const int64_t nt = N - n0;
  if (nt <= 8) return launch_dec<kFmt, 8>(blocks, Xq8, Y, M, K, N, n0, stream);
  return launch_dec<kFmt, 16>(blocks, Xq8, Y, M, K, N, n0, stream);
}

}  // namespace

#ifndef QMAT_DECODE_MFMA_Q4K
#define QMAT_DECODE_MFMA_Q4K 1
#endif
#ifndef QMAT_DECODE_MFMA_Q6K
#define QMAT_DECODE_MFMA_Q6K 1
#endif
bool decode_mfma_fits(int fmt, int64_t K) {
  return (fmt == kFmtQ4_0 || fmt == kFmtQ8_0 || (QMAT_DECODE_MFMA_Q4K && fmt == kFmtQ4_K) ||
          (QMAT_DECODE_MFMA_Q6K && fmt == kFmtQ6_K)) &&
         K >= 32 * kGroup && K % (32 * kGroup) == 0;
}

bool decode_mfma_tall(int64_t M) { return (M + kDecRows - 1) / kDecRows > kDecOneRound; }

hipError_t launch_decode_mfma(int fmt, const void* blocks, const void* Xq8, float* Y, int64_t M,
                              int64_t K, int64_t N, int64_t n0, hipStream_t stream) {
  if (M == 0 || N <= n0) return hipSuccess;
  switch (fmt) {
    case kFmtQ4_0:
      return launch_dec_fmt<kFmtQ4_0>(blocks, Xq8, Y, M, K, N, n0, stream);
    case kFmtQ8_0:
      return launch_dec_fmt<kFmtQ8_0>(blocks, Xq8, Y, M, K, N, n0, stream);
    case kFmtQ4_K:
      return launch_dec_fmt<kFmtQ4_K>(blocks, Xq8, Y, M, K, N, n0, stream);
    default:
      return launch_dec_fmt<kFmtQ6_K>(blocks, Xq8, Y, M, K, N, n0, stream);
  }
}

}  // namespace qmat
