// gemm_split.hpp — how qmat_gemm_ws divides a prefill product along K
// (host code, shared by the launcher and the argument checks).
//
// The prefill kernel (gemm.hip) computes 128 x 64 output tiles, one
// workgroup per CU (its LDS allows one), stepping through K in stages of 8
// blocks of 32. A product of few tiles leaves CUs idle, so its K blocks can
// also be cut into `splits` contiguous ranges of whole stages (pairs of
// stages for Q6_K-style, whose 210-byte stages alternate alignment), each
// range's partial product computed as a product of its own and the
// partials added afterwards.
//
// The split count minimises the modelled time
//   ceil(tiles * splits / kSplitTarget) * (stages of the longest range + kFillStages)
//   + the adding kernel,
// i.e. rounds of one workgroup per CU (an MI355X has 256), each as long as
// its range plus the fill of a tile's pipeline (about 3 stages, measured: a
// 6-stage range of 4096 x 11008 at 64 tokens takes as long as 9-10 stages
// of a long one). The adding kernel costs one stage plus one per
// kAddBytesPerStage bytes of partial products (a stage takes about 1.7 us;
// the adds move about 4 TB/s). A split is taken only when the model
// promises at least 15% (its error on measured shapes: a second round of
// workgroups gains less than it says), from kSplitMinN tokens (below, the
// decode batch's streaming of W once per 16 tokens is faster), with ranges
// of at least kMinSplitStages stages.
#pragma once

#include <stdint.h>

namespace qmat {
namespace split {

constexpr int64_t kTileM = 128, kTileN = 64, kStageBlocks = 8;  // gemm.hip's tile and stage
// The policy is plain constants, not build options: the launcher and the
// argument checks (qmat_gemm_workspace_bytes) are separate translation
// units and must agree on the workspace a shape needs.
constexpr int64_t kSplitTarget = 256;
constexpr int64_t kMinSplitStages = 2;
constexpr int64_t kFillStages = 3;
// measured at 4096 x 11008 and 11008 x 4096 in every format: from 17 to 32
// tokens a split product beats the decode batch
constexpr int64_t kSplitMinN = 17;
constexpr double kAddBytesPerStage = 6.8e6;
constexpr int64_t kMaxSplit = 16;
constexpr int64_t kMaxSplitTiles = 1 << 24;  // tiles of all ranges together

}  // namespace split

// K ranges for (fmt, M, K, N); 1 = not split. fmt 3 is Q6_K-style.
inline int gemm_splits(int fmt, int64_t M, int64_t K, int64_t N) {
  using namespace split;
  if (M <= 0 || N < kSplitMinN || K <= 0) return 1;
  const int64_t tiles = ((M + kTileM - 1) / kTileM) * ((N + kTileN - 1) / kTileN);
  const int64_t nst = (K / 32 + kStageBlocks - 1) / kStageBlocks;
  const int64_t unit = fmt == 3 ? 2 : 1;
  const int64_t units = (nst + unit - 1) / unit;
  int best_s = 1;
  double best = 0.85 * (double)(((tiles + kSplitTarget - 1) / kSplitTarget) * (nst + kFillStages));
  for (int64_t sp = 2; sp <= kMaxSplit && sp <= units && tiles * sp <= kMaxSplitTiles; ++sp) {
    const int64_t per = (units + sp - 1) / sp * unit;  // stages of the longest range
    if (per < kMinSplitStages) break;
    const double cost =
        (double)(((tiles * sp + kSplitTarget - 1) / kSplitTarget) * (per + kFillStages)) + 1.0 +
        (double)(sp - 1) * (double)N * (double)M * 4.0 / kAddBytesPerStage;
    if (cost < best) {
      best = cost;
      best_s = (int)sp;
    }
  }
  return best_s;
}

// Without a K split: whether N tokens go to the decode batch's kernels (the
// weights streamed once per 16 tokens) instead of the 128 x 64 tiles. A
// model of the two, in microseconds: the tiles take
//   ceil(tiles / kSplitTarget) * (stages + kFillStages) * s_fmt
// (s_fmt about 1.3 us per stage for Q4_0 while at most one round of
// workgroups runs, scaled by the formats' measured GEMM times), and each
// chunk of up to 16 tokens of the decode batch
//   (3.5 + 0.2 * M * K / 10^6) * d_fmt
// (a fit of the matrix-core kernel's Q4_0 times at 16 tokens: 12.9 us at
// 4096 x 11008, 6.3 at 4096 x 4096, 13.4 at 11008 x 4096, 16.9 at
// 14336 x 4096, 26.5 at 28672 x 4096, 7.9 at 11008 x 2048, 16.0 at
// 8192 x 8192; d_fmt scales it by the formats' measured chunk times: 1,
// 1.2, 1.2 and 1.55 for Q4_0, Q8_0, Q4_K-style and Q6_K-style), half that
// for chunks of up to 4 tokens (the row-per-wave kernel). Measured against a fixed limit of 48
// tokens: 4096 x 11008 at 56 / 64 tokens 59.0 -> 43.5 / 44.9 us (Q4_0) and
// 79.8 / 80.0 -> 53.0 / 53.5 (Q4_K-style); 11008 x 4096 Q4_0 at 24 / 48
// tokens 28.5 / 48.2 -> 25.8 / 26.4.
constexpr int64_t kDecodeMaxN = 64;
inline bool gemm_uses_decode(int fmt, int64_t M, int64_t K, int64_t N) {
  using namespace split;
  if (N <= 16) return true;
  if (N > kDecodeMaxN) return false;
  static constexpr double kStageUs[4] = {1.3, 1.35, 1.7, 2.2};  // Q4_0, Q8_0, Q4_K, Q6_K
  static constexpr double kChunk[4] = {1.0, 1.2, 1.2, 1.55};
  const int f = fmt >= 0 && fmt < 4 ? fmt : 0;
  const int64_t tiles = ((M + kTileM - 1) / kTileM) * ((N + kTileN - 1) / kTileN);
  const int64_t nst = (K / 32 + kStageBlocks - 1) / kStageBlocks;
  const double t_tiles =
      (double)((tiles + kSplitTarget - 1) / kSplitTarget) * (double)(nst + kFillStages) * kStageUs[f];
  const double chunk = 3.5 + 0.2e-6 * (double)M * (double)K;
  const int64_t tail = N % 16;
  const double t_dec = (double)(N / 16) * chunk * kChunk[f] +
                       (tail == 0 ? 0.0 : tail <= 4 ? 0.5 * chunk : chunk * kChunk[f]);
  return t_dec < t_tiles;
}

// Workspace for the partial products of ranges 1 .. splits-1 (range 0 is
// written to Y): (splits - 1) * N * M fp32 values.
inline int64_t gemm_workspace_bytes(int fmt, int64_t M, int64_t K, int64_t N) {
  return (int64_t)(gemm_splits(fmt, M, K, N) - 1) * N * M * (int64_t)sizeof(float);
}

}  // namespace qmat
