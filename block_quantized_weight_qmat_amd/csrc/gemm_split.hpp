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
#ifndef QMAT_GEMM_SPLIT_TARGET
#define QMAT_GEMM_SPLIT_TARGET 256
#endif
#ifndef QMAT_GEMM_SPLIT_MIN_STAGES
#define QMAT_GEMM_SPLIT_MIN_STAGES 2
#endif
#ifndef QMAT_GEMM_FILL_STAGES
#define QMAT_GEMM_FILL_STAGES 3
#endif
// measured at 4096 x 11008 and 11008 x 4096 in every format: from 17 to 32
// tokens a split product beats the decode batch
#ifndef QMAT_GEMM_SPLIT_MIN_N
#define QMAT_GEMM_SPLIT_MIN_N 17
#endif
constexpr int64_t kSplitTarget = QMAT_GEMM_SPLIT_TARGET;
constexpr int64_t kMinSplitStages = QMAT_GEMM_SPLIT_MIN_STAGES;
constexpr int64_t kFillStages = QMAT_GEMM_FILL_STAGES;
constexpr int64_t kSplitMinN = QMAT_GEMM_SPLIT_MIN_N;
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

// Workspace for the partial products of ranges 1 .. splits-1 (range 0 is
// written to Y): (splits - 1) * N * M fp32 values.
inline int64_t gemm_workspace_bytes(int fmt, int64_t M, int64_t K, int64_t N) {
  return (int64_t)(gemm_splits(fmt, M, K, N) - 1) * N * M * (int64_t)sizeof(float);
}

}  // namespace qmat
