// qmat_launch.hpp — internal launchers behind the C ABI (include/qmat.h).
// Arguments are already validated by the caller (qmat_api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_split.hpp"

namespace qmat {

constexpr int kFmtQ4_0 = 0;
constexpr int kFmtQ8_0 = 1;
constexpr int kFmtQ4_K = 2;
constexpr int kFmtQ6_K = 3;

hipError_t launch_quantize(int fmt, const float* W, void* blocks, int64_t rows, int64_t K,
                           hipStream_t stream);

// KV-cache write: n rows of dim elements, minus bias when non-null, as Q4_0
// or Q8_0 rows at dst (16-byte aligned).
hipError_t launch_kv_write(int fmt, const float* rows, const float* bias, void* dst, int64_t n,
                           int64_t dim, hipStream_t stream);

hipError_t launch_gemv(int fmt, const void* blocks, const float* x, float* y, int64_t M,
                       int64_t K, hipStream_t stream);

// One GEMV of a batch (the layout of qmat_gemv_job).
struct GemvJob {
  const void* blocks;
  const float* x;
  float* y;
  int64_t M, K;
};
hipError_t launch_gemv_batch(int fmt, const GemvJob* jobs, int64_t count, hipStream_t stream);

// Few-token product (the decode batch): W streamed once per 16 tokens.
hipError_t launch_gemm_small(int fmt, const void* blocks, const void* Xq8, float* Y, int64_t M,
                             int64_t K, int64_t N, hipStream_t stream);

// The decode batch on the matrix cores (decode.hip): rows of whole
// 256-element groups (K a positive multiple of 256) in any format; tokens
// n0 .. min(N, n0 + 16) - 1 of one launch (sized for 5 to 16 of them).
// decode_mfma_tall: whether M rows take its tall-matrix shape (more 16-row
// workgroups than CUs).
bool decode_mfma_fits(int fmt, int64_t K);
bool decode_mfma_tall(int64_t M);
hipError_t launch_decode_mfma(int fmt, const void* blocks, const void* Xq8, float* Y, int64_t M,
                              int64_t K, int64_t N, int64_t n0, hipStream_t stream);

// Prefill product (gemm.hip). With part non-NULL (gemm_workspace_bytes()
// bytes), it is split along K into gemm_splits() ranges (gemm_split.hpp)
// whose partial products go to Y and to part, then added into Y.
hipError_t launch_gemm(int fmt, const void* blocks, const void* Xq8, float* Y, int64_t M,
                       int64_t K, int64_t N, float* part, hipStream_t stream);


}  // namespace qmat
