// qmat_api.cpp — the C ABI declared in include/qmat.h.
//
// Every argument is validated on the host before anything is enqueued; the
// launchers in quantize.hip / gemv.hip / gemm.hip then enqueue the kernels on
// the caller's stream. No device memory is allocated. The one piece of
// library-owned device memory is the static activation workspace of
// qmat_prefill_noalloc below (a module global, resolved once per device).
#include "qmat.h"

#include <hip/hip_runtime.h>

#include <cstddef>
#include <mutex>

#include "qmat_launch.hpp"

namespace {

constexpr int64_t kMaxDim = 0x7FFFFFFFLL;
// The GEMM addresses a 128-row tile of W (and a 64-row tile of X_q8) with
// 32-bit byte offsets: 129 Q8_0 rows of K = 2^24 take 2.3e9 bytes.
constexpr int64_t kMaxGemmK = 1LL << 24;

bool fmt_ok(int fmt) {
  return fmt == QMAT_Q4_0 || fmt == QMAT_Q8_0 || fmt == QMAT_Q4_K || fmt == QMAT_Q6_K;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A buffer that must exist (non-empty) must be non-NULL and 16-byte aligned.
int check_buf(const void* p, bool nonempty) {
  if (!nonempty) return QMAT_OK;
  if (p == nullptr) return QMAT_E_NULL;
  if (!aligned16(p)) return QMAT_E_ALIGN;
  return QMAT_OK;
}

// rows x K matrix in fmt: sizes in range, K a multiple of the block, and the
// packed byte size representable.
int check_shape(int fmt, int64_t rows, int64_t K) {
  if (rows < 0 || K < 0 || rows > kMaxDim || K > kMaxDim) return QMAT_E_SHAPE;
  const int64_t be = qmat_block_elems(fmt);
  if (K % be != 0) return QMAT_E_SHAPE;
  const int64_t rb = qmat_row_bytes(fmt, K);
  if (rb > 0 && rows > INT64_MAX / rb) return QMAT_E_SHAPE;
  if (rows > 0 && K > INT64_MAX / 4 / rows) return QMAT_E_SHAPE;
  return QMAT_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? QMAT_OK : QMAT_E_HIP; }

// Arguments of the one-call prefill (with or without a caller workspace):
// format, shapes, the GEMM's K limit; QMAT_OK with *empty set when there is
// nothing to do.
int check_prefill(int fmt, int64_t M, int64_t K, int64_t N, bool* empty) {
  *empty = false;
  if (!fmt_ok(fmt)) return QMAT_E_FMT;
  int rc = check_shape(fmt, M, K);
  if (rc != QMAT_OK) return rc;
  if ((rc = check_shape(QMAT_Q8_0, N, K)) != QMAT_OK) return rc;
  if (K > kMaxGemmK) return QMAT_E_SHAPE;
  *empty = M == 0 || N == 0;
  return QMAT_OK;
}

// ---- static workspace of qmat_prefill_noalloc ----------------------------
// Each device that runs the library holds one copy of this array until the
// process ends. In host code `scratch` is only a stand-in for the symbol:
// its device address comes from hipGetSymbolAddress, called once per device
// with that device current, and only that address is ever passed on.
static __device__ __align__(256) uint8_t scratch[QMAT_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of the current device's workspace (nullptr on failure).
void* scratch_for_current_device(int* status) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = QMAT_E_HIP;
    return nullptr;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) {
    *status = QMAT_E_HIP;
    return nullptr;
  }
  *status = QMAT_OK;
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int64_t qmat_block_elems(int fmt) {
  switch (fmt) {
    case QMAT_Q4_0: return 32;
    case QMAT_Q8_0: return 32;
    case QMAT_Q4_K: return 256;
    case QMAT_Q6_K: return 256;
    default: return 0;
  }
}

int64_t qmat_block_bytes(int fmt) {
  switch (fmt) {
    case QMAT_Q4_0: return 18;
    case QMAT_Q8_0: return 34;
    case QMAT_Q4_K: return 144;
    case QMAT_Q6_K: return 210;
    default: return 0;
  }
}

int64_t qmat_row_bytes(int fmt, int64_t K) {
  if (!fmt_ok(fmt) || K < 0) return -1;
  const int64_t be = qmat_block_elems(fmt), bb = qmat_block_bytes(fmt);
  if (K % be != 0 || K / be > INT64_MAX / bb) return -1;
  return K / be * bb;
}

const char* qmat_strerror(int status) {
  switch (status) {
    case QMAT_OK: return "success";
    case QMAT_E_FMT: return "unknown or unsupported block format";
    case QMAT_E_SHAPE: return "invalid shape (negative, out of range, or K not a multiple of the block)";
    case QMAT_E_NULL: return "required pointer is NULL";
    case QMAT_E_HIP: return "HIP kernel launch failed";
    case QMAT_E_ALIGN: return "pointer is not 16-byte aligned";
    case QMAT_E_SCRATCH:
      return "the Q8_0 activations (N * row bytes) exceed the static workspace of "
             "qmat_prefill_noalloc (qmat_noalloc_scratch_bytes())";
    case QMAT_E_WORKSPACE:
      return "the workspace is NULL or smaller than qmat_gemm_workspace_bytes()";
    default: return "unknown status";
  }
}

int qmat_quantize(int fmt, const float* W, void* blocks, int64_t rows, int64_t K,
                  void* stream) {
  if (!fmt_ok(fmt)) return QMAT_E_FMT;
  int rc = check_shape(fmt, rows, K);
  if (rc != QMAT_OK) return rc;
  if (rows == 0 || K == 0) return QMAT_OK;  // nothing to read or write
  if ((rc = check_buf(W, true)) != QMAT_OK) return rc;
  if ((rc = check_buf(blocks, true)) != QMAT_OK) return rc;
  return hip_status(
      qmat::launch_quantize(fmt, W, blocks, rows, K, static_cast<hipStream_t>(stream)));
}

int qmat_gemv(int fmt, const void* blocks, const float* x, float* y, int64_t M, int64_t K,
              void* stream) {
  if (!fmt_ok(fmt)) return QMAT_E_FMT;
  int rc = check_shape(fmt, M, K);
  if (rc != QMAT_OK) return rc;
  if (M == 0) return QMAT_OK;  // nothing to read or write
  if ((rc = check_buf(blocks, K > 0)) != QMAT_OK) return rc;
  if ((rc = check_buf(x, K > 0)) != QMAT_OK) return rc;
  if ((rc = check_buf(y, true)) != QMAT_OK) return rc;
  return hip_status(qmat::launch_gemv(fmt, blocks, x, y, M, K, static_cast<hipStream_t>(stream)));
}

static_assert(sizeof(qmat_gemv_job) == sizeof(qmat::GemvJob) &&
                  offsetof(qmat_gemv_job, M) == offsetof(qmat::GemvJob, M) &&
                  offsetof(qmat_gemv_job, K) == offsetof(qmat::GemvJob, K),
              "job layouts");

int qmat_gemv_batch(int fmt, const qmat_gemv_job* jobs, int64_t count, void* stream) {
  if (!fmt_ok(fmt)) return QMAT_E_FMT;
  if (count < 0) return QMAT_E_SHAPE;
  if (count == 0) return QMAT_OK;
  if (jobs == nullptr) return QMAT_E_NULL;
  for (int64_t i = 0; i < count; ++i) {
    const qmat_gemv_job& j = jobs[i];
    int rc = check_shape(fmt, j.M, j.K);
    if (rc != QMAT_OK) return rc;
    if (j.M == 0) continue;
    if ((rc = check_buf(j.blocks, j.K > 0)) != QMAT_OK) return rc;
    if ((rc = check_buf(j.x, j.K > 0)) != QMAT_OK) return rc;
    if ((rc = check_buf(j.y, true)) != QMAT_OK) return rc;
  }
  return hip_status(qmat::launch_gemv_batch(fmt, reinterpret_cast<const qmat::GemvJob*>(jobs),
                                            count, static_cast<hipStream_t>(stream)));
}

namespace {
// qmat_gemm's checks; *empty when there is nothing to read or write
int check_gemm(int fmt, const void* blocks, const void* X_q8, const float* Y, int64_t M,
               int64_t K, int64_t N, bool* empty) {
  if (!fmt_ok(fmt)) return QMAT_E_FMT;
  int rc = check_shape(fmt, M, K);
  if (rc != QMAT_OK) return rc;
  if ((rc = check_shape(QMAT_Q8_0, N, K)) != QMAT_OK) return rc;
  if (K > kMaxGemmK) return QMAT_E_SHAPE;
  *empty = M == 0 || N == 0;
  if (*empty) return QMAT_OK;
  if ((rc = check_buf(blocks, K > 0)) != QMAT_OK) return rc;
  if ((rc = check_buf(X_q8, K > 0)) != QMAT_OK) return rc;
  return check_buf(Y, true);
}
}  // namespace

int qmat_gemm(int fmt, const void* blocks, const void* X_q8, float* Y, int64_t M, int64_t K,
              int64_t N, void* stream) {
  bool empty = false;
  int rc = check_gemm(fmt, blocks, X_q8, Y, M, K, N, &empty);
  if (rc != QMAT_OK || empty) return rc;
  return hip_status(qmat::launch_gemm(fmt, blocks, X_q8, Y, M, K, N, nullptr,
                                      static_cast<hipStream_t>(stream)));
}

int64_t qmat_gemm_workspace_bytes(int fmt, int64_t M, int64_t K, int64_t N) {
  if (!fmt_ok(fmt) || check_shape(fmt, M, K) != QMAT_OK ||
      check_shape(QMAT_Q8_0, N, K) != QMAT_OK || K > kMaxGemmK)
    return -1;
  return qmat::gemm_workspace_bytes(fmt, M, K, N);
}

int qmat_gemm_ws(int fmt, const void* blocks, const void* X_q8, float* Y, int64_t M, int64_t K,
                 int64_t N, void* workspace, int64_t workspace_bytes, void* stream) {
  bool empty = false;
  int rc = check_gemm(fmt, blocks, X_q8, Y, M, K, N, &empty);
  if (rc != QMAT_OK || empty) return rc;
  if (workspace_bytes < 0) return QMAT_E_SHAPE;
  const int64_t need = qmat::gemm_workspace_bytes(fmt, M, K, N);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return QMAT_E_WORKSPACE;
    if ((rc = check_buf(workspace, true)) != QMAT_OK) return rc;
  }
  return hip_status(qmat::launch_gemm(fmt, blocks, X_q8, Y, M, K, N,
                                      need > 0 ? static_cast<float*>(workspace) : nullptr,
                                      static_cast<hipStream_t>(stream)));
}

int qmat_prefill(int fmt, const void* blocks, const float* X, void* xq, float* Y, int64_t M,
                 int64_t K, int64_t N, void* stream) {
  bool empty = false;
  int rc = check_prefill(fmt, M, K, N, &empty);
  if (rc != QMAT_OK) return rc;
  if (empty) return QMAT_OK;  // nothing to read or write
  if ((rc = check_buf(blocks, K > 0)) != QMAT_OK) return rc;
  if ((rc = check_buf(X, K > 0)) != QMAT_OK) return rc;
  if ((rc = check_buf(xq, K > 0)) != QMAT_OK) return rc;
  if ((rc = check_buf(Y, true)) != QMAT_OK) return rc;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (K > 0 && (rc = hip_status(qmat::launch_quantize(QMAT_Q8_0, X, xq, N, K, st))) != QMAT_OK)
    return rc;
  return hip_status(qmat::launch_gemm(fmt, blocks, xq, Y, M, K, N, nullptr, st));
}

int64_t qmat_noalloc_scratch_bytes(void) { return QMAT_NOALLOC_SCRATCH_BYTES; }

int qmat_prefill_noalloc(int fmt, const void* blocks, const float* X, float* Y, int64_t M,
                         int64_t K, int64_t N, void* stream) {
  bool empty = false;
  int rc = check_prefill(fmt, M, K, N, &empty);
  if (rc != QMAT_OK) return rc;
  if (empty) return QMAT_OK;  // nothing to read or write
  // N * row bytes cannot overflow: check_shape bounded it by INT64_MAX
  if (N * qmat_row_bytes(QMAT_Q8_0, K) > (int64_t)QMAT_NOALLOC_SCRATCH_BYTES)
    return QMAT_E_SCRATCH;
  if ((rc = check_buf(blocks, K > 0)) != QMAT_OK) return rc;
  if ((rc = check_buf(X, K > 0)) != QMAT_OK) return rc;
  if ((rc = check_buf(Y, true)) != QMAT_OK) return rc;
  void* xq = scratch_for_current_device(&rc);
  if (xq == nullptr) return rc;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (K > 0 && (rc = hip_status(qmat::launch_quantize(QMAT_Q8_0, X, xq, N, K, st))) != QMAT_OK)
    return rc;
  return hip_status(qmat::launch_gemm(fmt, blocks, xq, Y, M, K, N, nullptr, st));
}

int qmat_kv_write(int fmt, const float* rows, const float* bias, void* cache, int64_t cell0,
                  int64_t n, int64_t cells, int64_t dim, void* stream) {
  if (fmt != QMAT_Q4_0 && fmt != QMAT_Q8_0) return QMAT_E_FMT;
  int rc = check_shape(fmt, cells, dim);
  if (rc != QMAT_OK) return rc;
  if (n < 0 || cell0 < 0 || n > cells || cell0 > cells - n) return QMAT_E_SHAPE;
  if (n == 0 || dim == 0) return QMAT_OK;  // nothing to read or write
  if ((rc = check_buf(rows, true)) != QMAT_OK) return rc;
  if (cache == nullptr) return QMAT_E_NULL;
  void* dst = static_cast<uint8_t*>(cache) + cell0 * qmat_row_bytes(fmt, dim);
  if ((rc = check_buf(dst, true)) != QMAT_OK) return rc;
  if (bias != nullptr && (rc = check_buf(bias, true)) != QMAT_OK) return rc;
  return hip_status(
      qmat::launch_kv_write(fmt, rows, bias, dst, n, dim, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
