// Runs the C ABI's argument cases (those of tests/test_abi.py and more)
// against qmat_api.cpp built with sanitizers and stub launchers: every
// rejected call must return its status without reaching a launcher, and
// every accepted call must reach the launchers.
#include <stdio.h>
#include <stdlib.h>

#include <initializer_list>

#include "qmat.h"

extern int g_launches;

static int failures = 0;
#define EXPECT(call, want, launches)                                                   \
  do {                                                                                 \
    const int before = g_launches;                                                     \
    const int got = (call);                                                            \
    if (got != (want) || g_launches - before != (launches)) {                          \
      fprintf(stderr, "FAIL line %d: %s -> %d (want %d), %d launches (want %d)\n",     \
              __LINE__, #call, got, (want), g_launches - before, (launches));          \
      ++failures;                                                                      \
    }                                                                                  \
  } while (0)

int main() {
  void* A = (void*)0x10000;  // aligned stand-in addresses: never dereferenced
  char* Ab = (char*)A;
  float* F = (float*)A;
  const int64_t big = (int64_t)1 << 31;
  // sizes
  for (int f = -3; f < 8; ++f) {
    const int64_t be = qmat_block_elems(f), bb = qmat_block_bytes(f);
    if ((f >= 0 && f <= 3) != (be > 0 && bb > 0)) ++failures;
    for (int64_t K : {(int64_t)-32, (int64_t)0, (int64_t)31, (int64_t)32, (int64_t)256,
                      (int64_t)1 << 40, INT64_MAX, INT64_MAX - 31, INT64_MAX - 255})
      (void)qmat_row_bytes(f, K);
  }
  if (qmat_row_bytes(0, 33) != -1 || qmat_row_bytes(2, 32) != -1) ++failures;
  if (qmat_row_bytes(1, INT64_MAX - 31) != -1) ++failures;  // beyond int64 bytes
  if (qmat_row_bytes(0, (int64_t)1 << 40) != ((int64_t)1 << 35) * 18) ++failures;
  for (int s = -1; s < 10; ++s)
    if (qmat_strerror(s) == NULL) ++failures;
  // formats
  EXPECT(qmat_quantize(4, F, A, 1, 32, NULL), QMAT_E_FMT, 0);
  EXPECT(qmat_gemv(-1, A, F, F, 1, 32, NULL), QMAT_E_FMT, 0);
  EXPECT(qmat_gemm(5, A, A, F, 1, 32, 1, NULL), QMAT_E_FMT, 0);
  EXPECT(qmat_kv_write(2, F, NULL, A, 0, 1, 4, 256, NULL), QMAT_E_FMT, 0);
  EXPECT(qmat_prefill_noalloc(9, A, F, F, 1, 32, 1, NULL), QMAT_E_FMT, 0);
  // shapes, including values near the int64 edge
  EXPECT(qmat_quantize(0, F, A, 1, 48, NULL), QMAT_E_SHAPE, 0);
  EXPECT(qmat_quantize(2, F, A, 1, 288, NULL), QMAT_E_SHAPE, 0);
  EXPECT(qmat_quantize(1, F, A, -1, 32, NULL), QMAT_E_SHAPE, 0);
  EXPECT(qmat_quantize(1, F, A, INT64_MAX, 32, NULL), QMAT_E_SHAPE, 0);
  EXPECT(qmat_quantize(1, F, A, 1, INT64_MAX - 31, NULL), QMAT_E_SHAPE, 0);
  EXPECT(qmat_quantize(1, F, A, big - 1, big - 32, NULL), QMAT_E_SHAPE, 0);
  EXPECT(qmat_gemv(0, A, F, F, -5, 32, NULL), QMAT_E_SHAPE, 0);
  EXPECT(qmat_gemv(0, A, F, F, big, 32, NULL), QMAT_E_SHAPE, 0);
  EXPECT(qmat_gemv(0, A, F, F, 1, big + 32, NULL), QMAT_E_SHAPE, 0);
  EXPECT(qmat_gemm(0, A, A, F, 1, 32, -1, NULL), QMAT_E_SHAPE, 0);
  EXPECT(qmat_gemm(2, A, A, F, 1, 32, 1, NULL), QMAT_E_SHAPE, 0);
  EXPECT(qmat_gemm(0, A, A, F, 1, (1 << 24) + 32, 1, NULL), QMAT_E_SHAPE, 0);
  EXPECT(qmat_gemm(0, A, A, F, big - 1, big - 32, big - 1, NULL), QMAT_E_SHAPE, 0);
  EXPECT(qmat_prefill(0, A, F, A, F, 1, (1 << 24) + 32, 1, NULL), QMAT_E_SHAPE, 0);
  EXPECT(qmat_kv_write(0, F, NULL, A, 0, 1, 4, 48, NULL), QMAT_E_SHAPE, 0);
  EXPECT(qmat_kv_write(0, F, NULL, A, 3, 2, 4, 256, NULL), QMAT_E_SHAPE, 0);
  EXPECT(qmat_kv_write(0, F, NULL, A, INT64_MAX, 2, 4, 256, NULL), QMAT_E_SHAPE, 0);
  EXPECT(qmat_kv_write(0, F, NULL, A, -1, 1, 4, 256, NULL), QMAT_E_SHAPE, 0);
  EXPECT(qmat_prefill_noalloc(0, A, F, F, 4, 11008, 2000, NULL), QMAT_E_SCRATCH, 0);
  EXPECT(qmat_prefill_noalloc(0, A, F, F, 4, 32, big - 1, NULL), QMAT_E_SCRATCH, 0);
  // pointers
  EXPECT(qmat_quantize(0, NULL, A, 1, 32, NULL), QMAT_E_NULL, 0);
  EXPECT(qmat_gemv(0, A, F, NULL, 1, 32, NULL), QMAT_E_NULL, 0);
  EXPECT(qmat_gemm(0, A, NULL, F, 1, 32, 1, NULL), QMAT_E_NULL, 0);
  EXPECT(qmat_prefill(0, A, F, NULL, F, 1, 32, 1, NULL), QMAT_E_NULL, 0);
  EXPECT(qmat_kv_write(0, F, NULL, NULL, 0, 1, 4, 256, NULL), QMAT_E_NULL, 0);
  EXPECT(qmat_quantize(0, (float*)(Ab + 4), A, 1, 32, NULL), QMAT_E_ALIGN, 0);
  EXPECT(qmat_gemm(1, A, Ab + 8, F, 1, 32, 1, NULL), QMAT_E_ALIGN, 0);
  EXPECT(qmat_kv_write(0, F, (float*)(Ab + 4), A, 0, 1, 4, 256, NULL), QMAT_E_ALIGN, 0);
  EXPECT(qmat_kv_write(0, F, NULL, A, 1, 1, 4, 32, NULL), QMAT_E_ALIGN, 0);  // 18-byte rows
  // nothing to do: no pointer needed, nothing launched
  EXPECT(qmat_quantize(0, NULL, NULL, 0, 32, NULL), QMAT_OK, 0);
  EXPECT(qmat_gemv(1, NULL, NULL, NULL, 0, 64, NULL), QMAT_OK, 0);
  EXPECT(qmat_gemm(0, NULL, NULL, NULL, 3, 64, 0, NULL), QMAT_OK, 0);
  EXPECT(qmat_kv_write(0, NULL, NULL, NULL, 0, 0, 4, 256, NULL), QMAT_OK, 0);
  // batched GEMVs: every job checked before anything is enqueued
  {
    qmat_gemv_job good = {A, F, F, 64, 1024};
    qmat_gemv_job jobs[3] = {good, good, good};
    EXPECT(qmat_gemv_batch(7, jobs, 3, NULL), QMAT_E_FMT, 0);
    EXPECT(qmat_gemv_batch(0, jobs, -1, NULL), QMAT_E_SHAPE, 0);
    EXPECT(qmat_gemv_batch(0, NULL, 2, NULL), QMAT_E_NULL, 0);
    EXPECT(qmat_gemv_batch(0, NULL, 0, NULL), QMAT_OK, 0);
    jobs[2].K = 48;
    EXPECT(qmat_gemv_batch(0, jobs, 3, NULL), QMAT_E_SHAPE, 0);
    jobs[2].K = 1024;
    jobs[1].y = (float*)(Ab + 4);
    EXPECT(qmat_gemv_batch(0, jobs, 3, NULL), QMAT_E_ALIGN, 0);
    jobs[1].y = NULL;
    EXPECT(qmat_gemv_batch(0, jobs, 3, NULL), QMAT_E_NULL, 0);
    jobs[1].M = 0;  // skipped: no pointer needed
    EXPECT(qmat_gemv_batch(0, jobs, 3, NULL), QMAT_OK, 1);
    jobs[0].M = INT64_MAX;
    EXPECT(qmat_gemv_batch(0, jobs, 3, NULL), QMAT_E_SHAPE, 0);
  }
  // the K-split GEMM: the workspace size is a function of the shape, and
  // the workspace is checked after qmat_gemm's arguments
  {
    const int64_t need = qmat_gemm_workspace_bytes(0, 4096, 11008, 64);
    if (need != (int64_t)7 * 64 * 4096 * 4) ++failures;
    if (qmat_gemm_workspace_bytes(0, 4096, 11008, 16) != 0) ++failures;
    if (qmat_gemm_workspace_bytes(0, 4096, 11008, 512) != 0) ++failures;
    if (qmat_gemm_workspace_bytes(9, 4096, 11008, 64) != -1) ++failures;
    if (qmat_gemm_workspace_bytes(0, big - 1, big - 32, big - 1) != -1) ++failures;  // K limit
    for (int64_t N : {(int64_t)0, (int64_t)17, (int64_t)1 << 20, big - 1})
      for (int64_t M : {(int64_t)1, (int64_t)4096, big - 1})
        if (qmat_gemm_workspace_bytes(3, M, 1 << 24, N) < 0) ++failures;
    EXPECT(qmat_gemm_ws(7, A, A, F, 4096, 11008, 64, A, need, NULL), QMAT_E_FMT, 0);
    EXPECT(qmat_gemm_ws(0, A, A, NULL, 4096, 11008, 64, A, need, NULL), QMAT_E_NULL, 0);
    EXPECT(qmat_gemm_ws(0, A, A, F, 4096, 11008, 64, A, -1, NULL), QMAT_E_SHAPE, 0);
    EXPECT(qmat_gemm_ws(0, A, A, F, 4096, 11008, 64, NULL, need, NULL), QMAT_E_WORKSPACE, 0);
    EXPECT(qmat_gemm_ws(0, A, A, F, 4096, 11008, 64, A, need - 1, NULL), QMAT_E_WORKSPACE, 0);
    EXPECT(qmat_gemm_ws(0, A, A, F, 4096, 11008, 64, Ab + 4, need, NULL), QMAT_E_ALIGN, 0);
    EXPECT(qmat_gemm_ws(0, A, A, F, 4096, 11008, 64, A, need, NULL), QMAT_OK, 1);
    EXPECT(qmat_gemm_ws(0, A, A, F, 4096, 11008, 16, NULL, 0, NULL), QMAT_OK, 1);  // no split
    EXPECT(qmat_gemm_ws(0, NULL, NULL, NULL, 0, 11008, 64, NULL, 0, NULL), QMAT_OK, 0);
  }
  // accepted calls reach the launchers (quantize + gemm for the prefills)
  EXPECT(qmat_quantize(3, F, A, 7, 512, NULL), QMAT_OK, 1);
  EXPECT(qmat_gemv(0, A, F, F, 4096, 11008, NULL), QMAT_OK, 1);
  EXPECT(qmat_gemv(0, NULL, NULL, F, 5, 0, NULL), QMAT_OK, 1);  // K = 0 writes zeros
  EXPECT(qmat_gemm(1, A, A, F, 4096, 11008, 512, NULL), QMAT_OK, 1);
  EXPECT(qmat_prefill(2, A, F, A, F, 64, 2048, 70, NULL), QMAT_OK, 2);
  EXPECT(qmat_prefill_noalloc(0, A, F, F, 4096, 11008, 512, NULL), QMAT_OK, 2);
  EXPECT(qmat_prefill_noalloc(0, A, F, F, 64, 0, 9, NULL), QMAT_OK, 1);  // K = 0: GEMM only
  EXPECT(qmat_kv_write(1, F, F, A, 16, 2, 40, 256, NULL), QMAT_OK, 1);
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("abi driver: all cases ok\n");
  return 0;
}
