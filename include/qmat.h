/*
 * qmat.h — C ABI of the block-quantized weight matmul for MI355X (gfx950).
 *
 * Six operations, all enqueued asynchronously on a caller-supplied HIP
 * stream:
 *   qmat_quantize  fp32 matrix  -> packed weight (or activation) blocks
 *   qmat_gemv      packed W × fp32 x        -> fp32 y        (decode)
 *   qmat_gemv_batch many independent GEMVs, few launches     (decode)
 *   qmat_gemm      packed W × Q8_0 X blocks -> fp32 Y        (prefill)
 *   qmat_prefill   packed W × fp32 X        -> fp32 Y        (prefill, one call)
 *   qmat_kv_write  fp32 K or V rows -> Q4_0 / Q8_0 rows of a KV cache
 * and qmat_prefill_noalloc, qmat_prefill without a caller workspace for
 * callers that cannot allocate device memory.
 *
 * Sources. Citations name the web page and the section or table of it
 * that fixes the fact:
 *   [LC05] "05. llama.cpp：从 GGUF 文件到本地推理服务" (niuwancheng.cn);
 *          table in section "量化类型：Q4_K_M 到底是什么" (quant families),
 *          section "性能直觉：带宽决定 Decode，算力决定 Prefill".
 *   [LCHW] "llama.cpp 原理：如何在普通硬件跑本地大模型"; section
 *          "量化：内存真正去哪了" (Q4_0: 32 weights, one fp16 scale,
 *          18 bytes, 4.5 bits per weight).
 *   [KVQ]  lpnh.cn KV-cache article; section "kv-mean-center 进阶技巧",
 *          paragraph "问题" (Q4_0 is symmetric: value ≈ scale × q), and
 *          the same section's bias subtracted from K before Q4_0
 *          quantization; section "量化 KV Cache 的一键配置方法" (K and V
 *          caches stored as q8_0 or q4_0).
 *   [BARE] xdnf.cn llama.cpp article; section 3.2 (dequant snippet: low
 *          nibbles are the first 16 elements of a block, high nibbles the
 *          last 16; fp16 parameters precede the nibbles).
 *   [LC05 KV] [LC05] section "KV Cache 类型与 Flash Attention" (the q6_K
 *          token embedding of 1024 x 151936 weights is 121.71 MiB, so q6_K
 *          stores 210 bytes per 256 weights).
 *
 * Block formats (byte-exact; little-endian; fp16 = IEEE binary16):
 *   Q4_0  (32 weights, 18 B)  [LCHW], [LC05 table], [KVQ], [BARE 3.2]
 *         [0:2]  fp16 scale d
 *         [2:18] 16 code bytes; byte t holds element t in its low nibble
 *                and element t+16 in its high nibble; code c in [0,15]
 *                stands for the integer c-8; weight = d*(c-8).
 *   Q8_0  (32 weights, 34 B)  [LC05 table] ("about 8.5 bits")
 *         [0:2]  fp16 scale d;  [2:34] int8 q[0..31];  weight = d*q.
 *   Q4_K  (256 weights = 8 sub-blocks of 32, 144 B)  [LC05 table]
 *         ("256-weight superblock, eight 32-element sub-blocks, sub-block
 *         scales themselves quantized to 6 bits"); the byte packing is this
 *         library's own and is not claimed compatible with GGUF's q4_K:
 *         [0:2]   fp16 super-scale d
 *         [2:4]   fp16 super-min  dmin
 *         [4:16]  96-bit little-endian integer V; 6-bit field f is
 *                 (V >> 6f) & 63; sc_j = field j, mn_j = field 8+j (j<8)
 *         [16:144] codes; sub-block j uses bytes 16+16j .. 16+16j+15 with
 *                 the Q4_0 nibble order; q in [0,15];
 *                 weight = (d*sc_j)*q - (dmin*mn_j).
 *   Q6_K  (256 weights = 16 sub-blocks of 16, 210 B)  [LC05 table] (the
 *         k-quant superblock, Q6_K its near-lossless member), [LC05 KV]
 *         (210 B). Sixteen 16-weight sub-blocks with int8 scales are the
 *         split that fills 210 bytes with 6-bit codes; the byte packing is
 *         this library's own, not GGUF's q6_K:
 *         [0:2]   fp16 super-scale d
 *         then for each group g = 0..7 of 32 weights (sub-blocks 2g, 2g+1),
 *         26 bytes at 2+26g:
 *           [+0], [+1]  int8 sc_2g, sc_2g+1
 *           [+2:+18]    byte t: low 4 bits of code 32g+t (low nibble) and
 *                       of code 32g+16+t (high nibble)
 *           [+18:+22]   little-endian word H0: bits 2w..2w+1 of its byte b
 *                       are the high 2 bits of code 32g+4w+b
 *           [+22:+26]   H1: the same for code 32g+16+4w+b
 *         code c in [0,63]; weight = (d*sc_j)*(c-32), j = element / 16.
 *
 * Matrix layout: a [rows][K] matrix is rows*(K/block_elems) blocks, row
 * after row, blocks running along K, no padding. Rows are therefore
 * qmat_row_bytes(fmt, K) bytes apart.
 *
 * Common contract for every entry point:
 *   - Pointers W, x, y, blocks, X_q8, Y are DEVICE pointers owned by the
 *     caller, each 16-byte aligned (QMAT_E_ALIGN otherwise). The library
 *     keeps no pointer after return and owns no device memory, except the
 *     static workspace of qmat_prefill_noalloc (below).
 *   - stream is a hipStream_t (NULL = the legacy default stream). The call
 *     returns once the work is enqueued; results are ready when the stream
 *     reaches that point.
 *   - Argument errors are detected on the host before anything is
 *     enqueued and are returned synchronously; a failed launch returns
 *     QMAT_E_HIP. Device faults surface at the caller's next
 *     synchronisation, as for any HIP kernel.
 *   - Inputs and outputs must not overlap. Identical inputs give
 *     bit-identical outputs (no atomics, fixed reduction order).
 *   - Limits: 0 <= rows, M, N <= 2^31-1; 0 <= K <= 2^31-1; K a multiple of
 *     qmat_block_elems(fmt); rows*row_bytes must fit in int64. A zero M or
 *     N (or rows, for quantize) enqueues nothing and dereferences no pointer.
 *     K == 0 is valid: quantize writes nothing, gemv
 *     and gemm write zeros (the empty sum).
 *   - Thread safe; no global mutable state apart from qmat_prefill_noalloc's
 *     per-device workspace (see there: its calls must not overlap).
 */
#ifndef QMAT_H
#define QMAT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qmat_fmt {
  QMAT_Q4_0 = 0,
  QMAT_Q8_0 = 1,
  QMAT_Q4_K = 2,
  QMAT_Q6_K = 3
} qmat_fmt;

typedef enum qmat_status {
  QMAT_OK = 0,
  QMAT_E_FMT = 1,   /* unknown format, or format not allowed here        */
  QMAT_E_SHAPE = 2, /* negative size, K not a multiple of the block, or
                       a size beyond the limits above                    */
  QMAT_E_NULL = 3,  /* a required pointer is NULL                         */
  QMAT_E_HIP = 4,   /* the HIP launch itself failed                       */
  QMAT_E_ALIGN = 5, /* a pointer is not 16-byte aligned                   */
  QMAT_E_SCRATCH = 6, /* qmat_prefill_noalloc: the activation workspace it
                        needs exceeds its static scratch                   */
  QMAT_E_WORKSPACE = 7 /* qmat_gemm_ws: workspace NULL or smaller than
                          qmat_gemm_workspace_bytes()                      */
} qmat_status;

/* Bytes of the static device workspace of qmat_prefill_noalloc (16 MiB):
 * room for the Q8_0 activations of N tokens of K elements while
 * N * K / 32 * 34 <= this, e.g. 1024 tokens at K = 14336. */
#define QMAT_NOALLOC_SCRATCH_BYTES (16u << 20)

/* Elements per block: 32 (Q4_0, Q8_0), 256 (Q4_K, Q6_K); 0 if unknown. */
int64_t qmat_block_elems(int fmt);

/* Bytes per block: 18 (Q4_0) [LCHW], 34 (Q8_0), 144 (Q4_K), 210 (Q6_K)
 * [LC05 KV]; 0 if unknown. */
int64_t qmat_block_bytes(int fmt);

/* Bytes of one packed row of K elements; -1 for an unknown fmt, a negative
 * K, a K that is not a multiple of the block, or a byte count beyond int64. */
int64_t qmat_row_bytes(int fmt, int64_t K);

/* Static English text for a status code (never NULL). */
const char *qmat_strerror(int status);

/*
 * qmat_quantize — round-to-nearest block quantization of an fp32 matrix.
 *   W:      fp32 [rows][K], row-major.
 *   blocks: output, rows*qmat_row_bytes(fmt,K) bytes in the layout above.
 *   Rules (per block, fp32 IEEE arithmetic, correctly rounded division,
 *   rnd = round half away from zero, fp16 = round to nearest even with
 *   subnormals, codes computed from the stored fp16 scale):
 *     Q4_0: d = amax/7; D = fp16(d); c = clamp(rnd(w/D),-8,7)+8 (8 if D==0)
 *           [LCHW] one fp16 scale per 32 weights; [KVQ] symmetric.
 *     Q8_0: d = amax/127; q = clamp(rnd(w/D),-127,127) (0 if D==0).
 *           With fmt = QMAT_Q8_0 this is also the activation quantizer
 *           whose output qmat_gemm consumes.
 *     Q4_K: per sub-block j: lo = min(0, min w), hi = max w,
 *           scale_j = (hi-lo)/15, off_j = -lo; d = max scale_j / 63,
 *           dmin = max off_j / 63 (both stored fp16); sc_j, mn_j =
 *           clamp(rnd(scale_j/D),0,63), clamp(rnd(off_j/Dmin),0,63);
 *           q = clamp(rnd((w + Dmin*mn_j)/(D*sc_j)),0,15) (0 if D*sc_j==0).
 *           [LC05 table] two-level scaling with 6-bit sub-block scales.
 *     Q6_K: per 16-weight sub-block j: s_j = amax_j/31; d = max s_j / 127
 *           (stored fp16); sc_j = clamp(rnd(s_j/D),0,127);
 *           c = clamp(rnd(w/(D*sc_j)),-32,31)+32 (32 if D*sc_j==0).
 *   Non-finite inputs or a scale above 65504 give unspecified bytes (never
 *   a fault).
 */
int qmat_quantize(int fmt, const float *W, void *blocks, int64_t rows,
                  int64_t K, void *stream);

/*
 * qmat_gemv — decode-time matrix-vector product (one token):
 *   y[m] = sum_k dequant(W)[m][k] * x[k],  m < M.
 *   [LC05 "带宽决定 Decode"]: every weight byte is read once per token, so
 *   this is bound by HBM bandwidth.
 *   blocks: W in fmt (Q4_0, Q8_0, Q4_K or Q6_K), M rows of K.
 *   x: fp32 [K]; y: fp32 [M], overwritten.
 *   Accuracy: relative L2 error against the exact (fp64) product of the
 *   dequantized weights with x is below 1e-3 for finite x; internally each
 *   32-element slice of x is scaled by a power of two and rounded to a
 *   20-bit integer (|X| < 2^19, relative step <= 2^-17.9 of the slice's
 *   largest element), the integer dot products with the codes are exact,
 *   and the per-block results are accumulated in fp32.
 *   Rows of 4096 to 16384 elements (and of 1024 to 4095 when M <= 8192)
 *   are computed by waves that wait, with a bounded number of polls, for
 *   activation records that other waves of their workgroup publish; a wave whose wait ran out (never expected: the
 *   records are always published) writes NaN to its rows rather than a
 *   value computed from incomplete records.
 */
int qmat_gemv(int fmt, const void *blocks, const float *x, float *y,
              int64_t M, int64_t K, void *stream);

/*
 * qmat_gemv_batch — many independent decode GEMVs in as few launches as
 *   possible: job i computes jobs[i].y = dequant(W_i) x_i with qmat_gemv's
 *   arithmetic and accuracy bound. Rows shorter than 8192 elements may go
 *   through a different work split than a single qmat_gemv call of the same
 *   job, so the fp32 partial sums can be added in another order and the
 *   last bits can differ from that call's; repeated batch calls give the
 *   same bits. [LC05 "带宽决定
 *   Decode"]: each weight byte is read once per token; a decode step runs
 *   many small GEMVs (a 0.6B model's layers are 1024 to 3072 wide), whose
 *   cost at one launch each is mostly the launch.
 *   jobs: HOST array of count descriptors, read during the call only.
 *   fmt applies to every job. Every job is checked as qmat_gemv checks its
 *   arguments, all of them before anything is enqueued; the first failure
 *   is returned. Jobs with M == 0 are skipped. Outputs must not overlap each
 *   other or any input.
 *   Jobs are grouped, up to 64 per launch, by the parity of their row
 *   stride (rows starting at 2 mod 4 or not), by kernel (rows of 8192 to
 *   16384 elements, or shorter) and by the shape of their workgroups (rows
 *   of at most 1024 elements, or the number of 2048-element strips a row
 *   spans), so a call makes at most a few launches per shape present. The launches are enqueued in order
 *   on stream; the host returns once they are enqueued.
 */
typedef struct qmat_gemv_job {
  const void *blocks; /* W: M rows of K in fmt */
  const float *x;     /* fp32 [K] */
  float *y;           /* fp32 [M], overwritten */
  int64_t M;
  int64_t K;
} qmat_gemv_job;

int qmat_gemv_batch(int fmt, const qmat_gemv_job *jobs, int64_t count, void *stream);

/*
 * qmat_gemm — prefill matrix product over N tokens:
 *   Y[n][m] = sum_k dequant(W)[m][k] * dequant(X_q8)[n][k].
 *   [LC05 "算力决定 Prefill"]: one weight read serves many tokens, so this
 *   is bound by the matrix cores (int8 MFMA over each 32-element block,
 *   then the two fp16 block scales applied in fp32).
 *   blocks: W in fmt (Q4_0, Q8_0, Q4_K or Q6_K), M rows of K.
 *   X_q8: Q8_0 blocks of the activations, N rows of K, exactly as
 *         qmat_quantize(QMAT_Q8_0, X, X_q8, N, K, stream) writes them.
 *   Y: fp32 [N][M] (token-major), overwritten.
 *   K is at most 2^24 here (QMAT_E_SHAPE above that): the kernel addresses
 *   a 128-row tile with 32-bit byte offsets.
 *   For a few tokens (a decode batch: up to 16, and up to 64 where a model
 *   of the two paths' times favours it, e.g. long rows) the weights are
 *   instead streamed once per 16 tokens and each weight block is applied
 *   to every token's block with int8 dot products; the
 *   arithmetic (exact block sums, the fp16 block scales applied in fp32;
 *   Q6_K: per 16-weight half) and the accuracy bound are the same.
 *   Accuracy: relative L2 error against the exact (fp64) product of the
 *   dequantized operands is below 2e-3; the per-block integer dot products
 *   are exact. Q4_K's min term (dmin*mn_j times the block sums of X_q8) is
 *   accumulated in fp32.
 */
int qmat_gemm(int fmt, const void *blocks, const void *X_q8, float *Y,
              int64_t M, int64_t K, int64_t N, void *stream);

/*
 * qmat_gemm_workspace_bytes — bytes of device workspace qmat_gemm_ws needs
 *   for this product: 0 when it runs as qmat_gemm does, else
 *   (splits - 1) * N * M * 4 (see qmat_gemm_ws). A function of the
 *   arguments alone. -1 for an unknown format or a shape qmat_gemm rejects.
 */
int64_t qmat_gemm_workspace_bytes(int fmt, int64_t M, int64_t K, int64_t N);

/*
 * qmat_gemm_ws — qmat_gemm with a caller workspace, which lets a product
 *   whose 128 x 64 output tiles are too few to occupy every compute unit
 *   (up to a few hundred tokens) also be divided along K. [LC05
 *   "算力决定 Prefill"] as for qmat_gemm: the same block products and
 *   scales; only the order in which block contributions are summed
 *   changes. The K blocks are cut into `splits` contiguous ranges (whole
 *   stages of 8 blocks), each range's partial product is computed as
 *   qmat_gemm computes the whole one, and the partial products are added
 *   in range order by a second kernel on the same stream.
 *   Arguments: as for qmat_gemm, plus
 *   workspace: device buffer of at least qmat_gemm_workspace_bytes(fmt, M,
 *     K, N) bytes, 16-byte aligned, owned by the caller, used only while
 *     the call's work runs on stream (its contents are not needed before
 *     and are garbage after); may be NULL when that size is 0.
 *   workspace_bytes: its size in bytes (>= 0).
 *   Results: deterministic, and identical to qmat_gemm's whenever the size
 *   is 0; otherwise within qmat_gemm's accuracy bound of them (they differ
 *   only in summation order).
 *   Errors: qmat_gemm's, then QMAT_E_SHAPE for workspace_bytes < 0,
 *   QMAT_E_WORKSPACE when a nonzero size is needed and workspace is NULL
 *   or workspace_bytes is smaller, QMAT_E_ALIGN for a misaligned workspace.
 *   Two calls that share a workspace must not overlap in time.
 */
int qmat_gemm_ws(int fmt, const void *blocks, const void *X_q8, float *Y,
                 int64_t M, int64_t K, int64_t N, void *workspace,
                 int64_t workspace_bytes, void *stream);

/*
 * qmat_prefill — the prefill product from fp32 activations in one call:
 *   the activations are quantized to Q8_0 into the caller's workspace, then
 *   multiplied as by qmat_gemm. [LC05 "算力决定 Prefill"] as for qmat_gemm;
 *   the activation rule is qmat_quantize's Q8_0 rule.
 *   blocks: W in fmt (Q4_0, Q8_0, Q4_K or Q6_K), M rows of K.
 *   X: fp32 [N][K] activations.
 *   xq: workspace of N * qmat_row_bytes(QMAT_Q8_0, K) bytes, owned by the
 *       caller; afterwards it holds exactly what
 *       qmat_quantize(QMAT_Q8_0, X, xq, N, K, stream) writes, so the same
 *       activations can be multiplied by further weight matrices with
 *       qmat_gemm.
 *   Y: fp32 [N][M] (token-major), overwritten.
 *   The two kernels are enqueued on stream in that order; Y is exactly
 *   qmat_gemm(fmt, blocks, xq, Y, M, K, N, stream)'s result. Shapes, the K
 *   limit and errors are qmat_gemm's; X and xq follow the same rules as
 *   the other buffers (non-NULL and 16-byte aligned when K > 0). X, xq and Y
 *   must not overlap. M == 0 or N == 0 enqueues nothing.
 */
int qmat_prefill(int fmt, const void *blocks, const float *X, void *xq, float *Y,
                 int64_t M, int64_t K, int64_t N, void *stream);

/*
 * qmat_prefill_noalloc — qmat_prefill for callers that cannot allocate
 *   device memory (code under HIP graph capture, tight serving loops,
 *   harnesses that forbid hipMalloc): the same product, with the Q8_0
 *   activation workspace taken from a static device array of the library
 *   (QMAT_NOALLOC_SCRATCH_BYTES, one per device, held until the process
 *   ends) instead of a caller buffer. No call allocates or frees memory.
 *   The workspace is looked up once per device (hipGetSymbolAddress, with
 *   that device current) on the first call made there; calls must run on a
 *   stream of the current device.
 *   blocks, X, Y, M, K, N: as for qmat_prefill; Y is exactly what
 *   qmat_prefill writes for the same inputs.
 *   Errors: qmat_prefill's, checked in the same order, then QMAT_E_SCRATCH
 *   when N * qmat_row_bytes(QMAT_Q8_0, K) > QMAT_NOALLOC_SCRATCH_BYTES (before
 *   the pointer checks and before anything is enqueued); QMAT_E_HIP if the
 *   workspace's address cannot be obtained.
 *   Every call on one device shares that device's workspace, which keeps the
 *   last call's activations (nothing in it needs to start at zero): calls
 *   whose work overlaps on one device — on two streams, or from two threads
 *   without ordering — race on it and give undefined results. Serialise them
 *   (one stream, or events), or use qmat_prefill with separate workspaces.
 */
int qmat_prefill_noalloc(int fmt, const void *blocks, const float *X, float *Y,
                         int64_t M, int64_t K, int64_t N, void *stream);

/* QMAT_NOALLOC_SCRATCH_BYTES, as a call (for bindings without the header). */
int64_t qmat_noalloc_scratch_bytes(void);

/*
 * qmat_kv_write — quantize new key or value rows into a KV cache.
 *   [KVQ] "量化 KV Cache 的一键配置方法": K and V rows are stored as q8_0 or
 *   q4_0 blocks. [KVQ] "kv-mean-center 进阶技巧": a fixed per-channel bias may
 *   be subtracted from K first; attention is unchanged (a query's scores all
 *   move by the same q·bias, and softmax ignores a constant per row) while
 *   the centred values quantize with less error.
 *   fmt:   QMAT_Q4_0 or QMAT_Q8_0 (others: QMAT_E_FMT).
 *   rows:  fp32 [n][dim], one new vector per token (dim = KV heads × head
 *          dimension), a multiple of 32.
 *   bias:  fp32 [dim] subtracted from every row (fp32, correctly rounded)
 *          before quantizing, or NULL.
 *   cache: cells rows of qmat_row_bytes(fmt, dim) bytes in the block layout
 *          above; rows cell0 .. cell0+n-1 are overwritten, every other byte is
 *          left as it was. Each written row holds exactly the bytes
 *          qmat_quantize(fmt, rows[i] - bias, ...) would write.
 *   Shapes: 0 <= n, cell0 and cell0 + n <= cells (QMAT_E_SHAPE otherwise).
 *   rows, bias (if given) and cache + cell0 * row_bytes must be 16-byte
 *   aligned (QMAT_E_ALIGN); any cell0 qualifies when dim is a multiple of 256.
 *   rows and bias must not overlap the cache.
 *   n == 0 or dim == 0 enqueues nothing.
 */
int qmat_kv_write(int fmt, const float *rows, const float *bias, void *cache,
                  int64_t cell0, int64_t n, int64_t cells, int64_t dim,
                  void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QMAT_H */
