// micro.hip — measured peaks of the GPU, for the rooflines the benchmark
// reports beside the nominal ones: HBM read bandwidth, the dense int8 MFMA
// rate, the non-packed fp32 FMA rate, and the fp32 FMA rate that a wave keeps
// while the same SIMD runs int8 MFMAs (the mix of the GEMM's scale step).
//
// Built into its own library (libqmat_micro.so); nothing in the product
// library calls it. Every kernel runs a fixed number of iterations and
// writes one value per lane, so that no work is dead code.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // 16-byte loads in flight per lane and iteration

// Reads n16 16-byte words once, coalesced, kUnroll loads in flight per lane.
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ src,
                                                        int64_t n16, uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= src[i];
  out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// Four independent chains of v_mfma_i32_32x32x32_i8 per wave.
__global__ __launch_bounds__(kThreads) void mfma_kernel(int iters, int32_t* __restrict__ out) {
  const int t = (int)threadIdx.x;
  const i32x4 a = {t, t + 1, t + 2, t + 3}, b = {3 * t, 1, -t, 7};
  i32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
  }
  uint32_t s = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) s += (uint32_t)(c0[k] ^ c1[k] ^ c2[k] ^ c3[k]);
  out[(int64_t)blockIdx.x * kThreads + t] = (int32_t)s;
}

// kChains independent fp32 FMA chains per lane (plain, non-packed FMAs).
// m and c come in as arguments, so that the FMAs take them from scalar
// registers rather than as 32-bit literals; the loop is unrolled so that
// its scalar bookkeeping is a small share of the issue slots.
constexpr int kChains = 8;
__global__ __launch_bounds__(kThreads) void fma_kernel(int iters, float m, float c,
                                                       float* __restrict__ out) {
  float x[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) x[k] = 1e-3f * (float)(threadIdx.x + k);
#pragma unroll 4
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kChains; ++k) x[k] = fmaf(x[k], m, c);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < kChains; ++k) s += x[k];
  out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

// Half of the waves run int8 MFMA chains, the other half fp32 FMA chains, so
// that every SIMD holds both; the FMA waves' rate shows what the VALU keeps
// while the matrix core is busy.
__global__ __launch_bounds__(2 * kThreads) void mix_kernel(int iters, float m, float c,
                                                           float* __restrict__ out) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t o = (int64_t)blockIdx.x * (2 * kThreads) + threadIdx.x;
  if ((wave & 4) == 0) {
    const int t = (int)threadIdx.x;
    const i32x4 a = {t, t + 1, t + 2, t + 3}, b = {3 * t, 1, -t, 7};
    i32x16 c0 = {}, c1 = {};
    // two MFMAs (64 matrix-core cycles) per 8 iterations of the FMA waves
    // (64 FMAs, 256 cycles at one per 4): the matrix core busy a quarter of
    // the time, as in the GEMM (2 MFMAs and 64 FMAs per block and wave tile)
    for (int i = 0; i < iters / 8; ++i) {
      c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
    }
    uint32_t s = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) s += (uint32_t)(c0[k] ^ c1[k]);
    out[o] = (float)s;
  } else {
    float x[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k) x[k] = 1e-3f * (float)(threadIdx.x + k);
#pragma unroll 4
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int k = 0; k < kChains; ++k) x[k] = fmaf(x[k], m, c);
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < kChains; ++k) s += x[k];
    out[o] = s;
  }
}

}  // namespace

// Each entry point enqueues one launch on stream and returns the launch
// status (0 = hipSuccess; 1 = a bad argument, nothing enqueued). out must
// hold grid * 256 four-byte values (qmat_micro_mix: grid * 512).
extern "C" {

// Read bytes (a multiple of 16, 16-byte aligned) of buf once.
int qmat_micro_read(const void* buf, int64_t bytes, void* out, int grid, void* stream) {
  if (buf == nullptr || out == nullptr || bytes < 16 || (bytes & 15) != 0 || grid < 1) return 1;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf), bytes / 16,
                     static_cast<uint32_t*>(out));
  return (int)hipGetLastError();
}

// iters * 4 int8 MFMAs (2 * 32 * 32 * 32 operations each) per wave.
int qmat_micro_mfma_i8(int iters, void* out, int grid, void* stream) {
  if (out == nullptr || iters < 1 || grid < 1) return 1;
  hipLaunchKernelGGL(mfma_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), iters, static_cast<int32_t*>(out));
  return (int)hipGetLastError();
}

// iters * 8 fp32 FMAs (2 flops each) per lane.
int qmat_micro_fma_f32(int iters, void* out, int grid, void* stream) {
  if (out == nullptr || iters < 1 || grid < 1) return 1;
  hipLaunchKernelGGL(fma_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), iters, 0.999999f, 1e-7f,
                     static_cast<float*>(out));
  return (int)hipGetLastError();
}

// Waves 0-3 of each workgroup: iters / 8 * 2 int8 MFMAs; waves 4-7: iters
// * 8 fp32 FMAs per lane. Launch with 512 threads per workgroup.
int qmat_micro_mix(int iters, void* out, int grid, void* stream) {
  if (out == nullptr || iters < 16 || grid < 1) return 1;
  hipLaunchKernelGGL(mix_kernel, dim3((unsigned)grid), dim3(2 * kThreads), 0,
                     static_cast<hipStream_t>(stream), iters, 0.999999f, 1e-7f,
                     static_cast<float*>(out));
  return (int)hipGetLastError();
}

}  // extern "C"
