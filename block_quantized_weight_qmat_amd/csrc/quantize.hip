// quantize.hip — fp32 -> Q4_0 / Q8_0 / Q4_K-style block quantizers (gfx950).
//
// Formats and rules: include/qmat.h. Sources: "05. llama.cpp：从 GGUF 文件到
// 本地推理服务", quant-type table in section "量化类型：Q4_K_M 到底是什么"
// (32-weight groups with one fp16 scale; 256-weight superblocks of eight
// 32-element sub-blocks with 6-bit sub-block scales); "llama.cpp 原理：如何在
// 普通硬件跑本地大模型", section "量化：内存真正去哪了" (Q4_0: 18 bytes per 32
// weights); lpnh.cn KV-cache article, paragraph "问题" (Q4_0 symmetric).
//
// Every step is IEEE fp32 with correctly rounded division (no fast-math, no
// contraction: this file is built with -ffp-contract=off), round half away
// from zero (roundf), and fp16 rounding to nearest even by v_cvt_f16_f32, so
// the bytes are identical to any other implementation of the same rules.
//
// Work split: 8 lanes own one 32-element block (4 consecutive floats each,
// one 16-byte load per lane, so a wave reads 1 KiB contiguously). The packed
// blocks of a workgroup are assembled in LDS and written out as 16-byte
// stores. Q4_K uses one wave per 256-element superblock.
#include "qmat_device.hpp"
#include "qmat_launch.hpp"

namespace qmat {
namespace {

constexpr int kQThreads = 256;
constexpr int kBlocksPerWG = kQThreads / 8;  // 32 blocks of 32 elements

__device__ __forceinline__ float clampf(float v, float lo, float hi) {
  return fminf(fmaxf(v, lo), hi);
}

// Copy `nbytes` (even) of LDS staging to global memory starting at a
// 16-byte aligned address: 16-byte stores, then 2-byte stores for the tail.
__device__ __forceinline__ void copy_out(const uint8_t* lds, uint8_t* dst, int nbytes) {
  const int n16 = nbytes >> 4;
  for (int i = threadIdx.x; i < n16; i += blockDim.x)
    reinterpret_cast<u32x4*>(dst)[i] = reinterpret_cast<const u32x4*>(lds)[i];
  const int tail = nbytes - (n16 << 4);
  for (int i = threadIdx.x; i < (tail >> 1); i += blockDim.x) {
    const int o = (n16 << 4) + 2 * i;
    *reinterpret_cast<uint16_t*>(dst + o) = *reinterpret_cast<const uint16_t*>(lds + o);
  }
}

// Q4_0 (kQ4 = true) or Q8_0 (false): one 32-element block per 8 lanes.
template <bool kQ4>
__global__ __launch_bounds__(kQThreads) void quantize_b32_kernel(
    const float* __restrict__ W, uint8_t* __restrict__ out, int64_t nblocks) {
  constexpr int kBB = kQ4 ? 18 : 34;
  constexpr float kQmax = kQ4 ? 7.0f : 127.0f;
  __shared__ __attribute__((aligned(16))) uint8_t stage[kBlocksPerWG * kBB];
  uint16_t* stage16 = reinterpret_cast<uint16_t*>(stage);

  const int tid = threadIdx.x;
  const int lb = tid >> 3;  // block within the workgroup
  const int j = tid & 7;    // this lane holds elements 4j..4j+3
  const int64_t nchunks = (nblocks + kBlocksPerWG - 1) / kBlocksPerWG;

  for (int64_t chunk = blockIdx.x; chunk < nchunks; chunk += gridDim.x) {
    const int64_t g = chunk * kBlocksPerWG + lb;
    const bool valid = g < nblocks;
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    if (valid) v = *reinterpret_cast<const f32x4*>(W + g * 32 + 4 * j);

    // amax over the block (|x| >= +0, so max order does not matter)
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    a = fmaxf(a, shfl_xor_f(a, 1));
    a = fmaxf(a, shfl_xor_f(a, 2));
    a = fmaxf(a, shfl_xor_f(a, 4));

    const float d = a / kQmax;
    const uint32_t h = f32_to_f16_bits(d);
    const float D = f16_bits_to_f32(h);

    uint32_t packed = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float t = v[k];
      int q = 0;
      if (D != 0.0f) q = (int)clampf(roundf(t / D), kQ4 ? -8.0f : -127.0f, kQ4 ? 7.0f : 127.0f);
      const uint32_t c = kQ4 ? (uint32_t)(q + 8) : ((uint32_t)q & 0xFFu);
      packed |= c << (8 * k);
    }

    uint8_t* blk = stage + lb * kBB;
    (void)blk;
    if (kQ4) {
      // byte t of the code area: element t (low nibble) | element t+16 (high)
      const uint32_t partner = shfl_xor_u(packed, 4);
      if (j < 4) {
        const uint32_t w = packed | (partner << 4);
        stage16[(lb * kBB) / 2 + 1 + 2 * j] = (uint16_t)(w & 0xFFFFu);
        stage16[(lb * kBB) / 2 + 2 + 2 * j] = (uint16_t)(w >> 16);
      }
    } else {
      stage16[(lb * kBB) / 2 + 1 + 2 * j] = (uint16_t)(packed & 0xFFFFu);
      stage16[(lb * kBB) / 2 + 2 + 2 * j] = (uint16_t)(packed >> 16);
    }
    if (j == 0) stage16[(lb * kBB) / 2] = (uint16_t)h;
    __syncthreads();

    const int64_t remaining = nblocks - chunk * kBlocksPerWG;
    const int nb = remaining < kBlocksPerWG ? (int)remaining : kBlocksPerWG;
    copy_out(stage, out + chunk * kBlocksPerWG * kBB, nb * kBB);
    __syncthreads();
  }
}

// Q4_K-style: one wave per 256-element superblock, 4 superblocks per
// workgroup. Lane l holds elements 4l..4l+3; sub-block j = lanes 8j..8j+7.
__global__ __launch_bounds__(kQThreads) void quantize_q4k_kernel(
    const float* __restrict__ W, uint8_t* __restrict__ out, int64_t nsuper) {
  constexpr int kSB = 144;
  constexpr int kSuperPerWG = kQThreads / kWave;
  __shared__ __attribute__((aligned(16))) uint8_t stage[kSuperPerWG * kSB];
  uint32_t* stage32 = reinterpret_cast<uint32_t*>(stage);

  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int lane = tid & 63;
  const int sub = lane >> 3;  // sub-block
  const int jl = lane & 7;
  const int64_t nchunks = (nsuper + kSuperPerWG - 1) / kSuperPerWG;

  for (int64_t chunk = blockIdx.x; chunk < nchunks; chunk += gridDim.x) {
    const int64_t s = chunk * kSuperPerWG + wv;
    const bool valid = s < nsuper;
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    if (valid) v = *reinterpret_cast<const f32x4*>(W + s * 256 + 4 * lane);

    // 1. sub-block min and max (comparison order is irrelevant: the values
    //    and the derived bytes do not depend on which zero sign wins)
    float mn = fminf(fminf(v.x, v.y), fminf(v.z, v.w));
    float mx = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
      mn = fminf(mn, shfl_xor_f(mn, m));
      mx = fmaxf(mx, shfl_xor_f(mx, m));
    }
    const float lo = mn < 0.0f ? mn : 0.0f;
    const float hi = mx;
    // 2. sub-block scale and offset
    const float scale = (hi - lo) / 15.0f;
    const float off = -lo;
    // 3. super-scale and super-min: max over sub-blocks, starting from +0
    float smax = scale > 0.0f ? scale : 0.0f;
    float omax = off > 0.0f ? off : 0.0f;
#pragma unroll
    for (int m = 8; m < 64; m <<= 1) {
      const float so = shfl_xor_f(smax, m), oo = shfl_xor_f(omax, m);
      smax = so > smax ? so : smax;
      omax = oo > omax ? oo : omax;
    }
    const float d = smax / 63.0f, dmin = omax / 63.0f;
    const uint32_t hd = f32_to_f16_bits(d), hm = f32_to_f16_bits(dmin);
    const float D = f16_bits_to_f32(hd), Dm = f16_bits_to_f32(hm);
    // 4. 6-bit sub-block scale and min
    const int sc = (D == 0.0f) ? 0 : (int)clampf(roundf(scale / D), 0.0f, 63.0f);
    const int mq = (Dm == 0.0f) ? 0 : (int)clampf(roundf(off / Dm), 0.0f, 63.0f);
    // 5. exact effective scale and offset
    const float S = D * (float)sc;
    const float O = Dm * (float)mq;
    // 6. 4-bit codes
    uint32_t packed = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      int q = 0;
      if (S != 0.0f) q = (int)clampf(roundf((v[k] + O) / S), 0.0f, 15.0f);
      packed |= (uint32_t)q << (8 * k);
    }
    const uint32_t partner = shfl_xor_u(packed, 4);
    uint8_t* blk = stage + wv * kSB;
    if (jl < 4)
      reinterpret_cast<uint32_t*>(blk + 16 + 16 * sub)[jl] = packed | (partner << 4);

    // 96-bit field word: sc at bit 6*sub, min at bit 48 + 6*sub
    uint32_t f0 = 0, f1 = 0, f2 = 0;
    if (jl == 0) {
      const int ps = 6 * sub, pm = 48 + 6 * sub;
      uint32_t fw[3] = {0, 0, 0};
      fw[ps >> 5] |= (uint32_t)sc << (ps & 31);
      if ((ps & 31) > 26) fw[(ps >> 5) + 1] |= (uint32_t)sc >> (32 - (ps & 31));
      fw[pm >> 5] |= (uint32_t)mq << (pm & 31);
      if ((pm & 31) > 26) fw[(pm >> 5) + 1] |= (uint32_t)mq >> (32 - (pm & 31));
      f0 = fw[0];
      f1 = fw[1];
      f2 = fw[2];
    }
#pragma unroll
    for (int m = 8; m < 64; m <<= 1) {
      f0 |= shfl_xor_u(f0, m);
      f1 |= shfl_xor_u(f1, m);
      f2 |= shfl_xor_u(f2, m);
    }
    if (lane == 0) {
      uint32_t* h32 = reinterpret_cast<uint32_t*>(blk);
      h32[0] = hd | (hm << 16);
      h32[1] = f0;
      h32[2] = f1;
      h32[3] = f2;
    }
    (void)stage32;
    __syncthreads();
    const int64_t remaining = nsuper - chunk * kSuperPerWG;
    const int ns = remaining < kSuperPerWG ? (int)remaining : kSuperPerWG;
    copy_out(stage, out + chunk * kSuperPerWG * kSB, ns * kSB);
    __syncthreads();
  }
}

constexpr int64_t kMaxGrid = 1 << 24;

int64_t grid_for(int64_t chunks) { return chunks < kMaxGrid ? chunks : kMaxGrid; }

}  // namespace

hipError_t launch_quantize(int fmt, const float* W, void* blocks, int64_t rows, int64_t K,
                           hipStream_t stream) {
  uint8_t* out = static_cast<uint8_t*>(blocks);
  if (fmt == kFmtQ4_K) {
    const int64_t nsuper = rows * (K / 256);
    const int64_t chunks = (nsuper + 3) / 4;
    if (chunks == 0) return hipSuccess;
    hipLaunchKernelGGL(quantize_q4k_kernel, dim3((unsigned)grid_for(chunks)), dim3(kQThreads), 0,
                       stream, W, out, nsuper);
  } else {
    const int64_t nb = rows * (K / 32);
    const int64_t chunks = (nb + kBlocksPerWG - 1) / kBlocksPerWG;
    if (chunks == 0) return hipSuccess;
    if (fmt == kFmtQ4_0)
      hipLaunchKernelGGL(quantize_b32_kernel<true>, dim3((unsigned)grid_for(chunks)),
                         dim3(kQThreads), 0, stream, W, out, nb);
    else
      hipLaunchKernelGGL(quantize_b32_kernel<false>, dim3((unsigned)grid_for(chunks)),
                         dim3(kQThreads), 0, stream, W, out, nb);
  }
  return hipGetLastError();
}

}  // namespace qmat
