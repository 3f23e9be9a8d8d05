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
// Work split: one lane per 32-element block (Q4_K-style: per sub-block), so
// the per-block steps run once; a wave's 64 blocks are staged through LDS.
#include "qmat_device.hpp"
#include "qmat_launch.hpp"

namespace qmat {
namespace {

constexpr int kQThreads = 256;

__device__ __forceinline__ float clampf(float v, float lo, float hi) {
  return fminf(fmaxf(v, lo), hi);
}

// Staging of 64 consecutive 32-element blocks (8 KB) of one wave, copied
// from memory straight into LDS (1 KB per instruction, 16 bytes per lane).
// Part k (elements 4k..4k+3) of block b sits in column (k + b / 2) mod 8 of
// row b, so the 16 lanes of an LDS access phase hit 16 different 16-byte bank
// groups when lane b reads its block back.

__device__ __forceinline__ void stage_blocks(const float* __restrict__ src, int nblk, float* lds,
                                             int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int b = 8 * i + (lane >> 3);  // block filled by this lane's slot
    const int k = ((lane & 7) - (b >> 1)) & 7;
    if (8 * i < nblk && b < nblk)
      __builtin_amdgcn_global_load_lds(src + 32 * b + 4 * k, (lds_ptr_t)(lds + 256 * i), 16, 0,
                                       0);
  }
  // the compiler does not track direct-to-LDS loads: wait for all of them
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), other counters free
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void read_block(const float* lds, int lane, bool valid,
                                           float (&v)[32]) {
  const float* row = lds + 32 * lane;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(row + 4 * ((k + (lane >> 1)) & 7));
    v[4 * k + 0] = valid ? t.x : 0.0f;
    v[4 * k + 1] = valid ? t.y : 0.0f;
    v[4 * k + 2] = valid ? t.z : 0.0f;
    v[4 * k + 3] = valid ? t.w : 0.0f;
  }
}

// a / b correctly rounded, for a divisor shared by many quotients: with
// y = 1/b correctly rounded (one IEEE division per block), q0 = a * y and
// the residual a - q0 * b exact in one fma, q0 + residual * y rounded once
// is the correctly rounded quotient whenever it can round to a code. Checked
// against IEEE division on the CPU (tests/shared_divisor_check.c) over the
// fp16 divisor range, quotients within +-135 (half-integer neighbourhoods
// included) and random operands: only subnormal numerators differ, and
// those round to code 0 either way.
__device__ __forceinline__ float div_shared(float a, float b, float y) {
  const float q0 = a * y;
  return fmaf(fmaf(-q0, b, a), y, q0);
}

// Q4_0 (kQ4 = true) or Q8_0 (false): one lane per 32-element block, 64
// blocks per wave. The packed blocks of a wave are assembled in LDS and
// written out with 16-byte stores. With a bias (the KV-cache write), element
// e of block g is x - bias[32 (g % nb_row) + e] (fp32) before quantizing.
// Waves share nothing, so the workgroup size (kThreads) only sets how the
// blocks spread over the CUs. kBias compiles the bias in (the KV-cache
// write); the weight quantizer keeps its registers free of it.
template <bool kQ4, int kThreads, bool kBias>
__global__ __launch_bounds__(kThreads) void quantize_b32_kernel(
    const float* __restrict__ W, uint8_t* __restrict__ out, int64_t nblocks,
    const float* __restrict__ bias, int64_t nb_row) {
  constexpr int kBB = kQ4 ? 18 : 34;
  constexpr float kQmax = kQ4 ? 7.0f : 127.0f;
  constexpr int kWaves = kThreads / kWave;
  __shared__ __attribute__((aligned(16))) float xs[kWaves][kWave * 32];
  __shared__ __attribute__((aligned(16))) uint8_t ob[kWaves][kWave * kBB];

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  constexpr int kPerWG = kWaves * kWave;
  const int64_t nchunks = (nblocks + kPerWG - 1) / kPerWG;

  for (int64_t chunk = blockIdx.x; chunk < nchunks; chunk += gridDim.x) {
    const int64_t g0 = chunk * kPerWG + (int64_t)wv * kWave;  // first block of this wave
    const int64_t left = nblocks - g0;
    const int nblk = left <= 0 ? 0 : (left < kWave ? (int)left : kWave);
    const bool valid = lane < nblk;
    // the bias loads go out before the staging wait, so both overlap
    f32x4 bb[8];
    const bool biased = kBias && valid;
    if (biased) {
      // block index within its row; 32-bit division whenever the counts fit
      const int64_t g = g0 + lane;
      const int64_t c = nblocks <= 0xFFFFFFFFLL ? (int64_t)((uint32_t)g % (uint32_t)nb_row)
                                                : g % nb_row;
      const f32x4* bp = reinterpret_cast<const f32x4*>(bias + c * 32);
#pragma unroll
      for (int k = 0; k < 8; ++k) bb[k] = bp[k];
    }
    stage_blocks(W + g0 * 32, nblk, xs[wv], lane);
    float v[32];
    read_block(xs[wv], lane, valid, v);
    if (biased) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        v[4 * k + 0] -= bb[k].x;
        v[4 * k + 1] -= bb[k].y;
        v[4 * k + 2] -= bb[k].z;
        v[4 * k + 3] -= bb[k].w;
      }
    }

    // amax over the block (|x| >= +0, so the max order does not matter)
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) a = fmaxf(a, fabsf(v[e]));
    const float d = a / kQmax;
    const uint32_t h = f32_to_f16_bits(d);
    const float D = f16_bits_to_f32(h);

    // codes q = clamp(round(x / D)); Q4_0 stores q + 8, element t in the low
    // nibble of code byte t and element t + 16 in its high nibble
    uint32_t w[kQ4 ? 4 : 8];
#pragma unroll
    for (int i = 0; i < (kQ4 ? 4 : 8); ++i) w[i] = kQ4 ? 0x88888888u : 0u;
    if (D != 0.0f) {
      const float y = 1.0f / D;
#pragma unroll
      for (int i = 0; i < (kQ4 ? 4 : 8); ++i) w[i] = 0u;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int q =
            (int)clampf(roundf(div_shared(v[e], D, y)), kQ4 ? -8.0f : -127.0f, kQ4 ? 7.0f : 127.0f);
        if (kQ4)
          w[(e & 15) >> 2] |= (uint32_t)(q + 8) << (8 * (e & 3) + (e >= 16 ? 4 : 0));
        else
          w[e >> 2] |= ((uint32_t)q & 0xFFu) << (8 * (e & 3));
      }
    }

    // the block at byte 18 * lane (34 * lane) of the wave's output: written
    // as 4-byte words where aligned, 2-byte pieces at the ends
    uint8_t* o = ob[wv] + kBB * lane;
    if (((kBB * lane) & 2) == 0) {
      // scale and the first two code bytes share a word
      reinterpret_cast<uint32_t*>(o)[0] = h | (w[0] << 16);
#pragma unroll
      for (int i = 1; i < (kQ4 ? 4 : 8); ++i)
        reinterpret_cast<uint32_t*>(o)[i] = __builtin_amdgcn_alignbyte(w[i], w[i - 1], 2);
      reinterpret_cast<uint16_t*>(o)[(kBB - 2) / 2] = (uint16_t)(w[(kQ4 ? 4 : 8) - 1] >> 16);
    } else {
      reinterpret_cast<uint16_t*>(o)[0] = (uint16_t)h;
#pragma unroll
      for (int i = 0; i < (kQ4 ? 4 : 8); ++i) reinterpret_cast<uint32_t*>(o + 2)[i] = w[i];
    }
    // the wave's blocks are contiguous in memory and start 16-byte aligned
    // (64 * 18 and 64 * 34 are multiples of 16)
    const int nbytes = nblk * kBB;
    uint8_t* dst = out + g0 * kBB;
    for (int i = lane; i < (nbytes >> 4); i += kWave)
      reinterpret_cast<u32x4*>(dst)[i] = reinterpret_cast<const u32x4*>(ob[wv])[i];
    const int t0 = nbytes & ~15;
    for (int i = t0 + 2 * lane; i < nbytes; i += 2 * kWave)
      *reinterpret_cast<uint16_t*>(dst + i) = *reinterpret_cast<const uint16_t*>(ob[wv] + i);
  }
}

// Q4_K-style: one lane per 32-element sub-block, so a wave quantizes 8
// superblocks and the per-sub-block work (range, scale, 6-bit codes) is done
// once. A wave copies its 8 superblocks (8 KB) from memory straight into its
// own LDS area (1 KB per instruction, 16 bytes per lane), then each lane reads
// its sub-block back. Part k (elements 4k..4k+3) of sub-block b sits in
// column (k + b / 2) mod 8 of row b, so the 16 lanes of an LDS access phase
// hit 16 different 16-byte bank groups.
constexpr int kQkWaves = kQThreads / kWave;
constexpr int kQkSuperPerWave = 8;

// max / or over the 8 lanes of a superblock (xor 1, 2, 4 within 32 lanes)
template <int kXor>
__device__ __forceinline__ uint32_t swz_xor(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (kXor << 10));
}

__device__ __forceinline__ float max8_from0(float v) {
  // the superblock maxima start from +0 and only see values >= +0
  float o = __builtin_bit_cast(float, swz_xor<1>(__builtin_bit_cast(uint32_t, v)));
  v = o > v ? o : v;
  o = __builtin_bit_cast(float, swz_xor<2>(__builtin_bit_cast(uint32_t, v)));
  v = o > v ? o : v;
  o = __builtin_bit_cast(float, swz_xor<4>(__builtin_bit_cast(uint32_t, v)));
  return o > v ? o : v;
}

__device__ __forceinline__ uint32_t or8(uint32_t v) {
  v |= swz_xor<1>(v);
  v |= swz_xor<2>(v);
  return v | swz_xor<4>(v);
}

__global__ __launch_bounds__(kQThreads) void quantize_q4k_kernel(
    const float* __restrict__ W, uint8_t* __restrict__ out, int64_t nsuper) {
  constexpr int kSB = 144;
  __shared__ __attribute__((aligned(16))) float xs[kQkWaves][kQkSuperPerWave * 256];

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int sub = lane & 7;  // sub-block within the superblock
  constexpr int kPerWG = kQkWaves * kQkSuperPerWave;
  const int64_t nchunks = (nsuper + kPerWG - 1) / kPerWG;
  float* mine = xs[wv];

  for (int64_t chunk = blockIdx.x; chunk < nchunks; chunk += gridDim.x) {
    const int64_t s0 = chunk * kPerWG + (int64_t)wv * kQkSuperPerWave;
    const int64_t left = nsuper - s0;
    const int nsb = left <= 0 ? 0 : (left < kQkSuperPerWave ? (int)left : kQkSuperPerWave);

    // 8 superblocks = 64 sub-blocks, staged like 64 blocks
    stage_blocks(W + s0 * 256, 8 * nsb, mine, lane);

    const bool valid = (lane >> 3) < nsb;
    float v[32];
    read_block(mine, lane, valid, v);

    // 1. sub-block min and max (the derived bytes do not depend on which
    //    zero sign a comparison keeps)
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int e = 1; e < 32; ++e) {
      mn = fminf(mn, v[e]);
      mx = fmaxf(mx, v[e]);
    }
    const float lo = mn < 0.0f ? mn : 0.0f;
    const float hi = mx;
    // 2. sub-block scale and offset
    const float scale = (hi - lo) / 15.0f;
    const float off = -lo;
    // 3. super-scale and super-min: max over the superblock's sub-blocks,
    //    starting from +0
    const float smax = max8_from0(scale > 0.0f ? scale : 0.0f);
    const float omax = max8_from0(off > 0.0f ? off : 0.0f);
    const float d = smax / 63.0f, dmin = omax / 63.0f;
    const uint32_t hd = f32_to_f16_bits(d), hm = f32_to_f16_bits(dmin);
    const float D = f16_bits_to_f32(hd), Dm = f16_bits_to_f32(hm);
    // 4. 6-bit sub-block scale and min
    const int sc = (D == 0.0f) ? 0 : (int)clampf(roundf(scale / D), 0.0f, 63.0f);
    const int mq = (Dm == 0.0f) ? 0 : (int)clampf(roundf(off / Dm), 0.0f, 63.0f);
    // 5. exact effective scale and offset
    const float S = D * (float)sc;
    const float O = Dm * (float)mq;
    // 6. 4-bit codes q = clamp(round((v + O) / S), 0, 15), the 32
    //    quotients sharing the divisor (div_shared)
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (S != 0.0f) {
      const float y = 1.0f / S;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const uint32_t c = (uint32_t)(int)clampf(roundf(div_shared(v[e] + O, S, y)), 0.0f, 15.0f);
        // byte t of the code area: element t (low nibble) | t + 16 (high)
        w[(e & 15) >> 2] |= c << (8 * (e & 3) + (e >= 16 ? 4 : 0));
      }
    }
    // 96-bit field word: sc at bit 6 * sub, min at bit 48 + 6 * sub
    uint32_t fw[3] = {0u, 0u, 0u};
    {
      const int ps = 6 * sub, pm = 48 + 6 * sub;
      fw[ps >> 5] |= (uint32_t)sc << (ps & 31);
      if ((ps & 31) > 26) fw[(ps >> 5) + 1] |= (uint32_t)sc >> (32 - (ps & 31));
      fw[pm >> 5] |= (uint32_t)mq << (pm & 31);
      if ((pm & 31) > 26 && (pm >> 5) + 1 < 3) fw[(pm >> 5) + 1] |= (uint32_t)mq >> (32 - (pm & 31));
    }
    const uint32_t f0 = or8(fw[0]), f1 = or8(fw[1]), f2 = or8(fw[2]);
    if (valid) {
      uint8_t* blk = out + (s0 + (lane >> 3)) * kSB;
      reinterpret_cast<u32x4*>(blk + 16 + 16 * sub)[0] = u32x4{w[0], w[1], w[2], w[3]};
      if (sub == 0) reinterpret_cast<u32x4*>(blk)[0] = u32x4{hd | (hm << 16), f0, f1, f2};
    }
  }
}

// Q6_K-style: one lane per 32-weight group (two 16-weight sub-blocks), so
// 8 lanes per superblock and 8 superblocks per wave, staged like the Q4_K
// kernel. Steps as the format's rule: s_j = amax_j / 31; d = max s_j / 127
// (fp16); sc_j = clamp(rnd(s_j / D), 0, 127); S_j = D sc_j; codes
// clamp(rnd(x / S_j), -32, 31) + 32. A wave's 8 packed superblocks (1680
// bytes, 16-byte aligned) are assembled in LDS with 2-byte writes (group
// starts are even) and written out with 16-byte stores.
__global__ __launch_bounds__(kQThreads) void quantize_q6k_kernel(
    const float* __restrict__ W, uint8_t* __restrict__ out, int64_t nsuper) {
  constexpr int kSB = 210;
  __shared__ __attribute__((aligned(16))) float xs[kQkWaves][kQkSuperPerWave * 256];
  __shared__ __attribute__((aligned(16))) uint8_t ob[kQkWaves][kQkSuperPerWave * kSB];

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int g = lane & 7;  // group within the superblock
  constexpr int kPerWG = kQkWaves * kQkSuperPerWave;
  const int64_t nchunks = (nsuper + kPerWG - 1) / kPerWG;
  float* mine = xs[wv];

  for (int64_t chunk = blockIdx.x; chunk < nchunks; chunk += gridDim.x) {
    const int64_t s0 = chunk * kPerWG + (int64_t)wv * kQkSuperPerWave;
    const int64_t left = nsuper - s0;
    const int nsb = left <= 0 ? 0 : (left < kQkSuperPerWave ? (int)left : kQkSuperPerWave);

    // 8 superblocks = 64 groups of 32, staged like 64 blocks
    stage_blocks(W + s0 * 256, 8 * nsb, mine, lane);
    const bool valid = (lane >> 3) < nsb;
    float v[32];
    read_block(mine, lane, valid, v);

    // 1. the two sub-blocks' scales (|x| >= +0: max order does not matter)
    float aa = 0.0f, ab = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      aa = fmaxf(aa, fabsf(v[e]));
      ab = fmaxf(ab, fabsf(v[16 + e]));
    }
    const float sa = aa / 31.0f, sb = ab / 31.0f;
    // 2. super-scale: max over the superblock's 16 sub-blocks, from +0
    const float d = max8_from0(sa > sb ? sa : sb) / 127.0f;
    const uint32_t hd = f32_to_f16_bits(d);
    const float D = f16_bits_to_f32(hd);
    // 3. int8 sub-block scales; 4. their exact values
    const int sca = (D == 0.0f) ? 0 : (int)clampf(roundf(sa / D), 0.0f, 127.0f);
    const int scb = (D == 0.0f) ? 0 : (int)clampf(roundf(sb / D), 0.0f, 127.0f);
    const float Sa = D * (float)sca, Sb = D * (float)scb;
    // 5. codes c = q + 32 (32 where the scale is 0); code 32g+t's low 4
    //    bits go to the low nibble of byte t, code 32g+16+t's to its high
    //    nibble; the high 2 bits of code 32g+4w+b (32g+16+4w+b) go to bits
    //    2w..2w+1 of byte b of H0 (H1)
    const float ya = Sa != 0.0f ? 1.0f / Sa : 0.0f, yb = Sb != 0.0f ? 1.0f / Sb : 0.0f;
    uint32_t nib[4] = {0u, 0u, 0u, 0u}, h0 = 0u, h1 = 0u;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int qa = Sa != 0.0f ? (int)clampf(roundf(div_shared(v[e], Sa, ya)), -32.0f, 31.0f) : 0;
      const int qb =
          Sb != 0.0f ? (int)clampf(roundf(div_shared(v[16 + e], Sb, yb)), -32.0f, 31.0f) : 0;
      const uint32_t ca = (uint32_t)(qa + 32), cb = (uint32_t)(qb + 32);
      nib[e >> 2] |= ((ca & 15u) << (8 * (e & 3))) | ((cb & 15u) << (8 * (e & 3) + 4));
      h0 |= (ca >> 4) << (8 * (e & 3) + 2 * (e >> 2));
      h1 |= (cb >> 4) << (8 * (e & 3) + 2 * (e >> 2));
    }

    // the group's 26 bytes at superblock offset 2 + 26 g, then d at 0
    uint16_t* o = reinterpret_cast<uint16_t*>(ob[wv] + (lane >> 3) * kSB + 2 + 26 * g);
    o[0] = (uint16_t)((sca & 0xFF) | ((scb & 0xFF) << 8));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[1 + 2 * i] = (uint16_t)nib[i];
      o[2 + 2 * i] = (uint16_t)(nib[i] >> 16);
    }
    o[9] = (uint16_t)h0;
    o[10] = (uint16_t)(h0 >> 16);
    o[11] = (uint16_t)h1;
    o[12] = (uint16_t)(h1 >> 16);
    if (g == 0) reinterpret_cast<uint16_t*>(ob[wv] + (lane >> 3) * kSB)[0] = (uint16_t)hd;

    // the wave's superblocks are contiguous and start 16-byte aligned
    // (s0 is a multiple of 8 and 8 * 210 = 1680 of 16)
    const int nbytes = nsb * kSB;
    uint8_t* dst = out + s0 * kSB;
    for (int i = lane; i < (nbytes >> 4); i += kWave)
      reinterpret_cast<u32x4*>(dst)[i] = reinterpret_cast<const u32x4*>(ob[wv])[i];
    const int t0 = nbytes & ~15;
    for (int i = t0 + 2 * lane; i < nbytes; i += 2 * kWave)
      *reinterpret_cast<uint16_t*>(dst + i) = *reinterpret_cast<const uint16_t*>(ob[wv] + i);
  }
}

constexpr int64_t kMaxGrid = 1 << 24;

int64_t grid_for(int64_t chunks) { return chunks < kMaxGrid ? chunks : kMaxGrid; }

// nb Q4_0 / Q8_0 blocks, one per lane. Below 1024 waves of work a launch of
// 256-thread workgroups leaves most CUs idle (a 512-token K or V write of
// dim 1024 is 256 waves), so small jobs go out one wave per workgroup.
template <bool kQ4, bool kBias>
void launch_b32_with(const float* src, uint8_t* out, int64_t nb, const float* bias, int64_t nb_row,
                hipStream_t stream) {
  const int64_t waves = (nb + kWave - 1) / kWave;
  if (waves < 1024)
    hipLaunchKernelGGL((quantize_b32_kernel<kQ4, kWave, kBias>), dim3((unsigned)waves),
                       dim3(kWave), 0, stream, src, out, nb, bias, nb_row);
  else
    hipLaunchKernelGGL((quantize_b32_kernel<kQ4, kQThreads, kBias>),
                       dim3((unsigned)grid_for((nb + kQThreads - 1) / kQThreads)),
                       dim3(kQThreads), 0, stream, src, out, nb, bias, nb_row);
}

template <bool kQ4>
void launch_b32(const float* src, uint8_t* out, int64_t nb, const float* bias, int64_t nb_row,
                hipStream_t stream) {
  if (bias != nullptr)
    launch_b32_with<kQ4, true>(src, out, nb, bias, nb_row, stream);
  else
    launch_b32_with<kQ4, false>(src, out, nb, nullptr, nb_row, stream);
}

}  // namespace

hipError_t launch_quantize(int fmt, const float* W, void* blocks, int64_t rows, int64_t K,
                           hipStream_t stream) {
  uint8_t* out = static_cast<uint8_t*>(blocks);
  if (fmt == kFmtQ4_K || fmt == kFmtQ6_K) {
    const int64_t nsuper = rows * (K / 256);
    const int64_t chunks = (nsuper + kQkWaves * kQkSuperPerWave - 1) / (kQkWaves * kQkSuperPerWave);
    if (chunks == 0) return hipSuccess;
    if (fmt == kFmtQ4_K)
      hipLaunchKernelGGL(quantize_q4k_kernel, dim3((unsigned)grid_for(chunks)), dim3(kQThreads),
                         0, stream, W, out, nsuper);
    else
      hipLaunchKernelGGL(quantize_q6k_kernel, dim3((unsigned)grid_for(chunks)), dim3(kQThreads),
                         0, stream, W, out, nsuper);
  } else {
    const int64_t nb = rows * (K / 32);
    if (nb == 0) return hipSuccess;
    if (fmt == kFmtQ4_0)
      launch_b32<true>(W, out, nb, nullptr, 1, stream);
    else
      launch_b32<false>(W, out, nb, nullptr, 1, stream);
  }
  return hipGetLastError();
}

hipError_t launch_kv_write(int fmt, const float* rows, const float* bias, void* dst, int64_t n,
                           int64_t dim, hipStream_t stream) {
  const int64_t nb = n * (dim / 32);
  if (nb == 0) return hipSuccess;
  uint8_t* out = static_cast<uint8_t*>(dst);
  if (fmt == kFmtQ4_0)
    launch_b32<true>(rows, out, nb, bias, dim / 32, stream);
  else
    launch_b32<false>(rows, out, nb, bias, dim / 32, stream);
  return hipGetLastError();
}

}  // namespace qmat
