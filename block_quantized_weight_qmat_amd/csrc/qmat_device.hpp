// qmat_device.hpp — small device-side helpers shared by the qmat kernels.
// gfx950 (CDNA4) only: 64-lane wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmat {

constexpr int kWave = 64;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// A 16-byte vector that is only known to be 4-byte aligned (packed blocks
// of 18 or 34 bytes start at 2- or 4-byte offsets).
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// Note: bit-cast whole vectors, never a subscripted element (vec[i]): clang
// lowers __builtin_bit_cast of a vector subscript as a read of element 0.

// Binary16 bits of an fp32 value: round to nearest even, subnormals kept
// (v_cvt_f16_f32 in the default IEEE mode).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float v) {
  _Float16 h = (_Float16)v;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// fp32 value of binary16 bits held in the low half of a register (exact).
__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}

__device__ __forceinline__ half2_t as_half2(uint32_t v) {
  return __builtin_bit_cast(half2_t, v);
}

__device__ __forceinline__ uint32_t as_u32(half2_t v) {
  return __builtin_bit_cast(uint32_t, v);
}

// Byte permute: result byte k = byte sel[k] of the 8-byte value {hi:lo}
// (bytes 0..3 from lo, 4..7 from hi; selector 0x0c gives 0x00).
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// v_dot2_f32_f16: a.lo*b.lo + a.hi*b.hi + c with fp32 accumulation; the
// fp16 products are exact in fp32.
__device__ __forceinline__ float dot2(uint32_t a, half2_t b, float c) {
  return __builtin_amdgcn_fdot2(as_half2(a), b, c, false);
}

// Buffer resource over [base, base + bytes) for raw buffer loads (gfx9
// descriptor: stride 0, 32-bit dword data format). Lane offsets are 32-bit;
// a load at or past `bytes` returns zeros without a memory access, which
// lets a kernel issue the same loads on every lane and path.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes < (int64_t)0xFFFFFFFF ? (uint32_t)bytes : 0xFFFFFFFFu;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n,
                                           0x00020000);
}

// LDS pointers for the direct memory-to-LDS loads (global_load_lds).
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt immediate (gfx9 encoding) that waits until at most N vector
// memory operations are outstanding, leaving the other counters free.
template <int N>
constexpr int vmcnt_imm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  return (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ uint32_t shfl_xor_u(uint32_t v, int mask) {
  return (uint32_t)__shfl_xor((int)v, mask, kWave);
}

}  // namespace qmat
