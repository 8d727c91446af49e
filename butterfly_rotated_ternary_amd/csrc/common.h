// Device helpers shared by the ButterflyMoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bmoe.h"

namespace bmoe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxExperts = 4096;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even:
// one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
// fp32 -> bf16 bit pattern, round to nearest even.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.f) & 0xFFFFu; }
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Packed substrate word -> 8 dwords, each two bf16 values of {-2, 0, +2}:
// twice the ternary weights, so every kernel applies alpha / 2 to its fp32
// accumulator (a power-of-two rescale: the result is bit-identical to using
// +-1 and alpha). Word layout: 2-bit codes (flag low bit, sign high bit);
// column 2j at bits 2j..2j+1, column 2j+1 at bits 16+2j..17+2j. Shifting left
// by 14 - 2j puts the pair's codes at bits 14..15 and 30..31, exactly where
// bf16 2.0 (0x4000) has its one exponent bit and where the sign bit sits, so
// one shift and one mask give dword j = (value 2j, value 2j+1).
__device__ __forceinline__ uint32_t unpack_pair(uint32_t w, int j) {
  return (w << (14 - 2 * j)) & 0xC000C000u;
}

// The scale kernels apply to an accumulator of expanded (+-2) substrate values.
__host__ __device__ __forceinline__ float substrate_scale(float alpha) { return 0.5f * alpha; }

// Workgroup barrier ordering LDS traffic only: waits for this wave's LDS
// operations, then s_barrier. Unlike __syncthreads it does not wait for
// global->LDS loads still in flight; code that needs their data waits for
// them explicitly (vmcnt) first. The memory clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16 bytes of a row (8 bf16 or 4 fp32) to fp32 (in LDS or registers).
template <typename T>
__device__ __forceinline__ void load16(const T* src, float* dst) {
  const uint4 v = *reinterpret_cast<const uint4*>(src);
  if constexpr (sizeof(T) == 2) {
    dst[0] = bf16_lo(v.x); dst[1] = bf16_hi(v.x);
    dst[2] = bf16_lo(v.y); dst[3] = bf16_hi(v.y);
    dst[4] = bf16_lo(v.z); dst[5] = bf16_hi(v.z);
    dst[6] = bf16_lo(v.w); dst[7] = bf16_hi(v.w);
  } else {  // padded LDS rows are only 4-byte aligned here
    dst[0] = __uint_as_float(v.x); dst[1] = __uint_as_float(v.y);
    dst[2] = __uint_as_float(v.z); dst[3] = __uint_as_float(v.w);
  }
}

// fp32 values from LDS (times `scale`) to 16 bytes of a row.
template <typename T>
__device__ __forceinline__ void store16(const float* s, T* dst, float scale) {
  uint4 v;
  if constexpr (sizeof(T) == 2) {
    v.x = pack_bf16x2(s[0] * scale, s[1] * scale);
    v.y = pack_bf16x2(s[2] * scale, s[3] * scale);
    v.z = pack_bf16x2(s[4] * scale, s[5] * scale);
    v.w = pack_bf16x2(s[6] * scale, s[7] * scale);
  } else {
    v.x = __float_as_uint(s[0] * scale);
    v.y = __float_as_uint(s[1] * scale);
    v.z = __float_as_uint(s[2] * scale);
    v.w = __float_as_uint(s[3] * scale);
  }
  *reinterpret_cast<uint4*>(dst) = v;
}

// Index of the j-th element of a block of 2^g elements whose varying index
// bits start at bit s_lo; `b` enumerates blocks (all other index bits).
__device__ __forceinline__ int block_base(int b, int s_lo, int g) {
  int low = b & ((1 << s_lo) - 1);
  return ((b >> s_lo) << (s_lo + g)) | low;
}

// Pair index of element i within stage s (element i has bit s clear).
__device__ __forceinline__ int pair_index(int i, int s) {
  return ((i >> (s + 1)) << s) | (i & ((1 << s) - 1));
}

}  // namespace bmoe
