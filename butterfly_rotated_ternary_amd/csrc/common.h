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

// fp32 -> bf16 bit pattern, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Packed substrate word -> 8 dwords, each two bf16 values of {-1, 0, +1}.
// Word layout: column v = 2j has its nonzero flag at bit j and sign at bit
// 8+j; v = 2j+1 at bits 16+j and 24+j. Dword j = (value 2j, value 2j+1):
// shifting left by 7-j puts the two nonzero flags at bits 7 and 23 and the
// two signs at bits 15 and 31; flag * 0x7F spreads a flag into 0x3F80 (the
// bf16 pattern of 1.0, shifted by 0 or 16) and the signs are added on top.
__device__ __forceinline__ uint32_t unpack_pair(uint32_t w, int j) {
  const uint32_t t = w << (7 - j);
  return __umul24(t & 0x00800080u, 0x7Fu) + (t & 0x80008000u);
}

// Workgroup barrier ordering LDS traffic only: waits for this wave's LDS
// operations, then s_barrier. Unlike __syncthreads it does not wait for
// global->LDS loads still in flight; code that needs their data waits for
// them explicitly (vmcnt) first. The memory clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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
