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
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left alone), visible to the
// compiler's own wait-count tracking: registers loaded before it need no
// further wait afterwards, on any path.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ void lds_barrier() {
  // The wait goes through the builtin too, so the compiler's own wait-count
  // tracking sees that every LDS operation issued before the barrier has
  // completed (an opaque asm wait makes it wait again after the barrier,
  // together with whatever LDS reads were issued there).
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt untouched
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

// (cos x, sin x) on the transcendental unit, whose v_sin /
// v_cos take revolutions. x is first reduced to [-pi, pi] by subtracting the
// nearest multiple of 2pi in two fused steps (Cody and Waite's method: 2pi
// split into its nearest float and the remainder), then scaled by 1/2pi.
// Measured against double precision: at most 4e-7 absolute error for
// |x| <= 1000 (sincosf: 7e-8).
__device__ __forceinline__ float2 tile_cos_sin(float x) {
  constexpr float kInv2Pi = 0.159154943091895336f;
  constexpr float k2PiHi = 6.28318548202514648f;   // float(2 pi)
  constexpr float k2PiLo = -1.74845553146951449e-7f;  // 2 pi - float(2 pi)
  const float k = rintf(x * kInv2Pi);
  const float r = fmaf(-k, k2PiLo, fmaf(-k, k2PiHi, x)) * kInv2Pi;
  return make_float2(__builtin_amdgcn_cosf(r), __builtin_amdgcn_sinf(r));
}

// Eight bf16 {-2,0,+2} of one packed word: values 8h .. 8h+7 (h = 0, 1).
__device__ __forceinline__ bf16x8 unpack_frag(uint32_t w, int h) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = unpack_pair(w, 4 * h + i);
  return __builtin_bit_cast(bf16x8, r);
}

// Wave-level exchanges of the register-resident butterflies.
__device__ __forceinline__ float fneg_if(float v, int neg) {
  return __int_as_float(__float_as_int(v) ^ (neg << 31));
}

// Register-resident rows are spread over the lanes in "row lane" order: the
// row position c of physical lane l is row_lane(l) = l ^ 3 * bit2(l) (an
// involution). Flipping bit 0, 1 or 3 of c flips the same lane bit, and
// flipping bit 2 of c flips lane bits 0-2 together, i.e. lane ^ 7, which is
// DPP row_half_mirror. So every partner within a row of 16 lanes is one
// full-mask DPP move that folds into the multiply using it.
__device__ __forceinline__ int row_lane(int l) { return l ^ (((l >> 2) & 1) * 3); }

// Partner value across bit M (0..3) of the row position (lanes in row_lane
// order).
template <int M>
__device__ __forceinline__ float lane_partner(float v) {
  const int iv = __float_as_int(v);
  int r;
  if constexpr (M == 0) {
    r = __builtin_amdgcn_mov_dpp(iv, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]: lane ^ 1
  } else if constexpr (M == 1) {
    r = __builtin_amdgcn_mov_dpp(iv, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]: lane ^ 2
  } else if constexpr (M == 2) {
    r = __builtin_amdgcn_mov_dpp(iv, 0x141, 0xF, 0xF, true); // row_half_mirror: lane ^ 7
  } else {
    r = __builtin_amdgcn_mov_dpp(iv, 0x128, 0xF, 0xF, true);  // row_ror:8: lane ^ 8
  }
  return __int_as_float(r);
}

// Inclusive prefix sum of v over the 64 lanes, in lane order, through DPP
// (no LDS round trip): shifts by 1, 2, 4 and 8 within each row of 16 lanes,
// then the last lane of row 0 (and 2) into row 1 (and 3), and lane 31 into
// rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false); // row_bcast:15, rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false); // row_bcast:31, rows 2, 3
  return v;
}

// Swap half of register a with half of register b across lane bit M (4 or
// 5, equal in row-lane order): afterwards lanes with that bit clear hold (a, partner of a), lanes with
// it set hold (partner of b, b). Applying it twice restores both.
template <int M>
__device__ __forceinline__ void lane_swap(float& a, float& b) {
  const unsigned ia = __float_as_uint(a), ib = __float_as_uint(b);
  if constexpr (M == 4) {
    const auto r = __builtin_amdgcn_permlane16_swap(ia, ib, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(ia, ib, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  }
}

}  // namespace bmoe
