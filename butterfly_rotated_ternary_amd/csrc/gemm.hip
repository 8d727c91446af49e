// Shared-substrate product H = alpha * Z W_base^T over every routed row at
// once (ButterflyMoE gist.science summary, §2.3 step 2: one ternary W_base
// serves all experts, so the contraction is a single dense GEMM).
//
// bf16 MFMA (v_mfma_f32_16x16x32_bf16) with fp32 accumulation. The packed
// 2-bit substrate is expanded to exact bf16 {-1,0,+1} while staging it in
// LDS, so the products are exact. For fp32 activations each Z value is split
// into three bf16 terms (hi + mid + lo represent it to within 2^-24 relative),
// and the three partial products accumulate in fp32.
#include "common.h"
#include "kernels.h"

namespace bmoe {
namespace {

constexpr int kThreads = 256;
constexpr int BM = 64, BN = 64, BK = 32;
constexpr int LDA = BK + 8;  // bf16 per LDS row (pad breaks bank aliasing)

__device__ __forceinline__ void split3(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = f32_to_bf16_bits(x);
  const float r1 = x - __uint_as_float(hi << 16);
  mid = f32_to_bf16_bits(r1);
  const float r2 = r1 - __uint_as_float(mid << 16);
  lo = f32_to_bf16_bits(r2);
}

template <bool F32A>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const void* zv, const uint32_t* wp,
                                                        float* H, int M, int d, float alpha) {
  constexpr int SPL = F32A ? 3 : 1;
  __shared__ __attribute__((aligned(16))) uint16_t As[SPL][BM * LDA];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDA];

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
  const int G = d / 16;

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < d; k0 += BK) {
    if constexpr (!F32A) {
      const uint16_t* Z = static_cast<const uint16_t*>(zv);
      const int row = tid >> 2, kc = (tid & 3) * 8;
      const int gr = m0 + row;
      uint4 v = {0u, 0u, 0u, 0u};
      if (gr < M && k0 + kc < d) v = *reinterpret_cast<const uint4*>(Z + (size_t)gr * d + k0 + kc);
      *reinterpret_cast<uint4*>(&As[0][row * LDA + kc]) = v;
    } else {
      const float* Z = static_cast<const float*>(zv);
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int idx = tid + it * kThreads;
        const int row = idx >> 3, kc = (idx & 7) * 4;
        const int gr = m0 + row;
        float4 v = {0.f, 0.f, 0.f, 0.f};
        if (gr < M && k0 + kc < d) v = *reinterpret_cast<const float4*>(Z + (size_t)gr * d + k0 + kc);
        uint32_t h[4], m[4], l[4];
        split3(v.x, h[0], m[0], l[0]);
        split3(v.y, h[1], m[1], l[1]);
        split3(v.z, h[2], m[2], l[2]);
        split3(v.w, h[3], m[3], l[3]);
        *reinterpret_cast<uint2*>(&As[0][row * LDA + kc]) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        *reinterpret_cast<uint2*>(&As[1][row * LDA + kc]) = make_uint2(m[0] | (m[1] << 16), m[2] | (m[3] << 16));
        *reinterpret_cast<uint2*>(&As[2][row * LDA + kc]) = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
      }
    }
    if (tid < BN * (BK / 16)) {
      const int o = tid >> 1, wi = tid & 1;
      const int go = n0 + o, c0 = k0 + wi * 16;
      uint32_t w = 0;
      if (go < d && c0 < d) w = wp[(size_t)go * G + c0 / 16];
      uint4 lo4, hi4;
      lo4.x = unpack_pair(w, 0); lo4.y = unpack_pair(w, 1);
      lo4.z = unpack_pair(w, 2); lo4.w = unpack_pair(w, 3);
      hi4.x = unpack_pair(w, 4); hi4.y = unpack_pair(w, 5);
      hi4.z = unpack_pair(w, 6); hi4.w = unpack_pair(w, 7);
      *reinterpret_cast<uint4*>(&Bs[o * LDA + wi * 16]) = lo4;
      *reinterpret_cast<uint4*>(&Bs[o * LDA + wi * 16 + 8]) = hi4;
    }
    __syncthreads();

    bf16x8 b[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      b[j] = *reinterpret_cast<const bf16x8*>(&Bs[(wn * 32 + j * 16 + (lane & 15)) * LDA + 8 * (lane >> 4)]);
#pragma unroll
    for (int sp = 0; sp < SPL; ++sp) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            &As[SPL - 1 - sp][(wm * 32 + i * 16 + (lane & 15)) * LDA + 8 * (lane >> 4)]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[j], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * 32 + i * 16 + 4 * (lane >> 4) + r;
        const int col = n0 + wn * 32 + j * 16 + (lane & 15);
        if (row < M && col < d) H[(size_t)row * d + col] = alpha * acc[i][j][r];
      }
}

}  // namespace

hipError_t launch_gemm(bmoe_dtype dt, int M, int d, const void* z, const uint32_t* w_packed,
                       float alpha, float* h, hipStream_t s) {
  dim3 grid((M + BM - 1) / BM, (d + BN - 1) / BN);
  if (dt == BMOE_BF16)
    hipLaunchKernelGGL(gemm_kernel<false>, grid, dim3(kThreads), 0, s, z, w_packed, h, M, d, alpha);
  else
    hipLaunchKernelGGL(gemm_kernel<true>, grid, dim3(kThreads), 0, s, z, w_packed, h, M, d, alpha);
  return hipGetLastError();
}

}  // namespace bmoe
