// Gate-weighted combine of the top-k expert outputs (standard top-k MoE
// mixing around the ButterflyMoE experts) and packing of the ternary substrate
// (ButterflyMoE gist.science summary, §2.1: W_base in {-1,0,+1}).
#include "common.h"
#include "kernels.h"

namespace bmoe {
namespace {

constexpr int kThreads = 256;

// y[t] = sum_j U[t*k + j] for ascending j, in fp32. U rows already carry
// their gate. Each thread handles 8 consecutive values of one token.
template <typename UT, typename YT>
__global__ __launch_bounds__(kThreads) void combine_kernel(const UT* U, YT* y, int T, int d,
                                                           int k) {
  const int d8 = d / 8;
  const size_t n = (size_t)T * d8;
  for (size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x; idx < n;
       idx += (size_t)gridDim.x * kThreads) {
    const size_t t = idx / d8, c = (idx % d8) * 8;
    float acc[8];
    for (int j = 0; j < k; ++j) {
      const UT* row = U + (t * k + j) * d + c;
      float v[8];
      if constexpr (sizeof(UT) == 2) {
        const uint4 w = *reinterpret_cast<const uint4*>(row);
        v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
        v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
      } else {
        const float4 a = *reinterpret_cast<const float4*>(row);
        const float4 b = *reinterpret_cast<const float4*>(row + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[m] = j == 0 ? v[m] : acc[m] + v[m];
    }
    YT* out = y + t * d + c;
    if constexpr (sizeof(YT) == 2) {
      *reinterpret_cast<uint4*>(out) = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                                  pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
    } else {
      *reinterpret_cast<float4*>(out) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *reinterpret_cast<float4*>(out + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

__global__ void set_status_kernel(int32_t* status, int32_t v) { *status = v; }

// One thread per packed word: 16 consecutive int8 entries of one row.
__global__ __launch_bounds__(kThreads) void pack_kernel(const int8_t* w, int d, uint32_t* packed,
                                                        int32_t* status) {
  const int G = d / 16;
  const size_t n = (size_t)d * G;
  for (size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x; idx < n;
       idx += (size_t)gridDim.x * kThreads) {
    const size_t o = idx / G, g = idx % G;
    const uint4 raw = *reinterpret_cast<const uint4*>(w + o * d + g * 16);
    const uint32_t parts[4] = {raw.x, raw.y, raw.z, raw.w};
    uint32_t word = 0;
    bool bad = false;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int8_t val = (int8_t)((parts[v >> 2] >> (8 * (v & 3))) & 0xFFu);
      const int j = v >> 1;
      const int nz_bit = (v & 1) ? 16 + 2 * j : 2 * j;
      const int sg_bit = nz_bit + 1;
      if (val == 1) {
        word |= 1u << nz_bit;
      } else if (val == -1) {
        word |= (1u << nz_bit) | (1u << sg_bit);
      } else if (val != 0) {
        bad = true;
      }
    }
    if (bad) *status = BMOE_E_TERNARY;  // every writer stores the same value
    packed[idx] = word;
  }
}

int grid_for(size_t n) {
  size_t b = (n + kThreads - 1) / kThreads;
  if (b > 8192) b = 8192;
  if (b < 1) b = 1;
  return (int)b;
}

}  // namespace

hipError_t launch_combine(bmoe_dtype dt, int T, int d, int k, const void* u, void* y,
                          hipStream_t s, const KernelTiming& t) {
  const int g = grid_for((size_t)T * (d / 8));
  if (dt == BMOE_BF16)
    return launch_kernel(combine_kernel<uint16_t, uint16_t>, dim3(g), dim3(kThreads), 0, s, t,
                         static_cast<const uint16_t*>(u), static_cast<uint16_t*>(y), T, d, k);
  return launch_kernel(combine_kernel<float, float>, dim3(g), dim3(kThreads), 0, s, t,
                       static_cast<const float*>(u), static_cast<float*>(y), T, d, k);
}

hipError_t launch_pack(const int8_t* w, int d, uint32_t* packed, int32_t* status,
                       hipStream_t s) {
  hipLaunchKernelGGL(set_status_kernel, dim3(1), dim3(1), 0, s, status, (int32_t)BMOE_OK);
  hipLaunchKernelGGL(pack_kernel, dim3(grid_for((size_t)d * (d / 16))), dim3(kThreads), 0, s, w, d,
                     packed, status);
  return hipGetLastError();
}

}  // namespace bmoe
