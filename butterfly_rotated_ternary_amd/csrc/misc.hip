// Gate-weighted combine of the top-k expert outputs (standard top-k MoE
// mixing around the ButterflyMoE experts) and packing of the ternary substrate
// (ButterflyMoE gist.science summary, §2.1: W_base in {-1,0,+1}).
#include "common.h"
#include "kernels.h"

namespace bmoe {
namespace {

constexpr int kThreads = 256;

// y[t] = sum_j U[t*k + j] for ascending j. U rows already carry their gate.
template <typename YT>
__global__ __launch_bounds__(kThreads) void combine_kernel(const float* U, YT* y, int T, int d,
                                                           int k) {
  const int d4 = d / 4;
  const size_t n = (size_t)T * d4;
  for (size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x; idx < n;
       idx += (size_t)gridDim.x * kThreads) {
    const size_t t = idx / d4, c = idx % d4;
    const float4* row = reinterpret_cast<const float4*>(U + t * k * d) + c;
    float4 acc = row[0];
    for (int j = 1; j < k; ++j) {
      const float4 v = row[(size_t)j * d4];
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    if constexpr (sizeof(YT) == 2) {
      reinterpret_cast<uint2*>(y)[idx] = make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
    } else {
      reinterpret_cast<float4*>(y)[idx] = acc;
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
      const int nz_bit = (v & 1) ? 16 + j : j;
      const int sg_bit = nz_bit + 8;
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

hipError_t launch_combine(bmoe_dtype dt, int T, int d, int k, const float* u, void* y,
                          hipStream_t s) {
  const int g = grid_for((size_t)T * (d / 4));
  if (dt == BMOE_BF16)
    hipLaunchKernelGGL(combine_kernel<uint16_t>, dim3(g), dim3(kThreads), 0, s, u,
                       static_cast<uint16_t*>(y), T, d, k);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3(g), dim3(kThreads), 0, s, u,
                       static_cast<float*>(y), T, d, k);
  return hipGetLastError();
}

hipError_t launch_pack(const int8_t* w, int d, uint32_t* packed, int32_t* status,
                       hipStream_t s) {
  hipLaunchKernelGGL(set_status_kernel, dim3(1), dim3(1), 0, s, status, (int32_t)BMOE_OK);
  hipLaunchKernelGGL(pack_kernel, dim3(grid_for((size_t)d * (d / 16))), dim3(kThreads), 0, s, w, d,
                     packed, status);
  return hipGetLastError();
}

}  // namespace bmoe
