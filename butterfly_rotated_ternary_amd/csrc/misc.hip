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

// One thread per packed word: 16 consecutive int8 entries of one row (d < 16:
// the row's d entries, the rest of the word zero codes).
__global__ __launch_bounds__(kThreads) void pack_kernel(const int8_t* w, int d, uint32_t* packed,
                                                        int32_t* status) {
  const int G = (d + 15) / 16;
  const size_t n = (size_t)d * G;
  for (size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x; idx < n;
       idx += (size_t)gridDim.x * kThreads) {
    const size_t o = idx / G, g = idx % G;
    uint32_t parts[4] = {0u, 0u, 0u, 0u};
    if (d >= 16) {
      const uint4 raw = *reinterpret_cast<const uint4*>(w + o * d + g * 16);
      parts[0] = raw.x; parts[1] = raw.y; parts[2] = raw.z; parts[3] = raw.w;
    } else {
      for (int v = 0; v < d; ++v)
        parts[v >> 2] |= (uint32_t)(uint8_t)w[o * d + v] << (8 * (v & 3));
    }
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

// ---- base-3 storage (summary §2.1: 1.58 bits per weight) --------------------
// Five ternary digits per byte over the row-major entries n = o*d + c:
// byte j = sum_i (w[5j+i] + 1) * 3^i, digits past d*d equal to 1 (value 0).
__global__ __launch_bounds__(kThreads) void pack_b3_kernel(const int8_t* w, size_t nw,
                                                           uint8_t* out, size_t nb,
                                                           int32_t* status) {
  for (size_t j = (size_t)blockIdx.x * kThreads + threadIdx.x; j < nb;
       j += (size_t)gridDim.x * kThreads) {
    uint32_t byte = 0, scale = 1;
    bool bad = false;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const size_t n = 5 * j + i;
      const int v = n < nw ? (int)w[n] : 0;
      if (v < -1 || v > 1) bad = true;
      byte += (uint32_t)(v < -1 || v > 1 ? 1 : v + 1) * scale;
      scale *= 3;
    }
    if (bad) *status = BMOE_E_TERNARY;  // every writer stores the same value
    out[j] = (uint8_t)byte;
  }
}

// One thread per 2-bit word (row o, columns 16g .. 16g+15): its 16 entries
// lie in at most 4 consecutive bytes. An LDS table maps each byte value to
// its five digits as 2-bit codes in entry order (digit t = 0, 1, 2, i.e.
// -1, 0, +1, becomes code 3, 0, 1; byte values above 242 map to 0xFFFF).
// The four bytes' codes are concatenated, shifted to the word's first entry,
// and split into the word layout: even columns in the low half, odd columns
// in the high half.
__global__ __launch_bounds__(kThreads) void unpack_b3_kernel(const uint8_t* in, size_t nb,
                                                             uint32_t* packed, size_t nwords,
                                                             int32_t* status) {
  __shared__ uint16_t lut[256];
  for (int v = threadIdx.x; v < 256; v += kThreads) {
    uint32_t codes = 0xFFFFu, rest = (uint32_t)v;
    if (v <= 242) {
      codes = 0;
      for (int i = 0; i < 5; ++i) {
        const uint32_t t = rest % 3u;
        rest /= 3u;
        codes |= (t == 0 ? 3u : t == 2 ? 1u : 0u) << (2 * i);
      }
    }
    lut[v] = (uint16_t)codes;
  }
  __syncthreads();
  for (size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x; idx < nwords;
       idx += (size_t)gridDim.x * kThreads) {
    const size_t e0 = idx * 16, b0 = e0 / 5;
    const int pos = (int)(e0 - 5 * b0);
    uint64_t seq = 0;
    bool bad = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t c = b0 + i < nb ? lut[in[b0 + i]] : 0u;
      bad |= c == 0xFFFFu;
      seq |= (uint64_t)(c & 0x3FFu) << (10 * i);
    }
    const uint32_t codes = (uint32_t)(seq >> (2 * pos));  // code of entry v at bits 2v, 2v+1
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      word |= ((codes >> (4 * j)) & 3u) << (2 * j);             // column 2j
      word |= ((codes >> (4 * j + 2)) & 3u) << (16 + 2 * j);    // column 2j + 1
    }
    if (bad) *status = BMOE_E_TERNARY;
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
  hipLaunchKernelGGL(pack_kernel, dim3(grid_for((size_t)d * ((d + 15) / 16))), dim3(kThreads), 0,
                     s, w, d, packed, status);
  return hipGetLastError();
}

hipError_t launch_pack_b3(const int8_t* w, int d, uint8_t* packed3, int32_t* status,
                          hipStream_t s) {
  const size_t nw = (size_t)d * d, nb = (nw + 4) / 5;
  hipLaunchKernelGGL(set_status_kernel, dim3(1), dim3(1), 0, s, status, (int32_t)BMOE_OK);
  hipLaunchKernelGGL(pack_b3_kernel, dim3(grid_for(nb)), dim3(kThreads), 0, s, w, nw, packed3, nb,
                     status);
  return hipGetLastError();
}

hipError_t launch_unpack_b3(const uint8_t* packed3, int d, uint32_t* packed, int32_t* status,
                            hipStream_t s, const KernelTiming& t) {
  hipLaunchKernelGGL(set_status_kernel, dim3(1), dim3(1), 0, s, status, (int32_t)BMOE_OK);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const size_t nw = (size_t)d * (d / 16), nb = ((size_t)d * d + 4) / 5;
  return launch_kernel(unpack_b3_kernel, dim3(grid_for(nw)), dim3(kThreads), 0, s, t, packed3, nb,
                       packed, nw, status);
}

}  // namespace bmoe
