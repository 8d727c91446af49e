// Measured ceilings of the resources the layer's kernels are bounded by, for
// reporting next to the published peaks: dense bf16 MFMA throughput, fp32
// vector FMA throughput (no packed ops, like every kernel here) and the
// bandwidth of a plain device copy. None of this is part of the layer.
#include "common.h"
#include "kernels.h"

namespace bmoe {
namespace {

constexpr int kCeilThreads = 256;
// Eight four-wave workgroups per CU: eight waves per SIMD.
constexpr int kCeilBlocks = 256 * 8;
constexpr int kChains = 4;

// Each wave runs kChains independent chains of v_mfma_f32_32x32x16_bf16 on
// operands held in registers.
__global__ __launch_bounds__(kCeilThreads) void mfma_ceiling_kernel(int iters, float* sink) {
  const int lane = threadIdx.x % kWave;
  u32x4 ra, rb;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ra[i] = pack_bf16x2(0.001f * (lane + i), 0.002f * i);
    rb[i] = pack_bf16x2(0.003f * i, 0.001f * (lane - i));
  }
  const bf16x8 a = __builtin_bit_cast(bf16x8, ra), b = __builtin_bit_cast(bf16x8, rb);
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[blockIdx.x * kCeilThreads + threadIdx.x] = s;
}

// Each thread runs eight independent chains of fp32 fused multiply-adds.
__global__ __launch_bounds__(kCeilThreads) void valu_ceiling_kernel(int iters, float* sink) {
  float v[8];
  const float m = 1.0f - 1e-7f * (threadIdx.x % 7), c = 1e-7f * (threadIdx.x % 5);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.5f + 0.01f * i + 1e-4f * threadIdx.x;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = fmaf(v[i], m, c);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += v[i];
  sink[blockIdx.x * kCeilThreads + threadIdx.x] = s;
}

// Copy in 16-byte units: a workgroup moves chunks of kCopyUnroll * 256
// consecutive units, each thread keeping kCopyUnroll loads in flight before
// its stores; the tail is copied one unit per thread.
constexpr int kCopyUnroll = 4;
__global__ __launch_bounds__(kCeilThreads) void copy_ceiling_kernel(const uint4* src, uint4* dst,
                                                                    size_t n) {
  constexpr size_t kChunk = (size_t)kCopyUnroll * kCeilThreads;
  const size_t nchunks = n / kChunk;
  for (size_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
    const size_t base = c * kChunk + threadIdx.x;
    uint4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) v[u] = src[base + (size_t)u * kCeilThreads];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) dst[base + (size_t)u * kCeilThreads] = v[u];
  }
  for (size_t i = nchunks * kChunk + (size_t)blockIdx.x * kCeilThreads + threadIdx.x; i < n;
       i += (size_t)gridDim.x * kCeilThreads)
    dst[i] = src[i];
}

KernelTiming timing_of(void* const* events) {
  KernelTiming t;
  if (events) {
    t.start = static_cast<hipEvent_t>(events[0]);
    t.stop = static_cast<hipEvent_t>(events[1]);
  }
  return t;
}

}  // namespace
}  // namespace bmoe

using namespace bmoe;

extern "C" {

bmoe_status bmoe_ceiling_mfma_bf16(int iters, float* sink, void* stream, void* const* events,
                                   double* flops) {
  if (iters < 1) return BMOE_E_SHAPE;
  if (!sink) return BMOE_E_NULL;
  if (launch_kernel(mfma_ceiling_kernel, dim3(kCeilBlocks), dim3(kCeilThreads), 0,
                    static_cast<hipStream_t>(stream), timing_of(events), iters,
                    sink) != hipSuccess)
    return BMOE_E_HIP;
  if (flops)
    *flops = (double)kCeilBlocks * (kCeilThreads / kWave) * kChains * iters * (32.0 * 32 * 16 * 2);
  return BMOE_OK;
}

bmoe_status bmoe_ceiling_valu_f32(int iters, float* sink, void* stream, void* const* events,
                                  double* flops) {
  if (iters < 1) return BMOE_E_SHAPE;
  if (!sink) return BMOE_E_NULL;
  if (launch_kernel(valu_ceiling_kernel, dim3(kCeilBlocks), dim3(kCeilThreads), 0,
                    static_cast<hipStream_t>(stream), timing_of(events), iters,
                    sink) != hipSuccess)
    return BMOE_E_HIP;
  if (flops) *flops = (double)kCeilBlocks * kCeilThreads * iters * 16.0 * 8 * 2;
  return BMOE_OK;
}

bmoe_status bmoe_ceiling_copy(const void* src, void* dst, size_t bytes, void* stream,
                              void* const* events) {
  if (!src || !dst) return BMOE_E_NULL;
  if (bytes == 0 || bytes % 16 != 0) return BMOE_E_SHAPE;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u)
    return BMOE_E_ALIGN;
  const size_t n = bytes / 16;
  size_t blocks = (n + kCopyUnroll * kCeilThreads - 1) / (kCopyUnroll * kCeilThreads);
  if (blocks > 256 * 32) blocks = 256 * 32;
  if (launch_kernel(copy_ceiling_kernel, dim3((unsigned)blocks), dim3(kCeilThreads), 0,
                    static_cast<hipStream_t>(stream), timing_of(events),
                    static_cast<const uint4*>(src), static_cast<uint4*>(dst), n) != hipSuccess)
    return BMOE_E_HIP;
  return BMOE_OK;
}

}  // extern "C"
