// Outlier-spreading measurement (ButterflyMoE gist.science summary, §2.4 and
// §4: the rotation B(theta_e) spreads activation energy over the dimensions,
// which lowers the activation quantisation error). Per row v of a matrix:
//   s = max|v| / m (mode 0, absmax) or mean|v| (mode 1, absmean)
//   q = s * clip(rint(v / s), -m, m),  err = ||v - q|| / ||v||,
//   crest = max|v| / rms(v);  a zero row gives 0 for both.
// Rounding a half either way leaves |v - q| = s/2, so err does not depend on
// the tie rule.
#include "common.h"
#include "kernels.h"

namespace bmoe {
namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// One wave per row, 16-byte loads; a second pass over the row (from cache)
// measures the error once the scale is known.
template <typename T>
__global__ __launch_bounds__(256) void quant_error_kernel(const T* src, int rows, int d, int m,
                                                          int mode, float* err, float* crest) {
  constexpr int VS = 16 / sizeof(T);
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wave
  const T* v = src + (size_t)row * d;
  const int nch = d / VS;
  float amax = 0.f, asum = 0.f, sq = 0.f;
  for (int c = lane; c < nch; c += 64) {
    float f[VS];
    load16<T>(v + c * VS, f);
#pragma unroll
    for (int i = 0; i < VS; ++i) {
      const float a = fabsf(f[i]);
      amax = fmaxf(amax, a);
      asum += a;
      sq += f[i] * f[i];
    }
  }
  amax = wave_max(amax);
  asum = wave_sum(asum);
  sq = wave_sum(sq);
  const float s = mode == 0 ? amax / (float)m : asum / (float)d;
  float e2 = 0.f;
  if (s > 0.f) {
    const float lim = (float)m;
    for (int c = lane; c < nch; c += 64) {
      float f[VS];
      load16<T>(v + c * VS, f);
#pragma unroll
      for (int i = 0; i < VS; ++i) {
        const float q = s * fminf(fmaxf(rintf(f[i] / s), -lim), lim);
        e2 += (f[i] - q) * (f[i] - q);
      }
    }
    e2 = wave_sum(e2);
  }
  if (lane == 0) {
    err[row] = s > 0.f ? sqrtf(e2 / sq) : 0.f;
    if (crest) crest[row] = sq > 0.f ? amax / sqrtf(sq / (float)d) : 0.f;
  }
}

}  // namespace

hipError_t launch_quant_error(bmoe_dtype dt, int rows, int d, const void* src, int m, int mode,
                              float* err, float* crest, hipStream_t s, const KernelTiming& t) {
  const dim3 grid((rows + 3) / 4);
  if (dt == BMOE_BF16)
    return launch_kernel(quant_error_kernel<uint16_t>, grid, dim3(256), 0, s, t,
                         static_cast<const uint16_t*>(src), rows, d, m, mode, err, crest);
  return launch_kernel(quant_error_kernel<float>, grid, dim3(256), 0, s, t,
                       static_cast<const float*>(src), rows, d, m, mode, err, crest);
}

}  // namespace bmoe
