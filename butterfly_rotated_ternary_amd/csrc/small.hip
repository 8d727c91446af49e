// Whole forward for d in {2, 4, 8} (ButterflyMoE gist.science summary, §2.3:
// rotate by B(theta_e)^T, multiply by the shared ternary W_base, rotate by
// B(phi_e), then the gate-weighted sum over the token's top-k experts).
//
// A row of at most 8 values fits in one thread's registers, and the product
// is at most 64 multiply-adds, so there is nothing for matrix cores or LDS to
// do: one thread per token runs its k routed rows in ascending j. The
// cos/sin tables come from the prep kernel (stage-major per expert), as on
// every other path. Rounding points follow the bf16 path elsewhere: Z is
// rounded to bf16 before the product, H stays fp32 (as in the fused kernel),
// each gate-weighted row g * U is rounded to the activation type, and the
// rows are summed in fp32 and rounded once.
#include "common.h"
#include "kernels.h"

namespace bmoe {
namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ float load_act(const T* p) {
  if constexpr (sizeof(T) == 2)
    return __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(p)) << 16);
  else
    return *p;
}

// Round to the activation type and back (identity for fp32).
template <typename T>
__device__ __forceinline__ float round_act(float v) {
  if constexpr (sizeof(T) == 2)
    return __uint_as_float(f32_to_bf16_bits(v) << 16);
  else
    return v;
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void small_kernel(const T* x, const int32_t* ids,
                                                         const float* gates, const float2* cs_in,
                                                         const float2* cs_out,
                                                         const uint32_t* w_packed, float alpha,
                                                         T* y, int Tn, int k, int N) {
  constexpr int L = D == 2 ? 1 : D == 4 ? 2 : 3;
  constexpr int P = D / 2;
  const int t = blockIdx.x * kThreads + threadIdx.x;
  if (t >= Tn) return;
  // Substrate rows: one word each, column c's code at bit 2(c/2) (+16 for
  // odd c), flag in the low bit, sign in the high bit.
  float w[D][D];
#pragma unroll
  for (int o = 0; o < D; ++o) {
    const uint32_t word = w_packed[o];
#pragma unroll
    for (int c = 0; c < D; ++c) {
      const int pos = (c & 1) ? 16 + 2 * (c >> 1) : 2 * (c >> 1);
      const uint32_t code = (word >> pos) & 3u;
      w[o][c] = code == 1u ? 1.f : code == 3u ? -1.f : 0.f;
    }
  }
  float xin[D];
#pragma unroll
  for (int c = 0; c < D; ++c) xin[c] = load_act(x + (size_t)t * D + c);
  float acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) acc[c] = 0.f;
  for (int j = 0; j < k; ++j) {
    const size_t r = (size_t)t * k + j;
    int e = ids[r];
    e = e < 0 ? 0 : e >= N ? N - 1 : e;  // the prep kernel reports bad ids
    const float g = gates[r];
    float v[D];
#pragma unroll
    for (int c = 0; c < D; ++c) v[c] = xin[c];
    // B(theta_e)^T: stages L-1 .. 0, each rotation by the negated angle.
#pragma unroll
    for (int s = L - 1; s >= 0; --s) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int i = ((p >> s) << (s + 1)) | (p & ((1 << s) - 1)), i2 = i + (1 << s);
        const float2 cs = cs_in[((size_t)e * L + s) * P + p];
        const float a = v[i], b = v[i2];
        v[i] = cs.x * a + cs.y * b;
        v[i2] = cs.x * b - cs.y * a;
      }
    }
    float z[D];
#pragma unroll
    for (int c = 0; c < D; ++c) z[c] = round_act<T>(v[c]);
    // H = alpha W_base z, fp32, ascending column.
#pragma unroll
    for (int o = 0; o < D; ++o) {
      float h = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) h = fmaf(w[o][c], z[c], h);
      v[o] = alpha * h;
    }
    // B(phi_e): stages 0 .. L-1.
#pragma unroll
    for (int s = 0; s < L; ++s) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int i = ((p >> s) << (s + 1)) | (p & ((1 << s) - 1)), i2 = i + (1 << s);
        const float2 cs = cs_out[((size_t)e * L + s) * P + p];
        const float a = v[i], b = v[i2];
        v[i] = cs.x * a - cs.y * b;
        v[i2] = cs.y * a + cs.x * b;
      }
    }
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] += round_act<T>(g * v[c]);
  }
#pragma unroll
  for (int c = 0; c < D; ++c) {
    if constexpr (sizeof(T) == 2)
      reinterpret_cast<uint16_t*>(y)[(size_t)t * D + c] = (uint16_t)f32_to_bf16_bits(acc[c]);
    else
      y[(size_t)t * D + c] = acc[c];
  }
}

template <typename T>
hipError_t launch_small_t(int T_, int d, int k, int N, const void* x, const int32_t* ids,
                          const float* gates, const float2* cs_in, const float2* cs_out,
                          const uint32_t* w_packed, float alpha, void* y, hipStream_t s,
                          const KernelTiming& t) {
  const dim3 grid((T_ + kThreads - 1) / kThreads), block(kThreads);
  const T* xt = static_cast<const T*>(x);
  T* yt = static_cast<T*>(y);
  switch (d) {
    case 2:
      return launch_kernel(small_kernel<T, 2>, grid, block, 0, s, t, xt, ids, gates, cs_in, cs_out,
                           w_packed, alpha, yt, T_, k, N);
    case 4:
      return launch_kernel(small_kernel<T, 4>, grid, block, 0, s, t, xt, ids, gates, cs_in, cs_out,
                           w_packed, alpha, yt, T_, k, N);
    case 8:
      return launch_kernel(small_kernel<T, 8>, grid, block, 0, s, t, xt, ids, gates, cs_in, cs_out,
                           w_packed, alpha, yt, T_, k, N);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_small(bmoe_dtype dt, int T, int d, int k, int N, const void* x,
                        const int32_t* ids, const float* gates, const float2* cs_in,
                        const float2* cs_out, const uint32_t* w_packed, float alpha, void* y,
                        hipStream_t s, const KernelTiming& t) {
  if (dt == BMOE_BF16)
    return launch_small_t<uint16_t>(T, d, k, N, x, ids, gates, cs_in, cs_out, w_packed, alpha, y,
                                    s, t);
  return launch_small_t<float>(T, d, k, N, x, ids, gates, cs_in, cs_out, w_packed, alpha, y, s,
                               t);
}

}  // namespace bmoe
