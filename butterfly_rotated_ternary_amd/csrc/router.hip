// Router in front of the expert layer: logits = x W_r^T, top-k experts per
// token, softmax gates over the k chosen logits. The pages describe the layer
// as a top-k mixture of experts (ButterflyMoE abstract; gist.science summary,
// §2.3) without a router formula; this is the usual top-k gate, with its
// readings stated in the C header.
//
//   logits[t][e] = sum_c x[t][c] * w_r[e][c]          (fp32 accumulation)
//   ids[t][0..k)  = experts by descending logit, ties to the lower id
//   gates[t][j]   = exp(l_j - l_0) / sum_i exp(l_i - l_0)
#include "common.h"
#include "kernels.h"

namespace bmoe {
namespace {

// ---- logits, bf16: MFMA --------------------------------------------------------
// 64 tokens x 64 experts per workgroup; wave w owns the 32 x 32 fragment
// (w >> 1, w & 1). Lane l feeds row / column l & 31 and a contiguous run of
// KC / 2 values of k (the half l >> 5 of each KC-wide chunk): the order of
// the k terms inside one dot product is free as long as A and B agree.
template <int KC>
__global__ __launch_bounds__(256) void logits_mfma_kernel(const uint16_t* x, const uint16_t* w,
                                                          int T, int d, int N, float* logits) {
  constexpr int NU = KC / 16;  // 16-byte loads (and MFMAs) per lane per chunk
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 64 + (wave >> 1) * 32, e0 = blockIdx.y * 64 + (wave & 1) * 32;
  const int row = lane & 31, half = lane >> 5;
  const int t = min(t0 + row, T - 1);
  const int e = e0 + row;
  const bool e_ok = e < N;
  const uint4* xa = reinterpret_cast<const uint4*>(x + (size_t)t * d + half * (KC / 2));
  const uint4* wb = reinterpret_cast<const uint4*>(w + (size_t)(e_ok ? e : 0) * d + half * (KC / 2));
  const int steps = d / KC;
  f32x16 acc = {};
  uint4 a[NU], b[NU], na[NU], nb[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    a[u] = xa[u];
    b[u] = e_ok ? wb[u] : make_uint4(0, 0, 0, 0);
  }
  for (int s = 0; s < steps; ++s) {
    if (s + 1 < steps) {
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        na[u] = xa[(s + 1) * (KC / 8) + u];
        nb[u] = e_ok ? wb[(s + 1) * (KC / 8) + u] : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < NU; ++u)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[u]),
                                                    __builtin_bit_cast(bf16x8, b[u]), acc, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      a[u] = na[u];
      b[u] = nb[u];
    }
  }
  if (!e_ok) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int tt = t0 + 8 * (r >> 2) + 4 * half + (r & 3);
    if (tt < T) logits[(size_t)tt * N + e] = acc[r];
  }
}

// ---- logits, fp32: FMA ---------------------------------------------------------
// 64 x 64 outputs per workgroup, 4 x 4 per thread, k in chunks of 32 via LDS.
__global__ __launch_bounds__(256) void logits_f32_kernel(const float* x, const float* w, int T,
                                                         int d, int N, float* logits) {
  __shared__ float xs[32][65];
  __shared__ float ws_[32][65];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  const int kc = d < 32 ? d : 32;
  for (int k0 = 0; k0 < d; k0 += kc) {
    for (int u = tid; u < 64 * kc; u += 256) {
      const int r = u / kc, c = u % kc;
      const int tt = min(t0 + r, T - 1), ee = e0 + r;
      xs[c][r] = x[(size_t)tt * d + k0 + c];
      ws_[c][r] = ee < N ? w[(size_t)ee * d + k0 + c] : 0.f;
    }
    __syncthreads();
    for (int c = 0; c < kc; ++c) {
      float xv[4], wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xv[i] = xs[c][ty + 16 * i];
        wv[i] = ws_[c][tx + 16 * i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xv[i], wv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tt = t0 + ty + 16 * i, ee = e0 + tx + 16 * j;
      if (tt < T && ee < N) logits[(size_t)tt * N + ee] = acc[i][j];
    }
}

// ---- top-k + softmax -------------------------------------------------------------
// One wave per token. Lane l holds logits l, l + 64, ... (PER of them). Each
// round takes the wave's largest not-yet-chosen logit (ties to the lower id);
// pick j stays in lane j.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

template <int PER>
__global__ __launch_bounds__(256) void topk_kernel(const float* logits, int T, int N, int k,
                                                   int32_t* ids, float* gates) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave
  const float* lt = logits + (size_t)t * N;
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < N ? lt[e] : -INFINITY;
  }
  uint64_t taken = 0u;
  float mine_v = -INFINITY;
  int mine_i = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + 64 * i;
      if (e < N && !(taken >> i & 1u) && better(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1ull << (bi >> 6);
    if (lane == j) {
      mine_v = bv;
      mine_i = bi;
    }
  }
  const float top = __shfl(mine_v, 0, 64);
  const float ex = lane < k ? expf(mine_v - top) : 0.f;
  float sum = ex;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
  if (lane < k) {
    ids[(size_t)t * k + lane] = mine_i;
    gates[(size_t)t * k + lane] = ex / sum;
  }
}

template <int PER>
hipError_t launch_topk_per(const float* logits, int T, int N, int k, int32_t* ids, float* gates,
                           hipStream_t s, const KernelTiming& tm) {
  return launch_kernel(topk_kernel<PER>, dim3((T + 3) / 4), dim3(256), 0, s, tm, logits, T, N, k,
                       ids, gates);
}

}  // namespace

hipError_t launch_router_logits(bmoe_dtype dt, int T, int d, int N, const void* x,
                                const void* w, float* logits, hipStream_t s,
                                const KernelTiming& tm) {
  const dim3 grid((T + 63) / 64, (N + 63) / 64);
  if (dt == BMOE_F32)
    return launch_kernel(logits_f32_kernel, grid, dim3(256), 0, s, tm,
                         static_cast<const float*>(x), static_cast<const float*>(w), T, d, N,
                         logits);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* wb = static_cast<const uint16_t*>(w);
  if (d % 64 == 0)
    return launch_kernel(logits_mfma_kernel<64>, grid, dim3(256), 0, s, tm, xb, wb, T, d, N, logits);
  if (d % 32 == 0)
    return launch_kernel(logits_mfma_kernel<32>, grid, dim3(256), 0, s, tm, xb, wb, T, d, N, logits);
  return launch_kernel(logits_mfma_kernel<16>, grid, dim3(256), 0, s, tm, xb, wb, T, d, N, logits);
}

hipError_t launch_topk(const float* logits, int T, int N, int k, int32_t* ids, float* gates,
                       hipStream_t s, const KernelTiming& tm) {
  if (N <= 64) return launch_topk_per<1>(logits, T, N, k, ids, gates, s, tm);
  if (N <= 128) return launch_topk_per<2>(logits, T, N, k, ids, gates, s, tm);
  if (N <= 256) return launch_topk_per<4>(logits, T, N, k, ids, gates, s, tm);
  if (N <= 512) return launch_topk_per<8>(logits, T, N, k, ids, gates, s, tm);
  if (N <= 1024) return launch_topk_per<16>(logits, T, N, k, ids, gates, s, tm);
  if (N <= 2048) return launch_topk_per<32>(logits, T, N, k, ids, gates, s, tm);
  return launch_topk_per<64>(logits, T, N, k, ids, gates, s, tm);
}

}  // namespace bmoe
