// Butterfly rotations of routed rows (ButterflyMoE gist.science summary,
// §2.1 and §2.3): input side z = B(theta_e)^T x, output side u = B(phi_e) h.
//
// B = S_{L-1} ... S_0; stage s rotates pairs (i, i + 2^s). B^T applies
// S_{L-1}^T first with each angle negated; B applies S_0 first.
//
// One workgroup owns R consecutive sorted rows (grouped by expert). The rows
// sit in LDS as fp32. Stages are taken in register blocks of up to three:
// a thread loads the 2^g elements of one block (indices that differ only in
// the g stage bits), rotates them through the g stages in registers and
// writes them back, so each element crosses LDS once per three stages. A
// thread loads the cos/sin of its block once per run of rows that share an
// expert and reuses them for every row of the run.
#include "common.h"
#include "kernels.h"

namespace bmoe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxRows = 64;

struct BflyParams {
  int M, d, L, k, R;
  const int32_t* perm;
  const int32_t* slot_e;
  const void* src;
  void* dst;
  const float2* cs;     // [N][L][d/2] (cos, sin)
  const float* gates;   // output side only, [M] in routed order
};

// Rotate the 2^G register values of one block through its G stages.
// TRANSPOSE: stages descending, rotation by -angle.
template <int G, bool TRANSPOSE>
__device__ __forceinline__ void rotate_block(float (&v)[8], const float2 (&c)[3][4]) {
#pragma unroll
  for (int tt = 0; tt < G; ++tt) {
    const int t = TRANSPOSE ? G - 1 - tt : tt;
#pragma unroll
    for (int u = 0; u < (1 << (G - 1)); ++u) {
      const int m = ((u >> t) << (t + 1)) | (u & ((1 << t) - 1));
      const int n = m + (1 << t);
      const float a = v[m], b = v[n];
      const float cc = c[t][u].x, ss = c[t][u].y;
      if (TRANSPOSE) {
        v[m] = cc * a + ss * b;
        v[n] = cc * b - ss * a;
      } else {
        v[m] = cc * a - ss * b;
        v[n] = ss * a + cc * b;
      }
    }
  }
}

template <int G, bool TRANSPOSE>
__device__ void apply_group(float* rows, int d, int L, int s_lo, const float2* cs,
                            const int* sh_e, const int* run_start, int nruns) {
  const int nb = d >> G;
  const int half = d >> 1;
  for (int b = threadIdx.x; b < nb; b += kThreads) {
    const int base = block_base(b, s_lo, G);
    for (int run = 0; run < nruns; ++run) {
      const int i0 = run_start[run], i1 = run_start[run + 1];
      const int e = sh_e[i0];
      float2 c[3][4];
#pragma unroll
      for (int t = 0; t < G; ++t) {
        const int s = s_lo + t;
        const float2* tab = cs + ((size_t)e * L + s) * half;
#pragma unroll
        for (int u = 0; u < (1 << (G - 1)); ++u) {
          const int m = ((u >> t) << (t + 1)) | (u & ((1 << t) - 1));
          c[t][u] = tab[pair_index(base + (m << s_lo), s)];
        }
      }
      for (int i = i0; i < i1; ++i) {
        float* row = rows + (size_t)i * d + base;
        float v[8];
#pragma unroll
        for (int m = 0; m < (1 << G); ++m) v[m] = row[m << s_lo];
        rotate_block<G, TRANSPOSE>(v, c);
#pragma unroll
        for (int m = 0; m < (1 << G); ++m) row[m << s_lo] = v[m];
      }
    }
  }
}

template <bool TRANSPOSE>
__device__ void apply_all_stages(float* rows, int d, int L, const float2* cs, const int* sh_e,
                                 const int* run_start, int nruns) {
  // Input side walks the stages from L-1 down, output side from 0 up; both
  // in blocks of three.
  int done = 0;
  while (done < L) {
    const int g = min(3, L - done);
    const int s_lo = TRANSPOSE ? L - done - g : done;
    if (g == 3)
      apply_group<3, TRANSPOSE>(rows, d, L, s_lo, cs, sh_e, run_start, nruns);
    else if (g == 2)
      apply_group<2, TRANSPOSE>(rows, d, L, s_lo, cs, sh_e, run_start, nruns);
    else
      apply_group<1, TRANSPOSE>(rows, d, L, s_lo, cs, sh_e, run_start, nruns);
    done += g;
    __syncthreads();
  }
}

__device__ __forceinline__ void load_vec8(const uint16_t* src, float* dst) {
  const uint4 v = *reinterpret_cast<const uint4*>(src);
  dst[0] = bf16_lo(v.x); dst[1] = bf16_hi(v.x);
  dst[2] = bf16_lo(v.y); dst[3] = bf16_hi(v.y);
  dst[4] = bf16_lo(v.z); dst[5] = bf16_hi(v.z);
  dst[6] = bf16_lo(v.w); dst[7] = bf16_hi(v.w);
}

// Shared prologue: row metadata and runs of equal experts.
__device__ int setup_rows(const BflyParams& p, int q0, int nr, int* sh_e, int* sh_r,
                          int* run_start) {
  __shared__ int nruns_sh;
  if ((int)threadIdx.x < nr) {
    sh_e[threadIdx.x] = p.slot_e[q0 + threadIdx.x];
    sh_r[threadIdx.x] = p.perm[q0 + threadIdx.x];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    run_start[n++] = 0;
    for (int i = 1; i < nr; ++i)
      if (sh_e[i] != sh_e[i - 1]) run_start[n++] = i;
    run_start[n] = nr;
    nruns_sh = n;
  }
  __syncthreads();
  return nruns_sh;
}

// z[q] = B(theta_e)^T x[perm[q] / k]
template <typename XT>
__global__ __launch_bounds__(kThreads) void bfly_in_kernel(BflyParams p) {
  extern __shared__ float rows[];
  __shared__ int sh_e[kMaxRows], sh_r[kMaxRows], run_start[kMaxRows + 1];
  const int q0 = blockIdx.x * p.R;
  const int nr = min(p.R, p.M - q0);
  const int d = p.d;
  const int nruns = setup_rows(p, q0, nr, sh_e, sh_r, run_start);

  constexpr int VEC = 16 / sizeof(XT);
  const int chunks = d / VEC;
  for (int c = threadIdx.x; c < nr * chunks; c += kThreads) {
    const int i = c / chunks, off = (c % chunks) * VEC;
    const size_t t = (size_t)(sh_r[i] / p.k);
    float* dst = rows + (size_t)i * d + off;
    if constexpr (sizeof(XT) == 2) {
      load_vec8(static_cast<const uint16_t*>(p.src) + t * d + off, dst);
    } else {
      *reinterpret_cast<float4*>(dst) =
          *reinterpret_cast<const float4*>(static_cast<const float*>(p.src) + t * d + off);
    }
  }
  __syncthreads();

  apply_all_stages<true>(rows, d, p.L, p.cs, sh_e, run_start, nruns);

  for (int c = threadIdx.x; c < nr * chunks; c += kThreads) {
    const int i = c / chunks, off = (c % chunks) * VEC;
    const float* s = rows + (size_t)i * d + off;
    const size_t q = (size_t)(q0 + i);
    if constexpr (sizeof(XT) == 2) {
      uint4 v;
      v.x = pack_bf16x2(s[0], s[1]);
      v.y = pack_bf16x2(s[2], s[3]);
      v.z = pack_bf16x2(s[4], s[5]);
      v.w = pack_bf16x2(s[6], s[7]);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.dst) + q * d + off) = v;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(p.dst) + q * d + off) =
          *reinterpret_cast<const float4*>(s);
    }
  }
}

// u[r] = g_r * B(phi_e) h[q], r = perm[q]
__global__ __launch_bounds__(kThreads) void bfly_out_kernel(BflyParams p) {
  extern __shared__ float rows[];
  __shared__ int sh_e[kMaxRows], sh_r[kMaxRows], run_start[kMaxRows + 1];
  const int q0 = blockIdx.x * p.R;
  const int nr = min(p.R, p.M - q0);
  const int d = p.d;
  const int nruns = setup_rows(p, q0, nr, sh_e, sh_r, run_start);

  const int chunks = d / 4;
  const float* h = static_cast<const float*>(p.src);
  for (int c = threadIdx.x; c < nr * chunks; c += kThreads) {
    const int i = c / chunks, off = (c % chunks) * 4;
    *reinterpret_cast<float4*>(rows + (size_t)i * d + off) =
        *reinterpret_cast<const float4*>(h + (size_t)(q0 + i) * d + off);
  }
  __syncthreads();

  apply_all_stages<false>(rows, d, p.L, p.cs, sh_e, run_start, nruns);

  float* u = static_cast<float*>(p.dst);
  for (int c = threadIdx.x; c < nr * chunks; c += kThreads) {
    const int i = c / chunks, off = (c % chunks) * 4;
    const int r = sh_r[i];
    const float g = p.gates[r];
    float4 v = *reinterpret_cast<const float4*>(rows + (size_t)i * d + off);
    v.x *= g; v.y *= g; v.z *= g; v.w *= g;
    *reinterpret_cast<float4*>(u + (size_t)r * d + off) = v;
  }
}

int pick_rows(int M, int d) {
  int R = 32768 / d;  // R * d * 4 bytes <= 128 KiB of LDS
  if (R > kMaxRows) R = kMaxRows;
  if (R < 1) R = 1;
  while (R > 4 && (M + R - 1) / R < 512) R >>= 1;
  return R;
}

template <typename K>
hipError_t launch_rows(K kernel, const BflyParams& p, hipStream_t s) {
  const size_t shmem = (size_t)p.R * p.d * sizeof(float);
  if (shmem > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kernel, dim3((p.M + p.R - 1) / p.R), dim3(kThreads), shmem, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bfly_in(bmoe_dtype dt, int M, int d, int k, const void* x,
                          const RouteTables& rt, const float2* cs_in, void* z, hipStream_t s) {
  BflyParams p{};
  p.M = M; p.d = d; p.k = k;
  p.L = 0;
  while ((1 << p.L) < d) ++p.L;
  p.R = pick_rows(M, d);
  p.perm = rt.perm; p.slot_e = rt.slot_e;
  p.src = x; p.dst = z; p.cs = cs_in; p.gates = nullptr;
  if (dt == BMOE_BF16) return launch_rows(bfly_in_kernel<uint16_t>, p, s);
  return launch_rows(bfly_in_kernel<float>, p, s);
}

hipError_t launch_bfly_out(int M, int d, const float* h, const float* gates,
                           const RouteTables& rt, const float2* cs_out, float* u,
                           hipStream_t s) {
  BflyParams p{};
  p.M = M; p.d = d; p.k = 1;
  p.L = 0;
  while ((1 << p.L) < d) ++p.L;
  p.R = pick_rows(M, d);
  p.perm = rt.perm; p.slot_e = rt.slot_e;
  p.src = h; p.dst = u; p.cs = cs_out; p.gates = gates;
  return launch_rows(bfly_out_kernel, p, s);
}

}  // namespace bmoe
