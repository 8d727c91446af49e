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
// expert and reuses them for every row of that run it handles.
#include "common.h"
#include "kernels.h"

namespace bmoe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxRows = 64;

// LDS row layout: one pad float after every 8, so the register blocks of
// every stage group (8 contiguous values, or 8 values 8 apart, across 64
// lanes) fall on distinct banks.
__device__ __forceinline__ int pad(int i) { return i + (i >> 3); }
__host__ __device__ constexpr int padded_row(int d) { return d + d / 8; }

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
  // Threads per block (when a row has fewer blocks than threads) share the
  // rows of each run round-robin.
  const int tpb = nb >= kThreads ? 1 : kThreads / nb;
  const int ph = threadIdx.x / (kThreads / tpb) ;
  const int bstart = threadIdx.x % (kThreads / tpb);
  const int bstride = kThreads / tpb;
  for (int b = bstart; b < nb; b += bstride) {
    const int base = block_base(b, s_lo, G);
    for (int run = 0; run < nruns; ++run) {
      const int i0 = run_start[run], i1 = run_start[run + 1];
      if (i0 + ph >= i1) continue;
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
      int off[1 << G];
#pragma unroll
      for (int m = 0; m < (1 << G); ++m) off[m] = pad(base + (m << s_lo));
      for (int i = i0 + ph; i < i1; i += tpb) {
        float* row = rows + (size_t)i * padded_row(d);
        float v[8];
#pragma unroll
        for (int m = 0; m < (1 << G); ++m) v[m] = row[off[m]];
        rotate_block<G, TRANSPOSE>(v, c);
#pragma unroll
        for (int m = 0; m < (1 << G); ++m) row[off[m]] = v[m];
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

// 16 bytes of a row (8 bf16 or 4 fp32) to fp32 in LDS.
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

// IN_SIDE:  dst[q] = B(theta_e)^T x[perm[q] / k]          (sorted order)
// OUT_SIDE: dst[perm[q]] = g_{perm[q]} * B(phi_e) src[q]   (routed order)
template <bool IN_SIDE, typename SrcT, typename DstT>
__global__ __launch_bounds__(kThreads) void bfly_kernel(BflyParams p) {
  extern __shared__ float rows[];
  __shared__ int sh_e[kMaxRows], sh_r[kMaxRows], run_start[kMaxRows + 1];
  const int q0 = blockIdx.x * p.R;
  const int nr = min(p.R, p.M - q0);
  const int d = p.d;
  const int nruns = setup_rows(p, q0, nr, sh_e, sh_r, run_start);

  constexpr int VS = 16 / sizeof(SrcT);
  const int cs_ = d / VS;
  const SrcT* src = static_cast<const SrcT*>(p.src);
  for (int c = threadIdx.x; c < nr * cs_; c += kThreads) {
    const int i = c / cs_, off = (c % cs_) * VS;
    const size_t srow = IN_SIDE ? (size_t)(sh_r[i] / p.k) : (size_t)(q0 + i);
    load16<SrcT>(src + srow * d + off, rows + (size_t)i * padded_row(d) + pad(off));
  }
  __syncthreads();

  apply_all_stages<IN_SIDE>(rows, d, p.L, p.cs, sh_e, run_start, nruns);

  constexpr int VD = 16 / sizeof(DstT);
  const int cd = d / VD;
  DstT* dst = static_cast<DstT*>(p.dst);
  for (int c = threadIdx.x; c < nr * cd; c += kThreads) {
    const int i = c / cd, off = (c % cd) * VD;
    if (IN_SIDE) {
      store16<DstT>(rows + (size_t)i * padded_row(d) + pad(off), dst + (size_t)(q0 + i) * d + off, 1.0f);
    } else {
      const int r = sh_r[i];
      store16<DstT>(rows + (size_t)i * padded_row(d) + pad(off), dst + (size_t)r * d + off, p.gates[r]);
    }
  }
}

int pick_rows(int M, int d) {
  int R = 16384 / d;  // R * d * 4 bytes <= 64 KiB of LDS: two workgroups per CU
  if (R > kMaxRows) R = kMaxRows;
  if (R < 1) R = 1;
  while (R > 4 && (M + R - 1) / R < 512) R >>= 1;
  return R;
}

template <typename K>
hipError_t launch_rows(K kernel, const BflyParams& p, hipStream_t s) {
  const size_t shmem = (size_t)p.R * padded_row(p.d) * sizeof(float);
  if (shmem > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kernel, dim3((p.M + p.R - 1) / p.R), dim3(kThreads), shmem, s, p);
  return hipGetLastError();
}

BflyParams make_params(int M, int d, int k, const RouteTables& rt, const float2* cs,
                       const void* src, void* dst, const float* gates) {
  BflyParams p{};
  p.M = M; p.d = d; p.k = k;
  p.L = 0;
  while ((1 << p.L) < d) ++p.L;
  p.R = pick_rows(M, d);
  p.perm = rt.perm; p.slot_e = rt.slot_e;
  p.src = src; p.dst = dst; p.cs = cs; p.gates = gates;
  return p;
}

}  // namespace

hipError_t launch_bfly_in(bmoe_dtype dt, int M, int d, int k, const void* x,
                          const RouteTables& rt, const float2* cs_in, void* z, hipStream_t s) {
  const BflyParams p = make_params(M, d, k, rt, cs_in, x, z, nullptr);
  if (dt == BMOE_BF16) return launch_rows(bfly_kernel<true, uint16_t, uint16_t>, p, s);
  return launch_rows(bfly_kernel<true, float, float>, p, s);
}

hipError_t launch_bfly_out(bmoe_dtype dt, int M, int d, const void* h, const float* gates,
                           const RouteTables& rt, const float2* cs_out, void* u,
                           hipStream_t s) {
  const BflyParams p = make_params(M, d, 1, rt, cs_out, h, u, gates);
  if (dt == BMOE_BF16) return launch_rows(bfly_kernel<false, uint16_t, uint16_t>, p, s);
  return launch_rows(bfly_kernel<false, float, float>, p, s);
}

}  // namespace bmoe
