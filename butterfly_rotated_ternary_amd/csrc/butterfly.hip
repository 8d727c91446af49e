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
  int routed_out;       // input side: write row r = perm[q] instead of q
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

// IN_SIDE:  dst[q] = B(theta_e)^T x[perm[q] / k]          (sorted order, or
//           dst[perm[q]] with routed_out)
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
      const size_t row = p.routed_out ? (size_t)sh_r[i] : (size_t)(q0 + i);
      store16<DstT>(rows + (size_t)i * padded_row(d) + pad(off), dst + row * d + off, 1.0f);
    } else {
      const int r = sh_r[i];
      store16<DstT>(rows + (size_t)i * padded_row(d) + pad(off), dst + (size_t)r * d + off, p.gates[r]);
    }
  }
}

// ---------------------------------------------------------------------------
// Large-d kernel (bf16, d >= 1024): 8 waves, R rows per workgroup with R*d
// fp32 (padded) filling ~144 KiB of LDS, so each coefficient a thread loads
// serves R rows. Every stage group's coefficients are requested in one round
// trip up front; rows are rotated four at a time while they share an expert.
constexpr int kBigThreads = 512;

// Two workgroups per CU: R fp32 rows each (at most 74 KiB of LDS; 16 or 32
// rows at d = 256 and 512 keep two or more tiles per CU) and at most 128
// registers per lane (four waves per SIMD), so one workgroup's row loads and
// stores overlap the other's rotations. A thread holds the coefficients of
// the group it rotates and of the next one (fetched during the current one).
template <int D>
struct BigCfg {
  static_assert(D >= 256 && D <= 4096, "large-d kernel sizes");
  static constexpr int L = D == 256 ? 8 : D == 512 ? 9 : D == 1024 ? 10 : D == 2048 ? 11 : 12;
  static constexpr int PD = D + D / 8;
  static constexpr int R = D == 256 ? 32 : D == 512 ? 16 : D == 1024 ? 16 : D == 2048 ? 8 : 4;
  static constexpr int NG = (L + 2) / 3;
  static_assert(R * PD * 4 <= 80 * 1024, "two workgroups per CU");
};

template <int D, bool TR>
struct BigGroups {
  static constexpr int L = BigCfg<D>::L;
  static constexpr int s_hi(int g) { return TR ? L - 1 - 3 * g : (3 * g + 2 < L ? 3 * g + 2 : L - 1); }
  static constexpr int s_lo(int g) { return TR ? (L - 3 - 3 * g > 0 ? L - 3 - 3 * g : 0) : 3 * g; }
  static constexpr int G(int g) { return s_hi(g) - s_lo(g) + 1; }
  // Blocks of 2^G elements per row; at these sizes there are at most as many
  // blocks as threads, so each thread owns one block and TPB threads share it
  // (each taking every TPB-th row).
  static constexpr int NB(int g) { return D >> G(g); }
  static constexpr int TPB(int g) { return kBigThreads / NB(g); }
  static constexpr bool fits() {
    for (int g = 0; g < BigCfg<D>::NG; ++g)
      if (NB(g) > kBigThreads) return false;
    return true;
  }
};

template <int D, int G>
__device__ __forceinline__ void big_coef(float2 (&c)[3][4], const float2* cs, int e, int s_lo,
                                         int base) {
  constexpr int L = BigCfg<D>::L;
#pragma unroll
  for (int t = 0; t < G; ++t) {
    const int s = s_lo + t;
    const float2* tab = cs + ((size_t)e * L + s) * (D / 2);
#pragma unroll
    for (int u = 0; u < (1 << (G - 1)); ++u) {
      const int m = ((u >> t) << (t + 1)) | (u & ((1 << t) - 1));
      c[t][u] = tab[pair_index(base + (m << s_lo), s)];
    }
  }
}

// One group, one block: rotate this thread's rows [ph, ph+tpb, ...) of the
// tile; coefficients c are valid for expert ce (reloaded when a row differs).
template <int D, int G, bool TR>
__device__ __forceinline__ void big_rows(float* rows, const int* sh_e, int nrows, const float2* cs,
                                         float2 (&c)[3][4], int& ce, int s_lo, int base, int ph,
                                         int tpb) {
  constexpr int PD = BigCfg<D>::PD;
  int off[8];
#pragma unroll
  for (int m = 0; m < (1 << G); ++m) off[m] = pad(base + (m << s_lo));
  const int rpt = (nrows - ph + tpb - 1) / tpb;  // rows of this thread
  const int last = ph + (rpt - 1) * tpb;
  if (rpt > 0 && sh_e[ph] == ce && sh_e[last] == ce) {
    for (int j0 = 0; j0 < rpt; j0 += 4) {
      float v[4][8];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (j0 + q < rpt) {
          const float* row = rows + (ph + (j0 + q) * tpb) * PD;
#pragma unroll
          for (int m = 0; m < (1 << G); ++m) v[q][m] = row[off[m]];
        }
#pragma unroll
      for (int q = 0; q < 4; ++q) rotate_block<G, TR>(v[q], c);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (j0 + q < rpt) {
          float* row = rows + (ph + (j0 + q) * tpb) * PD;
#pragma unroll
          for (int m = 0; m < (1 << G); ++m) row[off[m]] = v[q][m];
        }
    }
    return;
  }
  for (int j = 0; j < rpt; ++j) {
    const int i = ph + j * tpb;
    if (sh_e[i] != ce) {
      ce = sh_e[i];
      big_coef<D, G>(c, cs, ce, s_lo, base);
    }
    float* row = rows + i * PD;
    float v[8];
#pragma unroll
    for (int m = 0; m < (1 << G); ++m) v[m] = row[off[m]];
    rotate_block<G, TR>(v, c);
#pragma unroll
    for (int m = 0; m < (1 << G); ++m) row[off[m]] = v[m];
  }
}

// Group g's coefficients for the expert of this thread's first row in that
// group (lane l < R of each wave holds row l's expert in my_e).
template <int D, bool IN_SIDE, int g>
__device__ __forceinline__ void big_group_coef(float2 (&c)[3][4], int& ce, const float2* cs,
                                               int my_e, int tid) {
  using Gr = BigGroups<D, IN_SIDE>;
  constexpr int G = Gr::G(g), NB = Gr::NB(g);
  const int base = block_base(tid % NB, Gr::s_lo(g), G);
  ce = __shfl(my_e, tid / NB, 64);
  big_coef<D, G>(c, cs, ce, Gr::s_lo(g), base);
}

// Groups g.. in application order, a barrier after each; group g+1's
// coefficients are requested before group g's rotations.
template <int D, bool IN_SIDE, int g>
__device__ __forceinline__ void big_groups(float* rows, const int* sh_e, const float2* cs,
                                           float2 (&coef)[2][3][4], int (&ce)[2], int my_e,
                                           int tid) {
  using Gr = BigGroups<D, IN_SIDE>;
  if constexpr (g < BigCfg<D>::NG) {
    if constexpr (g + 1 < BigCfg<D>::NG)
      big_group_coef<D, IN_SIDE, g + 1>(coef[(g + 1) & 1], ce[(g + 1) & 1], cs, my_e, tid);
    constexpr int G = Gr::G(g), NB = Gr::NB(g);
    const int base = block_base(tid % NB, Gr::s_lo(g), G);
    big_rows<D, G, IN_SIDE>(rows, sh_e, BigCfg<D>::R, cs, coef[g & 1], ce[g & 1], Gr::s_lo(g),
                            base, tid / NB, Gr::TPB(g));
    __syncthreads();
    big_groups<D, IN_SIDE, g + 1>(rows, sh_e, cs, coef, ce, my_e, tid);
  }
}

// IN_SIDE:  z[q] = B(theta_e)^T x[perm[q] / k]          (sorted order)
// OUT_SIDE: u[perm[q]] = g * B(phi_e) h[q]               (routed order)
template <int D, bool IN_SIDE>
__global__ __launch_bounds__(kBigThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void bfly_big_kernel(BflyParams p) {
  using C = BigCfg<D>;
  constexpr int PD = C::PD, R = C::R;
  extern __shared__ float rows[];
  __shared__ int sh_e[R], sh_r[R];
  const int tid = threadIdx.x, lane = tid % kWave;
  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a
  // contiguous run of tiles so an expert's coefficient tables are fetched
  // into one or two XCD L2s rather than all eight.
  const int nb = gridDim.x, xcd = blockIdx.x % 8, per = nb / 8, extra = nb % 8;
  const int tile = xcd * per + min(xcd, extra) + blockIdx.x / 8;
  const int q0 = tile * R;
  const int nr = min(R, p.M - q0);

  // Row metadata: lane l (< R) of every wave holds row l's (expert, routed
  // index); rows past nr repeat the last row (computed, never stored).
  const int qm = q0 + min(lane % R, nr - 1);
  const int my_e = p.slot_e[qm];
  const int my_r = p.perm[qm];
  const int my_src = IN_SIDE ? my_r / p.k : qm;
  if (tid < R) {
    sh_e[tid] = my_e;
    sh_r[tid] = my_r;
  }

  // Source rows: 16-byte chunks (8 bf16) into registers.
  constexpr int CPR = D / 8;
  constexpr int LPT = R * CPR / kBigThreads;
  uint4 xv[LPT];
  const uint16_t* src = static_cast<const uint16_t*>(p.src);
#pragma unroll
  for (int it = 0; it < LPT; ++it) {
    const int c = tid + it * kBigThreads;
    const int i = c / CPR, ch = c % CPR;
    const int sr = __shfl(my_src, i, 64);
    xv[it] = *reinterpret_cast<const uint4*>(src + (size_t)sr * D + ch * 8);
  }
  // Coefficients of group 0 for the expert of the thread's first row.
  float2 coef[2][3][4];
  int ce[2];
  big_group_coef<D, IN_SIDE, 0>(coef[0], ce[0], p.cs, my_e, tid);
#pragma unroll
  for (int it = 0; it < LPT; ++it) {
    const int c = tid + it * kBigThreads;
    const int i = c / CPR, ch = c % CPR;
    float* dst = rows + i * PD + pad(ch * 8);
    const uint4 v = xv[it];
    dst[0] = bf16_lo(v.x); dst[1] = bf16_hi(v.x); dst[2] = bf16_lo(v.y); dst[3] = bf16_hi(v.y);
    dst[4] = bf16_lo(v.z); dst[5] = bf16_hi(v.z); dst[6] = bf16_lo(v.w); dst[7] = bf16_hi(v.w);
  }
  __syncthreads();

  big_groups<D, IN_SIDE, 0>(rows, sh_e, p.cs, coef, ce, my_e, tid);

  uint16_t* dst = static_cast<uint16_t*>(p.dst);
#pragma unroll
  for (int it = 0; it < LPT; ++it) {
    const int c = tid + it * kBigThreads;
    const int i = c / CPR, ch = c % CPR;
    if (i < nr) {
      const float* s = rows + i * PD + pad(ch * 8);
      if (IN_SIDE) {
        const size_t row = p.routed_out ? (size_t)sh_r[i] : (size_t)(q0 + i);
        store16<uint16_t>(s, dst + row * D + ch * 8, 1.0f);
      } else {
        const int r = sh_r[i];
        store16<uint16_t>(s, dst + (size_t)r * D + ch * 8, p.gates[r]);
      }
    }
  }
}

template <int D, bool IN_SIDE>
hipError_t launch_big(const BflyParams& p, hipStream_t s, const KernelTiming& t) {
  using C = BigCfg<D>;
  static_assert(BigGroups<D, IN_SIDE>::fits(), "one block per thread");
  const size_t shmem = (size_t)C::R * C::PD * sizeof(float);
  auto kern = bfly_big_kernel<D, IN_SIDE>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
  if (e != hipSuccess) return e;
  return launch_kernel(kern, dim3((p.M + C::R - 1) / C::R), dim3(kBigThreads), (uint32_t)shmem, s,
                       t, p);
}

template <bool IN_SIDE>
hipError_t launch_big_d(const BflyParams& p, hipStream_t s, const KernelTiming& t) {
  switch (p.d) {
    case 256: return launch_big<256, IN_SIDE>(p, s, t);
    case 512: return launch_big<512, IN_SIDE>(p, s, t);
    case 1024: return launch_big<1024, IN_SIDE>(p, s, t);
    case 2048: return launch_big<2048, IN_SIDE>(p, s, t);
    case 4096: return launch_big<4096, IN_SIDE>(p, s, t);
  }
  return hipErrorInvalidValue;
}

int pick_rows(int M, int d) {
  int R = 16384 / d;  // R * d * 4 bytes <= 64 KiB of LDS: two workgroups per CU
  if (R > kMaxRows) R = kMaxRows;
  if (R < 1) R = 1;
  while (R > 4 && (M + R - 1) / R < 512) R >>= 1;
  return R;
}

template <typename K>
hipError_t launch_rows(K kernel, const BflyParams& p, hipStream_t s, const KernelTiming& t) {
  const size_t shmem = (size_t)p.R * padded_row(p.d) * sizeof(float);
  if (shmem > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  return launch_kernel(kernel, dim3((p.M + p.R - 1) / p.R), dim3(kThreads), (uint32_t)shmem, s, t,
                       p);
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
                          const RouteTables& rt, const float2* cs_in, void* z, hipStream_t s,
                          const KernelTiming& t, bool routed_out) {
  if (bfly_wave_supported(dt, d))
    return launch_bfly_wave(true, M, d, k, rt, cs_in, x, z, nullptr, routed_out, s, t);
  BflyParams p = make_params(M, d, k, rt, cs_in, x, z, nullptr);
  p.routed_out = routed_out ? 1 : 0;
  if (dt == BMOE_BF16 && d >= 256 && d <= 4096) return launch_big_d<true>(p, s, t);
  if (dt == BMOE_BF16) return launch_rows(bfly_kernel<true, uint16_t, uint16_t>, p, s, t);
  return launch_rows(bfly_kernel<true, float, float>, p, s, t);
}

hipError_t launch_bfly_out(bmoe_dtype dt, int M, int d, const void* h, const float* gates,
                           const RouteTables& rt, const float2* cs_out, void* u,
                           hipStream_t s, const KernelTiming& t) {
  if (bfly_wave_supported(dt, d))
    return launch_bfly_wave(false, M, d, 1, rt, cs_out, h, u, gates, false, s, t);
  const BflyParams p = make_params(M, d, 1, rt, cs_out, h, u, gates);
  if (dt == BMOE_BF16 && d >= 256 && d <= 4096) return launch_big_d<false>(p, s, t);
  if (dt == BMOE_BF16) return launch_rows(bfly_kernel<false, uint16_t, uint16_t>, p, s, t);
  return launch_rows(bfly_kernel<false, float, float>, p, s, t);
}

}  // namespace bmoe
