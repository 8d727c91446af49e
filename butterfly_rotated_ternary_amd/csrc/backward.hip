// Backward of the ButterflyMoE expert layer (ButterflyMoE gist.science
// summary, §2.1/§2.3 for the map; training the rotations, §2.4). For a loss L
// with dy = dL/dy and a routed row r = t*k + j of expert e:
//
//   dg_r = <dy_t, u>          u  = B(phi_e) h,  h = alpha W_base z,  z = B(theta_e)^T x_t
//   dh   = B(phi_e)^T (g_r dy_t)      dphi_e += per-stage pair terms
//   dz   = alpha W_base^T dh          dW     += alpha dh z^T   (library GEMM)
//   dx_t = sum_j B(theta_e) dz        dtheta_e += per-stage pair terms
//
// A stage maps a pair (x_i, x_j) to (c x_i - s x_j, s x_i + c x_j). Written
// with its OUTPUT v and the gradient G of the output, the angle gradient is
// G_j v_i - G_i v_j and the input gradient and input are S^T G and S^T v.
// So the kernels below hold a few rows in LDS (fp32), run them forward
// through their butterfly, then walk the stages backward from the outputs: no
// per-stage activations are stored. On the input side each stage runs with
// angle -a, so its angle gradient changes sign and its inverse is S(a).
//
// Angle gradients are summed per expert without atomics: rows are cut into
// tiles of a few sorted rows of one expert, each tile keeps its sums in
// registers and writes one partial, and a second kernel adds an expert's
// partials in tile order (bit-reproducible).
#include "common.h"
#include "kernels.h"

namespace bmoe {
namespace {

__device__ __forceinline__ int pad(int i) { return i + (i >> 3); }

// ---- butterfly backward --------------------------------------------------------
// Stages are grouped three at a time as in the forward kernels: group g holds
// stages 3g .. min(3g + 3, L) - 1. A thread owns register blocks of a group
// (the 2^G elements whose indices differ only in the group's stage bits) for
// a fixed set of rows of the tile, so the angle gradients of its blocks'
// pairs sum in registers over those rows, and each element crosses LDS once
// per group and pass.
constexpr int bwd_rows(int d) { return d >= 4096 ? 2 : (8192 / d > 32 ? 32 : 8192 / d); }
// Rows per tile (a workgroup walks them bwd_rows at a time). At d = 256 and
// 512 (bf16: the register-resident kernel, four rows per wave) 16-row tiles
// spread the rows more evenly over the SIMDs than 32-row ones.
constexpr int bwd_tile_rows(int d) {
  return d >= 1024 ? 64 : (d == 256 || d == 512) ? 16 : bwd_rows(d);
}

template <int D>
struct BwdCfg {
  static_assert(D >= 16 && D <= 4096, "backward sizes");
  static constexpr int L = D == 16 ? 4 : D == 32 ? 5 : D == 64 ? 6 : D == 128 ? 7 : D == 256 ? 8
                         : D == 512 ? 9 : D == 1024 ? 10 : D == 2048 ? 11 : 12;
  static constexpr int NG = (L + 2) / 3;
  static constexpr int NTHR = D >= 4096 ? 512 : 256;
  static constexpr int R = bwd_rows(D);        // rows held in LDS at a time
  static constexpr int PD = D + D / 8;         // padded LDS row
  static constexpr int TPR = NTHR / R;         // threads per row (gate dot products)
  static constexpr int gsize(int g) { return L - 3 * g < 3 ? L - 3 * g : 3; }
  static constexpr int nblk(int g) { return D >> gsize(g); }
  // threads sharing a block (each takes every tpb-th row) and blocks per thread
  static constexpr int tpb(int g) { return nblk(g) >= NTHR ? 1 : NTHR / nblk(g); }
  static constexpr int slots(int g) { return nblk(g) >= NTHR ? nblk(g) / NTHR : 1; }
  static constexpr int npairs(int g) { return gsize(g) << (gsize(g) - 1); }
  static constexpr int VSZ = R * PD > 12 * NTHR ? R * PD : 12 * NTHR;
};

struct BwdParams {
  int M, k;
  const int4* tiles;
  const int32_t* perm;
  const float2* cs;     // [N][L][D/2] cos/sin of this side's angles
  const float* gates;
  const void* src;      // out side: H [M][D] (sorted); in side: x [T][D]
  const void* grad;     // out side: dy [T][D];          in side: dZ [M][D] (sorted)
  void* dst;            // out side: dH [M][D] (sorted); in side: dX [M][D] (routed)
  float* dgates;        // out side only
  float* partial;       // [tiles][L][D/2]
};

// Element offsets of pair u of stage t within a block of 2^G elements.
__device__ __forceinline__ int pair_lo(int t, int u) {
  return ((u >> t) << (t + 1)) | (u & ((1 << t) - 1));
}

template <int D, int G>
__device__ __forceinline__ void block_of(int g, int sl, int tid, int& base, int& ph) {
  using C = BwdCfg<D>;
  const int bstride = C::NTHR / C::tpb(g);
  ph = tid / bstride;
  base = block_base(tid % bstride + sl * bstride, 3 * g, G);
}

// Forward rotation of one register block through its stages (IN_SIDE: stages
// descending, each by -angle).
template <int G, bool IN_SIDE>
__device__ __forceinline__ void fwd_block(float (&v)[8], const float2 (&c)[12]) {
#pragma unroll
  for (int tt = 0; tt < G; ++tt) {
    const int t = IN_SIDE ? G - 1 - tt : tt;
#pragma unroll
    for (int u = 0; u < (1 << (G - 1)); ++u) {
      const int m = pair_lo(t, u), n = m + (1 << t);
      const float a = v[m], b = v[n], cc = c[t * 4 + u].x, ss = c[t * 4 + u].y;
      if (IN_SIDE) {
        v[m] = cc * a + ss * b;
        v[n] = cc * b - ss * a;
      } else {
        v[m] = cc * a - ss * b;
        v[n] = ss * a + cc * b;
      }
    }
  }
}

// Backward through one register block: v holds the block's stage outputs and
// gr their gradients; walks the stages in reverse, adding each pair's angle
// gradient to acc and leaving the block's inputs and their gradients.
template <int G, bool IN_SIDE>
__device__ __forceinline__ void bwd_block(float (&v)[8], float (&gr)[8], const float2 (&c)[12],
                                          float (&acc)[12]) {
#pragma unroll
  for (int tt = 0; tt < G; ++tt) {
    const int t = IN_SIDE ? tt : G - 1 - tt;
#pragma unroll
    for (int u = 0; u < (1 << (G - 1)); ++u) {
      const int m = pair_lo(t, u), n = m + (1 << t);
      const float cc = c[t * 4 + u].x, ss = IN_SIDE ? -c[t * 4 + u].y : c[t * 4 + u].y;
      const float vm = v[m], vn = v[n], gm = gr[m], gn = gr[n];
      const float da = gn * vm - gm * vn;   // d L / d (applied angle)
      acc[t * 4 + u] += IN_SIDE ? -da : da;
      v[m] = cc * vm + ss * vn;
      v[n] = cc * vn - ss * vm;
      gr[m] = cc * gm + ss * gn;
      gr[n] = cc * gn - ss * gm;
    }
  }
}

template <int D, int g, bool IN_SIDE, bool BWD>
__device__ __forceinline__ void run_group(float* V, float* Gs, int nr, int tid,
                                          const float2 (&cf)[BwdCfg<D>::NG][2][12],
                                          float (&acc)[BwdCfg<D>::NG][2][12], bool keep_v) {
  using C = BwdCfg<D>;
  constexpr int G = C::gsize(g), TPB = C::tpb(g);
#pragma unroll
  for (int sl = 0; sl < C::slots(g); ++sl) {
    int base, ph;
    block_of<D, G>(g, sl, tid, base, ph);
    int off[8];
#pragma unroll
    for (int m = 0; m < (1 << G); ++m) off[m] = pad(base + (m << (3 * g)));
    // Two rows at a time (loads of both in flight before either is rotated),
    // then the odd row out.
    int i = ph;
    for (; i + TPB < nr; i += 2 * TPB) {
      float* vr0 = V + i * C::PD;
      float* vr1 = V + (i + TPB) * C::PD;
      float v0[8], v1[8];
#pragma unroll
      for (int m = 0; m < (1 << G); ++m) {
        v0[m] = vr0[off[m]];
        v1[m] = vr1[off[m]];
      }
      if (BWD) {
        float* gp0 = Gs + i * C::PD;
        float* gp1 = Gs + (i + TPB) * C::PD;
        float g0[8], g1[8];
#pragma unroll
        for (int m = 0; m < (1 << G); ++m) {
          g0[m] = gp0[off[m]];
          g1[m] = gp1[off[m]];
        }
        bwd_block<G, IN_SIDE>(v0, g0, cf[g][sl], acc[g][sl]);
        bwd_block<G, IN_SIDE>(v1, g1, cf[g][sl], acc[g][sl]);
#pragma unroll
        for (int m = 0; m < (1 << G); ++m) {
          gp0[off[m]] = g0[m];
          gp1[off[m]] = g1[m];
        }
        if (keep_v) {
#pragma unroll
          for (int m = 0; m < (1 << G); ++m) {
            vr0[off[m]] = v0[m];
            vr1[off[m]] = v1[m];
          }
        }
      } else {
        fwd_block<G, IN_SIDE>(v0, cf[g][sl]);
        fwd_block<G, IN_SIDE>(v1, cf[g][sl]);
#pragma unroll
        for (int m = 0; m < (1 << G); ++m) {
          vr0[off[m]] = v0[m];
          vr1[off[m]] = v1[m];
        }
      }
    }
    if (i < nr) {
      float* vr = V + i * C::PD;
      float v[8];
#pragma unroll
      for (int m = 0; m < (1 << G); ++m) v[m] = vr[off[m]];
      if (BWD) {
        float* gp = Gs + i * C::PD;
        float gr[8];
#pragma unroll
        for (int m = 0; m < (1 << G); ++m) gr[m] = gp[off[m]];
        bwd_block<G, IN_SIDE>(v, gr, cf[g][sl], acc[g][sl]);
#pragma unroll
        for (int m = 0; m < (1 << G); ++m) gp[off[m]] = gr[m];
        if (keep_v) {
#pragma unroll
          for (int m = 0; m < (1 << G); ++m) vr[off[m]] = v[m];
        }
      } else {
        fwd_block<G, IN_SIDE>(v, cf[g][sl]);
#pragma unroll
        for (int m = 0; m < (1 << G); ++m) vr[off[m]] = v[m];
      }
    }
  }
}

// Groups in forward order (out side ascending, in side descending), or in
// backward order; a barrier after each group.
template <int D, bool IN_SIDE, bool BWD, int I = 0>
__device__ __forceinline__ void run_groups(float* V, float* Gs, int nr, int tid,
                                           const float2 (&cf)[BwdCfg<D>::NG][2][12],
                                           float (&acc)[BwdCfg<D>::NG][2][12]) {
  using C = BwdCfg<D>;
  if constexpr (I < C::NG) {
    constexpr bool ascending = IN_SIDE == BWD;
    constexpr int g = ascending ? I : C::NG - 1 - I;
    // the values are dead after the last group of the backward walk
    run_group<D, g, IN_SIDE, BWD>(V, Gs, nr, tid, cf, acc, !(BWD && I == C::NG - 1));
    __syncthreads();
    run_groups<D, IN_SIDE, BWD, I + 1>(V, Gs, nr, tid, cf, acc);
  }
}

// This tile's angle-gradient partial for group g: blocks shared by several
// threads (each over its own rows) are summed in thread order through LDS.
template <int D, int g>
__device__ __forceinline__ void write_partial(float* red, float* out, int tid,
                                              const float (&acc)[BwdCfg<D>::NG][2][12]) {
  using C = BwdCfg<D>;
  constexpr int G = C::gsize(g), TPB = C::tpb(g), NP = C::npairs(g);
  constexpr int bstride = C::NTHR / TPB;
#pragma unroll
  for (int sl = 0; sl < C::slots(g); ++sl) {
    int base, ph;
    block_of<D, G>(g, sl, tid, base, ph);
    float sum[12];
    if (TPB > 1) {
#pragma unroll
      for (int t = 0; t < G; ++t)
#pragma unroll
        for (int u = 0; u < (1 << (G - 1)); ++u) red[(t * 4 + u) * C::NTHR + tid] = acc[g][sl][t * 4 + u];
      __syncthreads();
#pragma unroll
      for (int t = 0; t < G; ++t)
#pragma unroll
        for (int u = 0; u < (1 << (G - 1)); ++u) {
          float a = 0.f;
#pragma unroll 2
          for (int q = 0; q < TPB; ++q) a += red[(t * 4 + u) * C::NTHR + q * bstride + tid % bstride];
          sum[t * 4 + u] = a;
        }
      __syncthreads();
    } else {
#pragma unroll
      for (int j = 0; j < 12; ++j) sum[j] = acc[g][sl][j];
    }
    if (ph == 0) {
#pragma unroll
      for (int t = 0; t < G; ++t) {
        const int s = 3 * g + t;
#pragma unroll
        for (int u = 0; u < (1 << (G - 1)); ++u)
          out[s * (D / 2) + pair_index(base + (pair_lo(t, u) << (3 * g)), s)] = sum[t * 4 + u];
      }
    }
  }
  (void)NP;
}

template <int D, int I = 0>
__device__ __forceinline__ void write_partials(float* red, float* out, int tid,
                                               const float (&acc)[BwdCfg<D>::NG][2][12]) {
  if constexpr (I < BwdCfg<D>::NG) {
    write_partial<D, I>(red, out, tid, acc);
    write_partials<D, I + 1>(red, out, tid, acc);
  }
}

// IN_SIDE = false: from H and dy to dH, dgates and dphi partials.
// IN_SIDE = true:  from x and dZ to dX (routed order) and dtheta partials.
// T: element type of every activation (x, dy, H, dH, dZ, dX).
template <int D, bool IN_SIDE, typename T>
__global__ __launch_bounds__(BwdCfg<D>::NTHR) void bfly_bwd_kernel(BwdParams p) {
  using C = BwdCfg<D>;
  constexpr int L = C::L, NG = C::NG, R = C::R, PD = C::PD, NTHR = C::NTHR, TPR = C::TPR;
  __shared__ float V[C::VSZ];
  __shared__ float Gs[R * PD];
  __shared__ int rowr[R];
  __shared__ float red[NTHR / 64];

  const int4 tile = p.tiles[blockIdx.x];
  const int e = tile.x;
  if (e < 0) return;  // past the last tile (whole workgroup)
  const int q0 = tile.y, q1 = tile.z;
  const int tid = threadIdx.x;
  const float2* cse = p.cs + (size_t)e * L * (D / 2);

  // cos/sin of every block this thread owns, and its gradient sums
  float2 cf[NG][2][12];
  float acc[NG][2][12];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int G = C::gsize(g);
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
#pragma unroll
      for (int j = 0; j < 12; ++j) {
        acc[g][sl][j] = 0.f;
        cf[g][sl][j] = make_float2(1.f, 0.f);
      }
      if (sl < C::slots(g)) {
        const int bstride = NTHR / C::tpb(g);
        const int base = block_base(tid % bstride + sl * bstride, 3 * g, G);
#pragma unroll
        for (int t = 0; t < 3; ++t)
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (t < G && u < (1 << (G - 1))) {
              const int s = 3 * g + t;
              cf[g][sl][t * 4 + u] = cse[s * (D / 2) + pair_index(base + (pair_lo(t, u) << (3 * g)), s)];
            }
      }
    }
  }

  constexpr int VS = 16 / sizeof(T), CPR = D / VS;  // 16-byte chunks per row
  const T* src = static_cast<const T*>(p.src);
  const T* grad = static_cast<const T*>(p.grad);
  T* dst = static_cast<T*>(p.dst);
  for (int qb = q0; qb < q1; qb += R) {
    const int nr = min(R, q1 - qb);
    if (tid < nr) rowr[tid] = p.perm[qb + tid];
    __syncthreads();
    for (int c = tid; c < nr * CPR; c += NTHR) {
      const int i = c / CPR, off = (c % CPR) * VS;
      const size_t tok = (size_t)(rowr[i] / p.k), sorted = (size_t)(qb + i);
      load16<T>(src + (IN_SIDE ? tok : sorted) * D + off, V + i * PD + pad(off));
      load16<T>(grad + (IN_SIDE ? sorted : tok) * D + off, Gs + i * PD + pad(off));
    }
    __syncthreads();
    run_groups<D, IN_SIDE, false>(V, Gs, nr, tid, cf, acc);
    if (!IN_SIDE) {
      // dg_r = <dy_t, u_r>, then G = g_r dy_t (each thread scales what it read)
      const int i = tid / TPR, c0 = tid % TPR;
      float dot = 0.f;
      if (i < nr) {
#pragma unroll 4
        for (int c = c0; c < D; c += TPR) dot += V[i * PD + pad(c)] * Gs[i * PD + pad(c)];
        const float gate = p.gates[rowr[i]];
#pragma unroll 4
        for (int c = c0; c < D; c += TPR) Gs[i * PD + pad(c)] *= gate;
      }
      if (TPR <= 64) {
#pragma unroll
        for (int o = TPR / 2; o >= 1; o >>= 1) dot += __shfl_xor(dot, o, TPR);
        if (c0 == 0 && i < nr) p.dgates[rowr[i]] = dot;
      } else {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) dot += __shfl_xor(dot, o, 64);
        if (tid % 64 == 0) red[tid / 64] = dot;
        __syncthreads();
        if (c0 == 0 && i < nr) {
          float sum = 0.f;
          for (int w = 0; w < TPR / 64; ++w) sum += red[tid / 64 + w];
          p.dgates[rowr[i]] = sum;
        }
      }
      __syncthreads();
    }
    run_groups<D, IN_SIDE, true>(V, Gs, nr, tid, cf, acc);
    for (int c = tid; c < nr * CPR; c += NTHR) {
      const int i = c / CPR, off = (c % CPR) * VS;
      const size_t row = IN_SIDE ? (size_t)rowr[i] : (size_t)(qb + i);
      store16<T>(Gs + i * PD + pad(off), dst + row * D + off, 1.0f);
    }
    __syncthreads();
  }
  write_partials<D>(V, p.partial + (size_t)blockIdx.x * L * (D / 2), tid, acc);
}

// The backward's closing sums, one launch with three block roles (each a
// grid-stride loop over its own blocks):
//   * dx[t] = sum_j dX[t k + j], ascending j, fp32 (like the forward's combine);
//   * dA[e][s][p] = sum of expert e's tile partials in tile order (0 if no
//     rows), for both sides: indices below N * per_expert reduce the output
//     side into dphi, the rest the input side into dtheta;
//   * dW = sum over the row ranges' fp32 partial products, in range order
//     (when the substrate gradient was split, else no blocks).
struct FinishParams {
  const void* dxr;
  void* dx;
  int T, d, k;
  const float* part_out;
  const float* part_in;
  const int32_t* tile_base;
  int N, per_expert;
  float* dphi;
  float* dtheta;
  const float4* dw_part;
  int slices;
  size_t dw4;  // d * d / 4
  float4* dw;
  int32_t* status;
  int nb_combine, nb_angle;
};

template <typename T>
__global__ __launch_bounds__(256) void finish_kernel(FinishParams p) {
  const int b = blockIdx.x;
  if (b == 0 && threadIdx.x == 0 && p.status) *p.status = BMOE_OK;
  if (b < p.nb_combine) {
    const T* U = static_cast<const T*>(p.dxr);
    T* y = static_cast<T*>(p.dx);
    const int d8 = p.d / 8;
    const size_t n = (size_t)p.T * d8;
    for (size_t idx = (size_t)b * 256 + threadIdx.x; idx < n; idx += (size_t)p.nb_combine * 256) {
      const size_t t = idx / d8, c = (idx % d8) * 8;
      float acc[8];
      for (int j = 0; j < p.k; ++j) {
        float v[8];
        load16<T>(U + (t * p.k + j) * p.d + c, v);
        if constexpr (sizeof(T) == 4) load16<T>(U + (t * p.k + j) * p.d + c + 4, v + 4);
#pragma unroll
        for (int m = 0; m < 8; ++m) acc[m] = j == 0 ? v[m] : acc[m] + v[m];
      }
      store16<T>(acc, y + t * p.d + c, 1.0f);
      if constexpr (sizeof(T) == 4) store16<T>(acc + 4, y + t * p.d + c + 4, 1.0f);
    }
    return;
  }
  if (b < p.nb_combine + p.nb_angle) {
    const size_t n = (size_t)p.N * p.per_expert;
    for (size_t v = (size_t)(b - p.nb_combine) * 256 + threadIdx.x; v < 2 * n;
         v += (size_t)p.nb_angle * 256) {
      const bool second = v >= n;
      const size_t u = second ? v - n : v;
      const float* partial = second ? p.part_in : p.part_out;
      const int e = (int)(u / p.per_expert), off = (int)(u % p.per_expert);
      float sum = 0.f;
      for (int t = p.tile_base[e]; t < p.tile_base[e + 1]; ++t)
        sum += partial[(size_t)t * p.per_expert + off];
      (second ? p.dtheta : p.dphi)[u] = sum;
    }
    return;
  }
  const int nb = gridDim.x - p.nb_combine - p.nb_angle;
  for (size_t u = (size_t)(b - p.nb_combine - p.nb_angle) * 256 + threadIdx.x; u < p.dw4;
       u += (size_t)nb * 256) {
    float4 a = p.dw_part[u];
    for (int s = 1; s < p.slices; ++s) {
      const float4 v = p.dw_part[(size_t)s * p.dw4 + u];
      a.x += v.x;
      a.y += v.y;
      a.z += v.z;
      a.w += v.w;
    }
    p.dw[u] = a;
  }
}

int grid_for(size_t n) {
  size_t b = (n + 255) / 256;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return (int)b;
}

template <int D, bool IN_SIDE>
hipError_t launch_bwd_d(bmoe_dtype dt, int max_tiles, const BwdParams& p, hipStream_t s,
                        const KernelTiming& t) {
  using C = BwdCfg<D>;
  if (dt == BMOE_BF16)
    return launch_kernel(bfly_bwd_kernel<D, IN_SIDE, uint16_t>, dim3(max_tiles), dim3(C::NTHR), 0,
                         s, t, p);
  return launch_kernel(bfly_bwd_kernel<D, IN_SIDE, float>, dim3(max_tiles), dim3(C::NTHR), 0, s,
                       t, p);
}

template <bool IN_SIDE>
hipError_t launch_bwd(bmoe_dtype dt, int d, int max_tiles, const BwdParams& p, hipStream_t s,
                      const KernelTiming& t) {
  switch (d) {
    case 16: return launch_bwd_d<16, IN_SIDE>(dt, max_tiles, p, s, t);
    case 32: return launch_bwd_d<32, IN_SIDE>(dt, max_tiles, p, s, t);
    case 64: return launch_bwd_d<64, IN_SIDE>(dt, max_tiles, p, s, t);
    case 128: return launch_bwd_d<128, IN_SIDE>(dt, max_tiles, p, s, t);
    case 256: return launch_bwd_d<256, IN_SIDE>(dt, max_tiles, p, s, t);
    case 512: return launch_bwd_d<512, IN_SIDE>(dt, max_tiles, p, s, t);
    case 1024: return launch_bwd_d<1024, IN_SIDE>(dt, max_tiles, p, s, t);
    case 2048: return launch_bwd_d<2048, IN_SIDE>(dt, max_tiles, p, s, t);
    case 4096: return launch_bwd_d<4096, IN_SIDE>(dt, max_tiles, p, s, t);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int bwd_max_tiles(int M, int N, int d) {
  const int tr = bwd_tile_rows(d);
  return (M + tr - 1) / tr + N;
}

int bwd_tile_rows_for(int d) { return bwd_tile_rows(d); }

hipError_t launch_bfly_bwd(bool in_side, bmoe_dtype dt, int M, int d, int k, const int4* tiles,
                           int max_tiles, const int32_t* perm, const float2* cs,
                           const float* gates, const void* src, const void* grad, void* dst,
                           float* dgates, float* partial, hipStream_t s,
                           const KernelTiming& t) {
  if (bwd_wave_supported(dt, d))
    return launch_bfly_bwd_wave(in_side, d, k, tiles, max_tiles, perm, cs, gates, src, grad, dst,
                                dgates, partial, s, t);
  BwdParams p;
  p.M = M;
  p.k = k;
  p.tiles = tiles;
  p.perm = perm;
  p.cs = cs;
  p.gates = gates;
  p.src = src;
  p.grad = grad;
  p.dst = dst;
  p.dgates = dgates;
  p.partial = partial;
  return in_side ? launch_bwd<true>(dt, d, max_tiles, p, s, t)
                 : launch_bwd<false>(dt, d, max_tiles, p, s, t);
}

hipError_t launch_bwd_finish(bmoe_dtype dt, int T, int d, int k, const void* dxr, void* dx,
                             const float* part_out, const float* part_in,
                             const int32_t* tile_base, int N, float* dphi, float* dtheta,
                             const float* dw_part, int slices, float* dw, int32_t* status,
                             hipStream_t s, const KernelTiming& t) {
  int L = 0;
  while ((1 << L) < d) ++L;
  FinishParams p;
  p.dxr = dxr;
  p.dx = dx;
  p.T = T;
  p.d = d;
  p.k = k;
  p.part_out = part_out;
  p.part_in = part_in;
  p.tile_base = tile_base;
  p.N = N;
  p.per_expert = L * (d / 2);
  p.dphi = dphi;
  p.dtheta = dtheta;
  p.dw_part = reinterpret_cast<const float4*>(dw_part);
  p.slices = slices;
  p.dw4 = (size_t)d * d / 4;
  p.dw = reinterpret_cast<float4*>(dw);
  p.status = status;
  p.nb_combine = grid_for((size_t)T * (d / 8));
  p.nb_angle = grid_for(2 * (size_t)N * p.per_expert);
  const int nb_dw = slices > 1 && dw ? grid_for(p.dw4) : 0;
  const dim3 grid(p.nb_combine + p.nb_angle + nb_dw);
  if (dt == BMOE_BF16) return launch_kernel(finish_kernel<uint16_t>, grid, dim3(256), 0, s, t, p);
  return launch_kernel(finish_kernel<float>, grid, dim3(256), 0, s, t, p);
}

}  // namespace bmoe
