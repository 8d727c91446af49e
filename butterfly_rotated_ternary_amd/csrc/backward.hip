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
// So the kernels below first run a row forward through its butterfly (in
// LDS, fp32), then walk the stages backward from the outputs: no per-stage
// activations are stored. On the input side each stage runs with angle -a, so
// its angle gradient changes sign and its inverse is S(a).
//
// Angle gradients are summed per expert without atomics: rows are cut into
// tiles of at most kTileRows sorted rows of one expert, each tile keeps its
// sums in registers and writes one partial, and a second kernel adds an
// expert's partials in tile order (bit-reproducible).
#include "common.h"
#include "kernels.h"

namespace bmoe {
namespace {

constexpr int kTileRows = 64;

__device__ __forceinline__ int pad(int i) { return i + (i >> 3); }

__device__ __forceinline__ float ld_act(const uint16_t* p) { return bf16_lo(*p); }
__device__ __forceinline__ float ld_act(const float* p) { return *p; }
__device__ __forceinline__ void st_act(uint16_t* p, float v) { *p = (uint16_t)f32_to_bf16_bits(v); }
__device__ __forceinline__ void st_act(float* p, float v) { *p = v; }

// ---- expert-aligned row tiles ------------------------------------------------
// tiles[i] = (expert, first sorted row, end row, 0); tile_base[e] = first tile
// of expert e, tile_base[N] = number of tiles. One workgroup.
__global__ __launch_bounds__(1024) void tiles_kernel(const int32_t* offsets, int N, int4* tiles,
                                                     int32_t* tile_base, int max_tiles) {
  __shared__ int scan[1024];
  __shared__ int carry;
  const int tid = threadIdx.x;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int e0 = 0; e0 < N; e0 += 1024) {
    const int e = e0 + tid;
    const int cnt = e < N ? offsets[e + 1] - offsets[e] : 0;
    const int nt = (cnt + kTileRows - 1) / kTileRows;
    scan[tid] = nt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int v = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int base = carry + scan[tid] - nt;
    if (e < N) {
      tile_base[e] = base;
      const int q0 = offsets[e];
      for (int i = 0; i < nt; ++i)
        tiles[base + i] = make_int4(e, q0 + i * kTileRows, min(q0 + (i + 1) * kTileRows, q0 + cnt), 0);
    }
    __syncthreads();
    if (tid == 1023) carry += scan[1023];
    __syncthreads();
  }
  const int total = carry;
  if (tid == 0) tile_base[N] = total;
  for (int i = total + tid; i < max_tiles; i += 1024) tiles[i] = make_int4(-1, 0, 0, 0);
}

// ---- packed W_base^T ---------------------------------------------------------
// One thread per word of W^T: row c, columns o = 16 g .. 16 g + 15 (the codes
// W[o][c]), written row-major (wpt) and, when cb > 0, into the tile-major copy
// the large-tile GEMM reads (wtt: 4-word K-steps of 64 columns, cb rows each).
__device__ __forceinline__ int code_pos(int v) { return (v & 1) ? 16 + 2 * (v >> 1) : 2 * (v >> 1); }

__global__ __launch_bounds__(256) void pack_transpose_kernel(const uint32_t* wp, int d,
                                                             uint32_t* wpt, uint32_t* wtt,
                                                             int cb) {
  const int G = d / 16;
  const size_t n = (size_t)d * G;
  for (size_t u = (size_t)blockIdx.x * 256 + threadIdx.x; u < n; u += (size_t)gridDim.x * 256) {
    const int c = (int)(u / G), g = (int)(u % G);
    const int cw = c / 16, cpos = code_pos(c % 16);
    uint32_t out = 0u;
#pragma unroll
    for (int o16 = 0; o16 < 16; ++o16) {
      const uint32_t code = (wp[(size_t)(g * 16 + o16) * G + cw] >> cpos) & 3u;
      out |= code << code_pos(o16);
    }
    wpt[(size_t)c * G + g] = out;
    if (cb > 0) {
      const int nk = d / 64;
      wtt[(((size_t)(c / cb) * nk + g / 4) * cb + c % cb) * 4 + g % 4] = out;
    }
  }
}

// ---- butterfly backward --------------------------------------------------------
template <int D>
struct BwdCfg {
  static_assert(D >= 16 && D <= 4096, "backward sizes");
  static constexpr int L = D == 16 ? 4 : D == 32 ? 5 : D == 64 ? 6 : D == 128 ? 7 : D == 256 ? 8
                         : D == 512 ? 9 : D == 1024 ? 10 : D == 2048 ? 11 : 12;
  // Each thread keeps cos/sin and gradient sums for L * P pairs in registers.
  static constexpr int NTHR = D >= 4096 ? 512 : 256;
  static constexpr int NPAIR = D / 2;
  static constexpr int P = NPAIR >= NTHR ? NPAIR / NTHR : 1;   // pairs per thread per stage
  static constexpr int RB = NPAIR >= NTHR ? 1 : NTHR / NPAIR;  // rows per batch
  static constexpr int TPR = NTHR / RB;                        // threads per row
  static constexpr int EPT = D / TPR;                          // elements per thread
  static constexpr int PD = D + D / 8;
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

// Row batch load: zeros past the tile end.
template <int D, bool IN_SIDE, typename XT, typename AT>
__device__ __forceinline__ void bwd_load(const BwdParams& p, float* v, float* g, int q, bool valid,
                                         int t, int ec) {
  using C = BwdCfg<D>;
#pragma unroll
  for (int m = 0; m < C::EPT; ++m) {
    const int c = ec + m * C::TPR;
    float vv = 0.f, gg = 0.f;
    if (valid) {
      if (IN_SIDE) {
        vv = ld_act(static_cast<const XT*>(p.src) + (size_t)t * D + c);
        gg = ld_act(static_cast<const AT*>(p.grad) + (size_t)q * D + c);
      } else {
        vv = ld_act(static_cast<const AT*>(p.src) + (size_t)q * D + c);
        gg = ld_act(static_cast<const XT*>(p.grad) + (size_t)t * D + c);
      }
    }
    v[pad(c)] = vv;
    g[pad(c)] = gg;
  }
}

// Output side, after the forward pass: dg_r = <dy_t, u>, then G = g_r * dy_t.
template <int D>
__device__ __forceinline__ void bwd_gates(const BwdParams& p, float* v, float* g, float* red,
                                          bool valid, int r, int tid, int ec) {
  using C = BwdCfg<D>;
  float dot = 0.f;
#pragma unroll
  for (int m = 0; m < C::EPT; ++m) {
    const int c = ec + m * C::TPR;
    dot += g[pad(c)] * v[pad(c)];
  }
  if (C::TPR >= 64) {
    // a row spans TPR / 64 whole waves: wave sums, then the row's first thread
    constexpr int WPR = C::TPR / 64;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 64);
    if (tid % 64 == 0) red[tid / 64] = dot;
    __syncthreads();
    if (ec == 0 && valid) {
      float s = 0.f;
      for (int w = 0; w < WPR; ++w) s += red[(tid / 64) + w];
      p.dgates[r] = s;
    }
  } else {
#pragma unroll
    for (int off = C::TPR / 2; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, C::TPR);
    if (ec == 0 && valid) p.dgates[r] = dot;
  }
  const float gate = valid ? p.gates[r] : 0.f;
#pragma unroll
  for (int m = 0; m < C::EPT; ++m) {
    const int c = ec + m * C::TPR;
    g[pad(c)] *= gate;
  }
}

template <int D, bool IN_SIDE, typename AT>
__device__ __forceinline__ void bwd_store(const BwdParams& p, const float* g, int q, int r,
                                          bool valid, int ec) {
  using C = BwdCfg<D>;
  if (!valid) return;
  AT* dst = static_cast<AT*>(p.dst) + (size_t)(IN_SIDE ? r : q) * D;
#pragma unroll
  for (int m = 0; m < C::EPT; ++m) {
    const int c = ec + m * C::TPR;
    st_act(dst + c, g[pad(c)]);
  }
}

// Forward rotation of one pair (angle as applied: sn already signed).
__device__ __forceinline__ void rot_fwd(float* vr, int i, int j, float cs, float sn) {
  const float xi = vr[pad(i)], xj = vr[pad(j)];
  vr[pad(i)] = cs * xi - sn * xj;
  vr[pad(j)] = sn * xi + cs * xj;
}

// Backward step of one pair from the stage outputs: returns dL/d(applied angle).
__device__ __forceinline__ float rot_bwd(float* vr, float* gr, int i, int j, float cs, float sn) {
  const float vi = vr[pad(i)], vj = vr[pad(j)], gi = gr[pad(i)], gj = gr[pad(j)];
  vr[pad(i)] = cs * vi + sn * vj;
  vr[pad(j)] = -sn * vi + cs * vj;
  gr[pad(i)] = cs * gi + sn * gj;
  gr[pad(j)] = -sn * gi + cs * gj;
  return gj * vi - gi * vj;
}

__device__ __forceinline__ void pair_ij(int pp, int s, int& i, int& j) {
  i = ((pp >> s) << (s + 1)) | (pp & ((1 << s) - 1));
  j = i + (1 << s);
}

// IN_SIDE = false: from H and dy to dH, dgates and dphi partials.
// IN_SIDE = true:  from x and dZ to dX (routed order) and dtheta partials.
// XT: element type of x / dy; AT: element type of H, dH, dZ, dX.
// d <= 512: several rows per batch, cos/sin and gradient sums in registers.
template <int D, bool IN_SIDE, typename XT, typename AT>
__global__ __launch_bounds__(BwdCfg<D>::NTHR) void bfly_bwd_kernel(BwdParams p) {
  using C = BwdCfg<D>;
  constexpr int L = C::L, P = C::P, RB = C::RB, TPR = C::TPR, PD = C::PD;
  static_assert(D <= 512, "small-d variant");
  __shared__ float V[RB * PD];
  __shared__ float G[RB * PD];
  __shared__ float red[C::NTHR / 64];

  const int4 tile = p.tiles[blockIdx.x];
  const int e = tile.x;
  if (e < 0) return;  // past the last tile (whole workgroup)
  const int q0 = tile.y, q1 = tile.z;
  const int tid = threadIdx.x;
  // Stage work: thread -> (row slot, pairs). Element work: thread -> (row slot, elements).
  const int prs = RB > 1 ? tid / C::NPAIR : 0;
  const int ers = tid / TPR, ec = tid % TPR;

  float2 cf[L][P];
  float acc[L][P];
#pragma unroll
  for (int s = 0; s < L; ++s)
#pragma unroll
    for (int m = 0; m < P; ++m) {
      const int pp = RB > 1 ? tid % C::NPAIR : tid + m * C::NTHR;
      cf[s][m] = p.cs[((size_t)e * L + s) * C::NPAIR + pp];
      acc[s][m] = 0.f;
    }

  for (int qb = q0; qb < q1; qb += RB) {
    const int q = qb + ers;
    const bool valid = q < q1;
    const int r = valid ? p.perm[q] : 0;
    float* v = V + ers * PD;
    float* g = G + ers * PD;
    bwd_load<D, IN_SIDE, XT, AT>(p, v, g, q, valid, r / p.k, ec);
    __syncthreads();
#pragma unroll
    for (int ss = 0; ss < L; ++ss) {
      const int s = IN_SIDE ? L - 1 - ss : ss;
#pragma unroll
      for (int m = 0; m < P; ++m) {
        const int pp = RB > 1 ? tid % C::NPAIR : tid + m * C::NTHR;
        int i, j;
        pair_ij(pp, s, i, j);
        rot_fwd(V + prs * PD, i, j, cf[s][m].x, IN_SIDE ? -cf[s][m].y : cf[s][m].y);
      }
      __syncthreads();
    }
    if (!IN_SIDE) {
      bwd_gates<D>(p, v, g, red, valid, r, tid, ec);
      __syncthreads();
    }
#pragma unroll
    for (int ss = 0; ss < L; ++ss) {
      const int s = IN_SIDE ? ss : L - 1 - ss;
#pragma unroll
      for (int m = 0; m < P; ++m) {
        const int pp = RB > 1 ? tid % C::NPAIR : tid + m * C::NTHR;
        int i, j;
        pair_ij(pp, s, i, j);
        const float da = rot_bwd(V + prs * PD, G + prs * PD, i, j, cf[s][m].x,
                                 IN_SIDE ? -cf[s][m].y : cf[s][m].y);
        acc[s][m] += IN_SIDE ? -da : da;
      }
      __syncthreads();
    }
    bwd_store<D, IN_SIDE, AT>(p, g, q, r, valid, ec);
    __syncthreads();
  }

  // This tile's angle-gradient partial (row slots summed in slot order).
  float* out = p.partial + (size_t)blockIdx.x * L * C::NPAIR;
  if (RB == 1) {
#pragma unroll
    for (int s = 0; s < L; ++s)
#pragma unroll
      for (int m = 0; m < P; ++m) out[s * C::NPAIR + tid + m * C::NTHR] = acc[s][m];
  } else {
#pragma unroll
    for (int s = 0; s < L; ++s) {
      V[tid] = acc[s][0];
      __syncthreads();
      if (tid < C::NPAIR) {
        float sum = 0.f;
        for (int rs = 0; rs < RB; ++rs) sum += V[rs * C::NPAIR + tid];
        out[s * C::NPAIR + tid] = sum;
      }
      __syncthreads();
    }
  }
}

// d >= 1024: one row per batch; gradient sums in LDS (one slot per stage and
// pair, owned by one thread), cos/sin streamed one stage ahead.
template <int D, bool IN_SIDE, typename XT, typename AT>
__global__ __launch_bounds__(BwdCfg<D>::NTHR) void bfly_bwd_big_kernel(BwdParams p) {
  using C = BwdCfg<D>;
  constexpr int L = C::L, P = C::P, PD = C::PD, NPAIR = C::NPAIR, NTHR = C::NTHR;
  static_assert(D >= 1024 && C::RB == 1, "large-d variant");
  __shared__ float V[PD];
  __shared__ float G[PD];
  __shared__ float A[L * NPAIR];
  __shared__ float red[NTHR / 64];

  const int4 tile = p.tiles[blockIdx.x];
  const int e = tile.x;
  if (e < 0) return;  // past the last tile (whole workgroup)
  const int q0 = tile.y, q1 = tile.z;
  const int tid = threadIdx.x;
  const float2* cse = p.cs + (size_t)e * L * NPAIR;
  for (int u = tid; u < L * NPAIR; u += NTHR) A[u] = 0.f;

  for (int q = q0; q < q1; ++q) {
    const int r = p.perm[q];
    bwd_load<D, IN_SIDE, XT, AT>(p, V, G, q, true, r / p.k, tid);
    float2 cf[P], nf[P];
    {
      const int s = IN_SIDE ? L - 1 : 0;
#pragma unroll
      for (int m = 0; m < P; ++m) cf[m] = cse[s * NPAIR + tid + m * NTHR];
    }
    __syncthreads();
#pragma unroll 1
    for (int ss = 0; ss < L; ++ss) {
      const int s = IN_SIDE ? L - 1 - ss : ss;
      const int sn_next = IN_SIDE ? L - 2 - ss : ss + 1;  // forward stage after this one
      const int s_next = ss + 1 < L ? sn_next : (IN_SIDE ? 0 : L - 1);  // then backward's first
#pragma unroll
      for (int m = 0; m < P; ++m) nf[m] = cse[s_next * NPAIR + tid + m * NTHR];
#pragma unroll
      for (int m = 0; m < P; ++m) {
        int i, j;
        pair_ij(tid + m * NTHR, s, i, j);
        rot_fwd(V, i, j, cf[m].x, IN_SIDE ? -cf[m].y : cf[m].y);
      }
#pragma unroll
      for (int m = 0; m < P; ++m) cf[m] = nf[m];
      __syncthreads();
    }
    if (!IN_SIDE) {
      bwd_gates<D>(p, V, G, red, true, r, tid, tid);
      __syncthreads();
    }
#pragma unroll 1
    for (int ss = 0; ss < L; ++ss) {
      const int s = IN_SIDE ? ss : L - 1 - ss;
      const int s_next = IN_SIDE ? (ss + 1 < L ? ss + 1 : L - 1) : (ss + 1 < L ? L - 2 - ss : 0);
#pragma unroll
      for (int m = 0; m < P; ++m) nf[m] = cse[s_next * NPAIR + tid + m * NTHR];
#pragma unroll
      for (int m = 0; m < P; ++m) {
        int i, j;
        pair_ij(tid + m * NTHR, s, i, j);
        const float da = rot_bwd(V, G, i, j, cf[m].x, IN_SIDE ? -cf[m].y : cf[m].y);
        A[s * NPAIR + tid + m * NTHR] += IN_SIDE ? -da : da;
      }
#pragma unroll
      for (int m = 0; m < P; ++m) cf[m] = nf[m];
      __syncthreads();
    }
    bwd_store<D, IN_SIDE, AT>(p, G, q, r, true, tid);
    __syncthreads();
  }

  float* out = p.partial + (size_t)blockIdx.x * L * NPAIR;
  for (int u = tid; u < L * NPAIR; u += NTHR) out[u] = A[u];
}

// dA[e][s][p] = sum of expert e's tile partials, in tile order (0 if no rows).
__global__ __launch_bounds__(256) void angle_reduce_kernel(const float* partial,
                                                           const int32_t* tile_base, int N,
                                                           int per_expert, float* out) {
  const size_t n = (size_t)N * per_expert;
  for (size_t u = (size_t)blockIdx.x * 256 + threadIdx.x; u < n; u += (size_t)gridDim.x * 256) {
    const int e = (int)(u / per_expert), off = (int)(u % per_expert);
    float s = 0.f;
    for (int t = tile_base[e]; t < tile_base[e + 1]; ++t) s += partial[(size_t)t * per_expert + off];
    out[u] = s;
  }
}

int grid_for(size_t n) {
  size_t b = (n + 255) / 256;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return (int)b;
}

template <int D, bool IN_SIDE>
hipError_t launch_bwd_d(bmoe_dtype dt, int max_tiles, const BwdParams& p, hipStream_t s) {
  using C = BwdCfg<D>;
  if constexpr (D >= 1024) {
    if (dt == BMOE_BF16)
      return launch_kernel(bfly_bwd_big_kernel<D, IN_SIDE, uint16_t, uint16_t>, dim3(max_tiles),
                           dim3(C::NTHR), 0, s, KernelTiming{}, p);
    return launch_kernel(bfly_bwd_big_kernel<D, IN_SIDE, float, float>, dim3(max_tiles),
                         dim3(C::NTHR), 0, s, KernelTiming{}, p);
  } else {
    if (dt == BMOE_BF16)
      return launch_kernel(bfly_bwd_kernel<D, IN_SIDE, uint16_t, uint16_t>, dim3(max_tiles),
                           dim3(C::NTHR), 0, s, KernelTiming{}, p);
    return launch_kernel(bfly_bwd_kernel<D, IN_SIDE, float, float>, dim3(max_tiles),
                         dim3(C::NTHR), 0, s, KernelTiming{}, p);
  }
}

template <bool IN_SIDE>
hipError_t launch_bwd(bmoe_dtype dt, int d, int max_tiles, const BwdParams& p, hipStream_t s) {
  switch (d) {
    case 16: return launch_bwd_d<16, IN_SIDE>(dt, max_tiles, p, s);
    case 32: return launch_bwd_d<32, IN_SIDE>(dt, max_tiles, p, s);
    case 64: return launch_bwd_d<64, IN_SIDE>(dt, max_tiles, p, s);
    case 128: return launch_bwd_d<128, IN_SIDE>(dt, max_tiles, p, s);
    case 256: return launch_bwd_d<256, IN_SIDE>(dt, max_tiles, p, s);
    case 512: return launch_bwd_d<512, IN_SIDE>(dt, max_tiles, p, s);
    case 1024: return launch_bwd_d<1024, IN_SIDE>(dt, max_tiles, p, s);
    case 2048: return launch_bwd_d<2048, IN_SIDE>(dt, max_tiles, p, s);
    case 4096: return launch_bwd_d<4096, IN_SIDE>(dt, max_tiles, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int bwd_max_tiles(int M, int N) { return (M + kTileRows - 1) / kTileRows + N; }

hipError_t launch_tiles(const int32_t* offsets, int N, int4* tiles, int32_t* tile_base,
                        int max_tiles, hipStream_t s) {
  return launch_kernel(tiles_kernel, dim3(1), dim3(1024), 0, s, KernelTiming{}, offsets, N, tiles,
                       tile_base, max_tiles);
}

hipError_t launch_pack_transpose(const uint32_t* wp, int d, uint32_t* wpt, uint32_t* wtt, int cb,
                                 hipStream_t s) {
  return launch_kernel(pack_transpose_kernel, dim3(grid_for((size_t)d * (d / 16))), dim3(256), 0,
                       s, KernelTiming{}, wp, d, wpt, wtt, cb);
}

hipError_t launch_bfly_bwd(bool in_side, bmoe_dtype dt, int M, int d, int k, const int4* tiles,
                           int max_tiles, const int32_t* perm, const float2* cs,
                           const float* gates, const void* src, const void* grad, void* dst,
                           float* dgates, float* partial, hipStream_t s) {
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
  return in_side ? launch_bwd<true>(dt, d, max_tiles, p, s)
                 : launch_bwd<false>(dt, d, max_tiles, p, s);
}

hipError_t launch_angle_reduce(const float* partial, const int32_t* tile_base, int N, int d,
                               float* out, hipStream_t s) {
  int L = 0;
  while ((1 << L) < d) ++L;
  const int per = L * (d / 2);
  return launch_kernel(angle_reduce_kernel, dim3(grid_for((size_t)N * per)), dim3(256), 0, s,
                       KernelTiming{}, partial, tile_base, N, per, out);
}

}  // namespace bmoe
