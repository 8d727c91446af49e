// Backward of one butterfly side for bf16 d = 256 and 512 with the rows in
// registers (ButterflyMoE gist.science summary, §2.1 for the butterfly, §2.4
// for training the angles, §2.3 for the two rotation steps):
//   output side (u = g B(phi) h):   dH = B(phi)^T (g dy), dg = <dy, B(phi) h>,
//                                   dphi partials;
//   input side (z = B(theta)^T x):  dX = B(theta) dZ, dtheta partials.
//
// A workgroup of four waves takes one expert-aligned tile of at most 16
// sorted rows; each wave rotates up to four of them, one at a time, a row of
// d values spread over its 64 lanes (d/64 consecutive elements per lane, row
// position row_lane(l) as in the forward's fused kernel): stages inside a lane
// run in registers, partners across row-position bits 0-3 are one DPP move,
// bits 4 and 5 go through v_permlane16/32_swap. Every cos/sin the thread
// needs stays in registers for the whole tile (one expert), so a row costs
// only its loads, stores and arithmetic.
//
// A row first runs forward through its stages; then the stages are walked
// back: with the stage output v and its gradient G, the applied angle's
// gradient is G_upper v_lower - G_lower v_upper, and the inverse rotation
// gives both the stage input and its gradient (nothing is stored per stage).
// The angle gradients of a thread's pairs sum in registers over its rows;
// the four waves' sums are added through LDS in wave order into the tile's
// partial, which a later kernel adds per expert in tile order.
#include <type_traits>
#include <utility>

#include "common.h"
#include "kernels.h"

namespace bmoe {
namespace {

constexpr int kWavesB = 4;
constexpr int kThreadsB = kWavesB * kWave;
constexpr int kTileRowsB = 16;              // rows per tile (the tile list's)
constexpr int kRowsB = kTileRowsB / kWavesB;

template <int D>
struct BW {
  static constexpr int VPL = D / kWave;                      // values per lane
  static constexpr int RB = VPL == 8 ? 3 : 2;                // stages inside a lane
  static constexpr int L = RB + 6;
  static constexpr int P = D / 2;
};

// A thread's coefficients of the tile's expert. DPP stages keep
// (cos, sigma * sin), sigma the sign of the partner term in the forward
// rotation of this lane's element; the inverse rotation takes -sigma.
template <int D>
struct BCoef {
  float2 in[BW<D>::RB][BW<D>::VPL / 2];  // in the lane: (cos, sin) per pair
  float2 dp[4][BW<D>::VPL];              // row-position bit s - RB
  float2 sw[2][BW<D>::VPL / 2];          // row-position bits 4, 5, whole pairs after a swap
};

// Angle-gradient sums, same positions as the coefficients.
template <int D>
struct BAcc {
  float in[BW<D>::RB][BW<D>::VPL / 2];
  float dp[4][BW<D>::VPL];
  float sw[2][BW<D>::VPL / 2];
};

// Pair (within stage s) of the swap-stage register pair i of row position rl:
// after the swap across bit m, register pair (2i, 2i + 1) holds the pair of
// this lane's element 2i (bit clear) or of the partner's element 2i + 1.
template <int D>
__device__ __forceinline__ int swap_pair(int rl, int m, int s, int i) {
  constexpr int VPL = BW<D>::VPL;
  const int bit = 1 << m;
  const int lower = (rl & bit) ? VPL * (rl ^ bit) + 1 : VPL * rl;
  return pair_index(lower + 2 * i, s);
}

template <int D, bool TR>
__device__ __forceinline__ void load_bcoef(BCoef<D>& k, const float2* tab, int rl) {
  using C = BW<D>;
  constexpr int VPL = C::VPL, RB = C::RB, P = C::P;
#pragma unroll
  for (int s = 0; s < RB; ++s)
#pragma unroll
    for (int u = 0; u < VPL / 2; ++u) k.in[s][u] = tab[s * P + (VPL / 2) * rl + u];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int s = RB + m;
    const int upper = (rl >> m) & 1;
    // forward: lower element c a - s b (TR: c a + s b), upper c b + s a (TR: c b - s a)
    const int neg = TR ? upper : upper ^ 1;
#pragma unroll
    for (int r = 0; r < VPL; ++r) {
      const float2 c = tab[s * P + pair_index(VPL * rl + r, s)];
      k.dp[m][r] = make_float2(c.x, fneg_if(c.y, neg));
    }
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int s = RB + 4 + t;
#pragma unroll
    for (int i = 0; i < VPL / 2; ++i) k.sw[t][i] = tab[s * P + swap_pair<D>(rl, 4 + t, s, i)];
  }
}

// (a, b) = (lower, upper) element of a pair. TR: the transposed rotation.
template <bool TR>
__device__ __forceinline__ void rot2(float& a, float& b, float2 c) {
  const float x = a, y = b;
  if (TR) {
    a = c.x * x + c.y * y;
    b = c.x * y - c.y * x;
  } else {
    a = c.x * x - c.y * y;
    b = c.y * x + c.x * y;
  }
}

template <int D, int S>
__device__ __forceinline__ int lo_of(int u) {
  return ((u >> S) << (S + 1)) | (u & ((1 << S) - 1));
}

// ---- forward stages --------------------------------------------------------
template <int D, bool TR, int S>
__device__ __forceinline__ void fwd_stage(float (&v)[BW<D>::VPL], const BCoef<D>& k) {
  using C = BW<D>;
  constexpr int VPL = C::VPL, RB = C::RB;
  if constexpr (S < RB) {
#pragma unroll
    for (int u = 0; u < VPL / 2; ++u) {
      const int m = lo_of<D, S>(u);
      rot2<TR>(v[m], v[m + (1 << S)], k.in[S][u]);
    }
  } else if constexpr (S < RB + 4) {
    constexpr int M = S - RB;
#pragma unroll
    for (int r = 0; r < VPL; ++r)
      v[r] = fmaf(k.dp[M][r].x, v[r], k.dp[M][r].y * lane_partner<M>(v[r]));
  } else {
    constexpr int M = S - RB;
#pragma unroll
    for (int i = 0; i < VPL / 2; ++i) {
      float a = v[2 * i], b = v[2 * i + 1];
      lane_swap<M>(a, b);
      rot2<TR>(a, b, k.sw[M - 4][i]);
      lane_swap<M>(a, b);
      v[2 * i] = a;
      v[2 * i + 1] = b;
    }
  }
}

// ---- backward stages: v, g the stage's outputs and their gradients on entry,
// its inputs and their gradients on exit; the pair's angle gradient
// g_upper v_lower - g_lower v_upper added to the sums -------------------------
template <int D, bool TR, int S>
__device__ __forceinline__ void bwd_stage(float (&v)[BW<D>::VPL], float (&g)[BW<D>::VPL],
                                          const BCoef<D>& k, BAcc<D>& acc) {
  using C = BW<D>;
  constexpr int VPL = C::VPL, RB = C::RB;
  if constexpr (S < RB) {
#pragma unroll
    for (int u = 0; u < VPL / 2; ++u) {
      const int m = lo_of<D, S>(u), n = m + (1 << S);
      acc.in[S][u] = fmaf(g[n], v[m], fmaf(-g[m], v[n], acc.in[S][u]));
      rot2<!TR>(v[m], v[n], k.in[S][u]);
      rot2<!TR>(g[m], g[n], k.in[S][u]);
    }
  } else if constexpr (S < RB + 4) {
    constexpr int M = S - RB;
#pragma unroll
    for (int r = 0; r < VPL; ++r) {
      const float vp = lane_partner<M>(v[r]), gp = lane_partner<M>(g[r]);
      // g_partner v - g v_partner: the pair's term in a lower lane (only
      // lower lanes' sums are written)
      acc.dp[M][r] = fmaf(gp, v[r], fmaf(-g[r], vp, acc.dp[M][r]));
      const float c = k.dp[M][r].x, sn = -k.dp[M][r].y;
      v[r] = fmaf(c, v[r], sn * vp);
      g[r] = fmaf(c, g[r], sn * gp);
    }
  } else {
    constexpr int M = S - RB;
#pragma unroll
    for (int i = 0; i < VPL / 2; ++i) {
      float a = v[2 * i], b = v[2 * i + 1], ga = g[2 * i], gb = g[2 * i + 1];
      lane_swap<M>(a, b);
      lane_swap<M>(ga, gb);
      acc.sw[M - 4][i] = fmaf(gb, a, fmaf(-ga, b, acc.sw[M - 4][i]));
      rot2<!TR>(a, b, k.sw[M - 4][i]);
      rot2<!TR>(ga, gb, k.sw[M - 4][i]);
      lane_swap<M>(a, b);
      lane_swap<M>(ga, gb);
      v[2 * i] = a;
      v[2 * i + 1] = b;
      g[2 * i] = ga;
      g[2 * i + 1] = gb;
    }
  }
}

// Forward order: output side 0..L-1, input side (B^T) L-1..0; the backward
// walk the reverse.
template <int D, bool IN_SIDE, int... Ss>
__device__ __forceinline__ void fwd_all(float (&v)[BW<D>::VPL], const BCoef<D>& k,
                                        std::integer_sequence<int, Ss...>) {
  constexpr int L = BW<D>::L;
  if constexpr (IN_SIDE) (fwd_stage<D, true, L - 1 - Ss>(v, k), ...);
  else (fwd_stage<D, false, Ss>(v, k), ...);
}
template <int D, bool IN_SIDE, int... Ss>
__device__ __forceinline__ void bwd_all(float (&v)[BW<D>::VPL], float (&g)[BW<D>::VPL],
                                        const BCoef<D>& k, BAcc<D>& acc,
                                        std::integer_sequence<int, Ss...>) {
  constexpr int L = BW<D>::L;
  if constexpr (IN_SIDE) (bwd_stage<D, true, Ss>(v, g, k, acc), ...);
  else (bwd_stage<D, false, L - 1 - Ss>(v, g, k, acc), ...);
}

// A lane's d/64 bf16 of a row, raw: one 16- or 8-byte load.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
template <int D>
using RawRow = std::conditional_t<BW<D>::VPL == 8, u32x4, u32x2_t>;

template <int D>
__device__ __forceinline__ RawRow<D> load_raw(const uint16_t* src, int rl) {
  return *reinterpret_cast<const RawRow<D>*>(src + BW<D>::VPL * rl);
}

// Unpack a row's data here and not earlier: otherwise the compiler unpacks
// it before issuing the next row's loads (to reuse its registers) and waits
// for every load in flight. (One vector operand, so the registers stay a
// tuple.)
template <int D>
__device__ __forceinline__ void take_raw(RawRow<D> r, float (&v)[BW<D>::VPL]) {
  __asm__ volatile("" : "+v"(r));
#pragma unroll
  for (int c = 0; c < BW<D>::VPL / 2; ++c) {
    v[2 * c] = bf16_lo(r[c]);
    v[2 * c + 1] = bf16_hi(r[c]);
  }
}

template <int D>
__device__ __forceinline__ void store_row(uint16_t* dst, int rl, const float (&v)[BW<D>::VPL]) {
  constexpr int VPL = BW<D>::VPL;
  if constexpr (VPL == 8) {
    *reinterpret_cast<uint4*>(dst + VPL * rl) =
        make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                   pack_bf16x2(v[6], v[7]));
  } else {
    *reinterpret_cast<uint2*>(dst + VPL * rl) =
        make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  }
}

struct BwdWaveArgs {
  int k;
  const int4* tiles;
  const int32_t* perm;
  const float2* cs;     // [N][L][D/2] cos/sin of this side's angles
  const float* gates;
  const uint16_t* src;  // output side: H [M][D] (sorted); input side: x [T][D]
  const uint16_t* grad; // output side: dy [T][D];          input side: dZ [M][D] (sorted)
  uint16_t* dst;        // output side: dH [M][D] (sorted); input side: dX [M][D] (routed)
  float* dgates;        // output side only
  float* partial;       // [tiles][L][D/2]
};

template <int D, bool IN_SIDE>
__global__ __launch_bounds__(kThreadsB) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bfly_bwd_wave_kernel(BwdWaveArgs p) {
  using C = BW<D>;
  constexpr int VPL = C::VPL, RB = C::RB, L = C::L, P = C::P;
  __shared__ float red[kWavesB][L * P];  // each wave's angle-gradient sums

  const int4 tile = p.tiles[blockIdx.x];
  if (tile.x < 0) return;  // past the last tile (whole workgroup)
  const int e = tile.x, q0 = tile.y, q1 = tile.z;
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int rl = row_lane(lane);

  BCoef<D> k;
  load_bcoef<D, IN_SIDE>(k, p.cs + (size_t)e * L * P, rl);
  BAcc<D> acc = {};

  // This wave's rows r0 .. r0 + n - 1; lane j holds the routed index of row
  // r0 + j. Each row's loads are issued one row ahead, with no branch in the
  // row loop (the last row is loaded once more), so they overlap the row
  // before.
  const int r0 = q0 + wave * kRowsB, n = min(r0 + kRowsB, q1) - r0;
  const int pj = lane < n ? p.perm[r0 + lane] : 0;
  const float gj = !IN_SIDE && lane < n ? p.gates[pj] : 0.f;
  auto row_src = [&](int j, const uint16_t*& a, const uint16_t*& b) {
    const int r = __builtin_amdgcn_readlane(pj, j);
    const size_t tok = (size_t)(r / p.k), q = (size_t)(r0 + j);
    a = p.src + (IN_SIDE ? tok : q) * D;
    b = p.grad + (IN_SIDE ? q : tok) * D;
  };
  float dgj = 0.f;  // output side: lane j's row's dg
  RawRow<D> nv, ng;
  if (n > 0) {
    const uint16_t *a, *b;
    row_src(0, a, b);
    nv = load_raw<D>(a, rl);
    ng = load_raw<D>(b, rl);
  }
#pragma unroll 1
  for (int j = 0; j < n; ++j) {
    const int r = __builtin_amdgcn_readlane(pj, j);
    RawRow<D> cv = nv, cg = ng;
    {
      const uint16_t *a, *b;
      row_src(min(j + 1, n - 1), a, b);
      nv = load_raw<D>(a, rl);
      ng = load_raw<D>(b, rl);
    }
    float v[VPL], g[VPL];
    take_raw<D>(cv, v);
    take_raw<D>(cg, g);
    fwd_all<D, IN_SIDE>(v, k, std::make_integer_sequence<int, L>{});
    if constexpr (!IN_SIDE) {
      // dg = <dy, B(phi) h>; the gradient entering the rotation is g dy
      float dot = 0.f;
#pragma unroll
      for (int j = 0; j < VPL; ++j) dot = fmaf(g[j], v[j], dot);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) dot += __shfl_xor(dot, o, kWave);
      dgj = lane == j ? dot : dgj;  // stored after the row loop (no branch here)
      const float gate = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gj), j));
#pragma unroll
      for (int j = 0; j < VPL; ++j) g[j] *= gate;
    }
    bwd_all<D, IN_SIDE>(v, g, k, acc, std::make_integer_sequence<int, L>{});
    store_row<D>(p.dst + (IN_SIDE ? (size_t)r : (size_t)(r0 + j)) * D, rl, g);
  }
  if (!IN_SIDE && lane < n) p.dgates[pj] = dgj;

  // This wave's sums at their pairs (DPP stages: lower lanes only; the other
  // positions of a stage are covered by exactly one lane).
  float* const rw = red[wave];
#pragma unroll
  for (int s = 0; s < RB; ++s)
#pragma unroll
    for (int u = 0; u < VPL / 2; ++u) rw[s * P + (VPL / 2) * rl + u] = acc.in[s][u];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int s = RB + m;
    if (((rl >> m) & 1) == 0) {
#pragma unroll
      for (int r = 0; r < VPL; ++r) rw[s * P + pair_index(VPL * rl + r, s)] = acc.dp[m][r];
    }
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int s = RB + 4 + t;
#pragma unroll
    for (int i = 0; i < VPL / 2; ++i) rw[s * P + swap_pair<D>(rl, 4 + t, s, i)] = acc.sw[t][i];
  }
  __syncthreads();
  // The tile's partial: the waves' sums in wave order; on the input side the
  // angle is applied negated.
  float* const out = p.partial + (size_t)blockIdx.x * L * P;
  for (int i = threadIdx.x; i < L * P; i += kThreadsB) {
    float sum = red[0][i];
#pragma unroll
    for (int w = 1; w < kWavesB; ++w) sum += red[w][i];
    out[i] = IN_SIDE ? -sum : sum;
  }
}

template <int D, bool IN_SIDE>
hipError_t launch_bw(int max_tiles, const BwdWaveArgs& a, hipStream_t s, const KernelTiming& t) {
  return launch_kernel(bfly_bwd_wave_kernel<D, IN_SIDE>, dim3(max_tiles), dim3(kThreadsB), 0, s,
                       t, a);
}

}  // namespace

bool bwd_wave_supported(bmoe_dtype dt, int d) {
  return dt == BMOE_BF16 && (d == 256 || d == 512) && bwd_tile_rows_for(d) == kTileRowsB;
}

hipError_t launch_bfly_bwd_wave(bool in_side, int d, int k, const int4* tiles, int max_tiles,
                                const int32_t* perm, const float2* cs, const float* gates,
                                const void* src, const void* grad, void* dst, float* dgates,
                                float* partial, hipStream_t s, const KernelTiming& t) {
  BwdWaveArgs a;
  a.k = k;
  a.tiles = tiles;
  a.perm = perm;
  a.cs = cs;
  a.gates = gates;
  a.src = static_cast<const uint16_t*>(src);
  a.grad = static_cast<const uint16_t*>(grad);
  a.dst = static_cast<uint16_t*>(dst);
  a.dgates = dgates;
  a.partial = partial;
  switch (d) {
    case 256: return in_side ? launch_bw<256, true>(max_tiles, a, s, t)
                             : launch_bw<256, false>(max_tiles, a, s, t);
    case 512: return in_side ? launch_bw<512, true>(max_tiles, a, s, t)
                             : launch_bw<512, false>(max_tiles, a, s, t);
  }
  return hipErrorInvalidValue;
}

}  // namespace bmoe
