// Butterfly rotations of routed bf16 rows for d = 1024, 2048 and 4096 with
// the coefficients held in registers (ButterflyMoE gist.science summary,
// §2.1 for the butterfly, §2.3 for the two rotation steps): input side
// z = B(theta_e)^T x, output side u = g * B(phi_e) h.
//
// One workgroup of W = d / 512 waves rotates a run of up to 128 consecutive
// sorted rows (grouped by expert), one row at a time: every lane holds one
// 16-byte chunk of the row, 8 consecutive elements. Each thread keeps the
// cos/sin of every pair it touches in every stage in registers, loaded once
// per run of rows of one expert, so a row costs only its own load, store and
// arithmetic. Index
// bits of element i split three ways:
//   layout X: bits 0-2 in the lane, bits 3-8 the row position of the lane,
//             bits 9.. the wave;
//   layout Y: bits 0-2 in the lane, bits 7.. the low row-position bits,
//             bits 3-6 the remaining row-position bits and the wave.
// Stages 0-6 run in X (in the lane, then through DPP for lane distances 1,
// 2, 4, 8), stages 7.. in Y (DPP for the first four), so a row changes
// layout once, through LDS. At d = 4096 layout Y keeps element bit 11 in the
// lane instead of bit 2 (a lane holds elements 4g .. 4g+3 and 2048 + 4g ..
// 2048 + 4g+3 of its row), so stage 11 is a rotation in registers too: no
// stage needs a permlane swap, which costs about five plain VALU operations
// against two for a DPP-fed multiply. The output side runs stages 0-6 in X,
// then 7.. in Y; the input side (B^T: stages descending) the reverse. Rows
// are loaded four ahead.
#include "common.h"
#include "kernels.h"

namespace bmoe {
namespace {

template <int D>
struct WB {
  static_assert(D == 1024 || D == 2048 || D == 4096, "register butterfly sizes");
  static constexpr int W = D / 512;                          // waves per row
  static constexpr int LW = W == 2 ? 1 : W == 4 ? 2 : 3;     // wave bits
  static constexpr int L = 9 + LW;
  static constexpr int B = L - 7;                            // stages in layout Y
  static constexpr int NYD = B < 4 ? B : 4;                  // of them on DPP
  static constexpr int NYS = B - NYD;                        // in the lane (d = 4096)
  static constexpr bool YG = NYS > 0;                        // Y holds 4-element groups
  static constexpr int P = D / 2;
  static constexpr int THREADS = 64 * W;
  static constexpr int PF = 4;                               // rows loaded ahead
  // (pairs of rows alternate between two LDS buffers within a group of PF)
  static_assert(PF % 4 == 0, "an even number of row pairs per group");
  static constexpr int MAX_TILE = 128;
  // 16-byte chunk (elements 8c .. 8c+7) of lane l in wave w; the layouts
  // place row position c = row_lane(l), so every lane distance below 16 is
  // one DPP move.
  static __device__ __forceinline__ int chunk_x(int w, int l) { return (w << 6) | row_lane(l); }
  static __device__ __forceinline__ int chunk_y(int w, int l) {
    const int c = row_lane(l);
    return ((c & ((1 << B) - 1)) << 4) | (c >> B) | (w << (6 - B));
  }
  // d = 4096, layout Y: 4-element group g (elements 4g .. 4g+3, registers
  // 0-3; registers 4-7 hold group g + 512). Group bits: 0-1 from row-position
  // bits 4-5, 2-4 the wave, 5-8 row-position bits 0-3 (element bits 7-10).
  static __device__ __forceinline__ int group_y(int w, int l) {
    const int c = row_lane(l);
    return ((c >> 4) & 3) | (w << 2) | ((c & 15) << 5);
  }
  // Element held in register r of lane l in layout Y.
  static __device__ __forceinline__ int elem_y(int w, int l, int r) {
    if constexpr (YG) return ((r >> 2) << 11) | (group_y(w, l) << 2) | (r & 3);
    else return (chunk_y(w, l) << 3) | r;
  }
  // LDS slot of chunk c in each of the two 16-byte planes: any 16 lanes fall
  // on distinct 16-byte bank groups, in layout X (chunk bits 0-3 vary) and in
  // layout Y (chunk bits 4-7 vary; at d = 1024 bits 4-6 and bit 0; at d =
  // 4096 group g sits in plane g & 1 at chunk g >> 1, and 16 lanes vary
  // chunk bits 4-7 too).
  static __device__ __forceinline__ int lds_pos(int c) {
    return c ^ ((c >> 4) & 15) ^ ((c & 1) << 3);
  }
};

// A thread's coefficients of one side of one expert. DPP stages store
// (cos, +-sin) with the sign of this lane's element already applied:
// out = cos * mine + (+-sin) * partner.
template <int D>
struct Coef {
  float2 in[3][4];          // stages 0-2, in the lane: (cos, sin) per pair
  float2 dp[4][8];          // stages 3-6 (layout X, lane bit s - 3)
  float2 y[WB<D>::NYD][8];  // stages 7.. (layout Y, lane bit s - 7)
  float2 hi[1][4];          // stage 11 at d = 4096, in the lane (layout Y):
                            // registers r and r + 4
};


template <bool TR>
__device__ __forceinline__ float2 signed_coef(float2 c, int i, int s) {
  const int upper = (i >> s) & 1;
  return make_float2(c.x, fneg_if(c.y, TR ? upper : upper ^ 1));
}

// tab: the side's cos/sin of one expert, [L][D/2].
template <int D, bool TR>
__device__ __forceinline__ void load_coef(Coef<D>& k, const float2* tab, int w, int lane) {
  using C = WB<D>;
  // Recompute the (many) table offsets here rather than let the compiler
  // keep them live across the row loop: a reload is rare, registers are not.
  __asm__ volatile("" : "+v"(lane));
  const int cx = C::chunk_x(w, lane);
#pragma unroll
  for (int t = 0; t < C::NYD; ++t) {
    const int s = 7 + t;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = C::elem_y(w, lane, j);
      k.y[t][j] = signed_coef<TR>(tab[s * C::P + pair_index(i, s)], i, s);
    }
  }
  if constexpr (C::NYS > 0) {
    // stage 11: register r (element bit 11 clear) pairs with register r + 4
    const int s = 7 + C::NYD;
#pragma unroll
    for (int r = 0; r < 4; ++r) k.hi[0][r] = tab[s * C::P + pair_index(C::elem_y(w, lane, r), s)];
  }
#pragma unroll
  for (int s = 0; s < 3; ++s)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int m = ((u >> s) << (s + 1)) | (u & ((1 << s) - 1));
      k.in[s][u] = tab[s * C::P + pair_index((cx << 3) | m, s)];
    }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int s = 3 + t;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = (cx << 3) | j;
      k.dp[t][j] = signed_coef<TR>(tab[s * C::P + pair_index(i, s)], i, s);
    }
  }
  // Let every load complete here: the row loop's wait counts then stay exact
  // where this (rare) branch rejoins it, so the rows loaded ahead stay in
  // flight.
  wait_vm_all();
}

// (a, b) = (lower, upper) element of a pair. TR: the transposed rotation.
template <bool TR>
__device__ __forceinline__ void rot_pair(float& a, float& b, float2 c) {
  const float x = a, y = b;
  if (TR) {
    a = c.x * x + c.y * y;
    b = c.x * y - c.y * x;
  } else {
    a = c.x * x - c.y * y;
    b = c.y * x + c.x * y;
  }
}

template <int S, bool TR>
__device__ __forceinline__ void inlane_stage(float (&v)[8], const float2 (&c)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int m = ((u >> S) << (S + 1)) | (u & ((1 << S) - 1));
    rot_pair<TR>(v[m], v[m + (1 << S)], c[u]);
  }
}

template <int M>
__device__ __forceinline__ void dpp_stage(float (&v)[8], const float2 (&c)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = fmaf(c[j].x, v[j], c[j].y * lane_partner<M>(v[j]));
}

// Stages 0-6 in layout X, ascending (output side) or descending (input side).
template <bool TR, class K>
__device__ __forceinline__ void stages_x(float (&v)[8], const K& k) {
  if constexpr (TR) {
    dpp_stage<3>(v, k.dp[3]);
    dpp_stage<2>(v, k.dp[2]);
    dpp_stage<1>(v, k.dp[1]);
    dpp_stage<0>(v, k.dp[0]);
    inlane_stage<2, true>(v, k.in[2]);
    inlane_stage<1, true>(v, k.in[1]);
    inlane_stage<0, true>(v, k.in[0]);
  } else {
    inlane_stage<0, false>(v, k.in[0]);
    inlane_stage<1, false>(v, k.in[1]);
    inlane_stage<2, false>(v, k.in[2]);
    dpp_stage<0>(v, k.dp[0]);
    dpp_stage<1>(v, k.dp[1]);
    dpp_stage<2>(v, k.dp[2]);
    dpp_stage<3>(v, k.dp[3]);
  }
}

// Stages 7.. in layout Y (lane bits 0 .. B-1).
template <int D, bool TR>
__device__ __forceinline__ void stages_y(float (&v)[8], const Coef<D>& k) {
  constexpr int N = WB<D>::NYD;
  if constexpr (TR) {
    if constexpr (WB<D>::NYS > 0) inlane_stage<2, true>(v, k.hi[0]);
    if constexpr (N > 3) dpp_stage<3>(v, k.y[N > 3 ? 3 : 0]);
    if constexpr (N > 2) dpp_stage<2>(v, k.y[N > 2 ? 2 : 0]);
    dpp_stage<1>(v, k.y[1]);
    dpp_stage<0>(v, k.y[0]);
  } else {
    dpp_stage<0>(v, k.y[0]);
    dpp_stage<1>(v, k.y[1]);
    if constexpr (N > 2) dpp_stage<2>(v, k.y[N > 2 ? 2 : 0]);
    if constexpr (N > 3) dpp_stage<3>(v, k.y[N > 3 ? 3 : 0]);
    if constexpr (WB<D>::NYS > 0) inlane_stage<2, false>(v, k.hi[0]);
  }
}

struct WaveBflyArgs {
  int M, k, tile_rows, routed_out;
  const int32_t* perm;
  const int32_t* slot_e;
  const uint16_t* src;
  uint16_t* dst;
  const float2* cs;    // [N][L][d/2] (cos, sin) of this side
  const float* gates;  // output side, [M] routed order
};

__device__ __forceinline__ int row_meta(const int (&m)[2], int i) {
  return __builtin_amdgcn_readlane(i < 64 ? m[0] : m[1], i & 63);
}

// IN_SIDE:  dst[q] = B(theta_e)^T src[perm[q] / k]   (dst[perm[q]] with routed_out)
// OUT_SIDE: dst[perm[q]] = gate[perm[q]] * B(phi_e) src[q]
template <int D, bool IN_SIDE>
__global__ __launch_bounds__(WB<D>::THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bfly_wave_kernel(WaveBflyArgs p) {
  using C = WB<D>;
  constexpr bool TR = IN_SIDE;
  __shared__ float4 tb[2][2][2][D / 8];  // [pair parity][row][16-byte plane][slot]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // Workgroups are dealt round-robin to the 8 XCDs; each XCD takes a
  // contiguous run of tiles, so an expert's table is pulled into few L2s.
  const int nb = gridDim.x, xcd = blockIdx.x % 8, per = nb / 8, extra = nb % 8;
  const int tile = xcd * per + min(xcd, extra) + blockIdx.x / 8;
  const int q0 = tile * p.tile_rows;
  const int n = min(p.tile_rows, p.M - q0);

  // Lane l holds the metadata of rows l and 64 + l of the tile.
  int me[2], ms[2], md[2], mg[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = q0 + min(h * 64 + lane, n - 1);
    const int r = p.perm[q];
    me[h] = p.slot_e[q];
    ms[h] = IN_SIDE ? r / p.k : q;
    md[h] = IN_SIDE ? (p.routed_out ? r : q) : r;
    mg[h] = IN_SIDE ? 0 : __float_as_int(p.gates[r]);
  }
  wait_vm_all();  // metadata in before the row loads start
  const int cin = IN_SIDE ? C::chunk_y(w, lane) : C::chunk_x(w, lane);
  const int cout = IN_SIDE ? C::chunk_x(w, lane) : C::chunk_y(w, lane);
  const int wpos = C::lds_pos(cin), rpos = C::lds_pos(cout);
  // d = 4096, layout Y: groups gy and gy + 512, in plane gy & 1 at slots
  // ya and yb.
  const int gy = C::group_y(w, lane), py = gy & 1;
  const int ya = C::lds_pos(gy >> 1), yb = C::lds_pos((gy >> 1) + 256);
  auto load_row = [&](int i) -> u32x4 {
    const uint16_t* row = p.src + (size_t)row_meta(ms, i) * D;
    if constexpr (IN_SIDE && C::YG) {
      const u32x2 lo = *reinterpret_cast<const u32x2*>(row + 4 * gy);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(row + 2048 + 4 * gy);
      u32x4 x;
      x[0] = lo[0]; x[1] = lo[1]; x[2] = hi[0]; x[3] = hi[1];
      return x;
    } else {
      return *reinterpret_cast<const u32x4*>(row + cin * 8);
    }
  };
  // The first layout's values of a row into LDS buffer b, row q.
  auto put = [&](int b, int q, const float (&v)[8]) {
    if constexpr (IN_SIDE && C::YG) {
      tb[b][q][py][ya] = make_float4(v[0], v[1], v[2], v[3]);
      tb[b][q][py][yb] = make_float4(v[4], v[5], v[6], v[7]);
    } else {
      tb[b][q][0][wpos] = make_float4(v[0], v[1], v[2], v[3]);
      tb[b][q][1][wpos] = make_float4(v[4], v[5], v[6], v[7]);
    }
  };

  // Runs of rows with one expert: load the run's first rows and the expert's
  // coefficients, then a row loop with no branch at all, so the compiler's
  // wait counts stay exact and PF rows stay in flight. Rows go in pairs, one
  // barrier per pair, software-pipelined across it: after the barrier a wave
  // reads pair p back from LDS, runs the first layout's stages of pair p + 1
  // (which hides that read) and writes them to the other buffer, then
  // finishes pair p. A run is padded to whole groups of PF rows with copies
  // of its last row: the same input gives the same bytes, stored again to the
  // same place.
  auto take = [&](u32x4 x, float (&v)[8]) {
    // Take the row's data here and not earlier: the compiler would otherwise
    // hoist the unpacking of all rows in flight to the top of the loop and
    // wait for every load. (One 128-bit operand, so the four registers stay
    // a tuple.)
    __asm__ volatile("" : "+v"(x));
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[2 * c] = bf16_lo(x[c]);
      v[2 * c + 1] = bf16_hi(x[c]);
    }
  };
  auto first_layout = [&](float (&v)[8], const Coef<D>& k) {
    if constexpr (IN_SIDE) stages_y<D, true>(v, k);
    else stages_x<false>(v, k);
  };
  auto second_layout = [&](float (&v)[8], const Coef<D>& k) {
    if constexpr (IN_SIDE) stages_x<true>(v, k);
    else stages_y<D, false>(v, k);
  };
  u32x4 ring[C::PF];
  Coef<D> cf;
  for (int i = 0; i < n;) {
    const int e = row_meta(me, i);
    // first row at or after i with another expert (rows are sorted by expert)
    const uint64_t o0 = __ballot(me[0] != e && lane >= i && lane < n);
    const uint64_t o1 = __ballot(me[1] != e && 64 + lane >= i && 64 + lane < n);
    const int end = o0 ? __builtin_ctzll(o0) : o1 ? 64 + __builtin_ctzll(o1) : n;
    auto row = [&](int r) { return min(i + r, end - 1); };
#pragma unroll
    for (int j = 0; j < C::PF; ++j) ring[j] = load_row(row(j));
    load_coef<D, TR>(cf, p.cs + (size_t)e * C::L * C::P, w, lane);
    lds_barrier();  // the previous run's last reads are done everywhere
    float va[2][8], vb[2][8];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      take(ring[q], va[q]);
      first_layout(va[q], cf);
      put(0, q, va[q]);
      ring[q] = load_row(row(C::PF + q));
    }
    for (int r0 = 0; r0 < end - i; r0 += C::PF) {
#pragma unroll
      for (int h = 0; h < C::PF / 2; ++h) {
        const int pr = r0 + 2 * h;  // first row of pair p; pair p + 1 in slots sn
        const int sn = (2 * h + 2) % C::PF;
        lds_barrier();
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          float4 a, b;
          if constexpr (!IN_SIDE && C::YG) {
            a = tb[h & 1][q][py][ya];
            b = tb[h & 1][q][py][yb];
          } else {
            a = tb[h & 1][q][0][rpos];
            b = tb[h & 1][q][1][rpos];
          }
          vb[q][0] = a.x; vb[q][1] = a.y; vb[q][2] = a.z; vb[q][3] = a.w;
          vb[q][4] = b.x; vb[q][5] = b.y; vb[q][6] = b.z; vb[q][7] = b.w;
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          take(ring[sn + q], va[q]);
          first_layout(va[q], cf);
          put((h + 1) & 1, q, va[q]);
          ring[sn + q] = load_row(row(pr + 2 + C::PF + q));
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          second_layout(vb[q], cf);
          const int r = row(pr + q);
          const float g = IN_SIDE ? 1.0f : __int_as_float(row_meta(mg, r));
          u32x4 o;
#pragma unroll
          for (int c = 0; c < 4; ++c) o[c] = pack_bf16x2(vb[q][2 * c] * g, vb[q][2 * c + 1] * g);
          uint16_t* drow = p.dst + (size_t)row_meta(md, r) * D;
          if constexpr (!IN_SIDE && C::YG) {
            u32x2 lo, hi;
            lo[0] = o[0]; lo[1] = o[1]; hi[0] = o[2]; hi[1] = o[3];
            *reinterpret_cast<u32x2*>(drow + 4 * gy) = lo;
            *reinterpret_cast<u32x2*>(drow + 2048 + 4 * gy) = hi;
          } else {
            *reinterpret_cast<u32x4*>(drow + cout * 8) = o;
          }
        }
      }
    }
    i = end;
  }
}

template <int D, bool IN_SIDE>
hipError_t launch_d(const WaveBflyArgs& a, hipStream_t s, const KernelTiming& t) {
  using C = WB<D>;
  const int tiles = (a.M + a.tile_rows - 1) / a.tile_rows;
  return launch_kernel(bfly_wave_kernel<D, IN_SIDE>, dim3(tiles), dim3(C::THREADS), 0, s, t, a);
}

}  // namespace

bool bfly_wave_supported(bmoe_dtype dt, int d) {
  return dt == BMOE_BF16 && (d == 1024 || d == 2048 || d == 4096);
}

hipError_t launch_bfly_wave(bool in_side, int M, int d, int k, const RouteTables& rt,
                            const float2* cs, const void* src, void* dst, const float* gates,
                            bool routed_out, hipStream_t s, const KernelTiming& t) {
  if (M <= 0) return hipSuccess;
  WaveBflyArgs a{};
  a.M = M; a.k = k; a.routed_out = routed_out ? 1 : 0;
  a.perm = rt.perm; a.slot_e = rt.slot_e;
  a.src = static_cast<const uint16_t*>(src);
  a.dst = static_cast<uint16_t*>(dst);
  a.cs = cs; a.gates = gates;
  // Rows per workgroup: the most (up to 128) that still leaves a workgroup
  // for every slot of the chip (256 CUs, 8 / W workgroups each), so the
  // per-expert coefficient loads spread over many rows.
  const int resident = 256 * 8 / (d / 512);
  a.tile_rows = WB<4096>::MAX_TILE;
  while (a.tile_rows > 32 && (M + a.tile_rows - 1) / a.tile_rows < resident) a.tile_rows /= 2;
  switch (d) {
    case 1024: return in_side ? launch_d<1024, true>(a, s, t) : launch_d<1024, false>(a, s, t);
    case 2048: return in_side ? launch_d<2048, true>(a, s, t) : launch_d<2048, false>(a, s, t);
    case 4096: return in_side ? launch_d<4096, true>(a, s, t) : launch_d<4096, false>(a, s, t);
  }
  return hipErrorInvalidValue;
}

}  // namespace bmoe
