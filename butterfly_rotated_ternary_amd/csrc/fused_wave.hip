// Fused ButterflyMoE expert forward with register-resident butterflies, for
// bf16 d = 256 and 512, routing its own rows (M <= 8192 routed rows, N <= 512
// experts at d = 256, N <= 256 at d = 512) or reading the preparation
// kernel's routing. ButterflyMoE gist.science summary, §2.3: rotate
// each routed token by B(theta_e)^T, multiply by the one ternary W_base,
// rotate by B(phi_e); §2.1 for the butterfly structure.
//
// One workgroup per 32 consecutive sorted slots: 16 waves of two rows each at
// d = 512, 8 waves of four rows at d = 256. Each wave owns its rows
// outright: a row of d values lives in one wave, d/64 values per
// lane (lane l holds elements VPL*c .. VPL*c + VPL-1 of row position
// c = row_lane(l)), so every butterfly stage is a wave-local operation and no
// barrier separates stages:
//   * stages whose partner is in the same lane (the low log2(VPL) bits) run
//     in registers;
//   * partners across row-position bits 0-3 come through one DPP move each
//     (quad_perm, row_half_mirror, row_ror), folded into a multiply; each
//     lane computes its own element of the pair, c * mine +- s * partner;
//   * partners 16 and 32 lanes away: v_permlane16_swap / v_permlane32_swap
//     exchange half of one register with half of another, so that each lane
//     holds a whole pair, the pair is rotated in registers, and a second swap
//     restores the layout.
// LDS carries only what must cross waves: the bf16 A tile of the product, the
// fp32 H rows coming back from the product (each product wave's MFMA output is a
// column slice of all 32 rows), the routing scratch and the cos/sin tables of
// the tile's first and last expert. Rows of any expert strictly between those
// two take their coefficients straight from the angles.
//
// Routing: every workgroup reads all ids,
// counts them per wave in LDS, derives the per-expert offsets and ranks only
// its own slots (stable: ascending routed index within an expert), and writes
// the same routing tables as the preparation kernel.
#include <utility>

#include "common.h"
#include "kernels.h"

namespace bmoe {
namespace {

constexpr int kSlots = 32;                 // sorted slots per workgroup
constexpr int kMaxMW = 8192;               // routed rows the routing launch takes

// Workgroup shape: at d = 512, 16 waves of two rows (four waves per SIMD, so
// one wave's DPP and LDS waits are covered by the others' work); at d = 256,
// 8 waves of four rows, whose 68 KiB of LDS let two workgroups share a CU
// when there are more tiles than CUs (16 waves need 85 KiB: measured 4%
// faster when routing, 20% slower after prep at 1024 tiles).
template <int D>
struct WG {
  static constexpr int THREADS = D == 512 ? 1024 : 512;
  static constexpr int WAVES = THREADS / kWave;
  static constexpr int ROWS = kSlots / WAVES;       // rows per wave
  static constexpr int IDS = kMaxMW / THREADS;      // ids per thread
  static constexpr int MAX_N = D == 512 ? 256 : 512;  // experts the routing launch takes
};

template <int D>
struct WCfg {
  static constexpr int VPL = D / kWave;                        // values per lane
  static constexpr int RB = VPL == 8 ? 3 : VPL == 4 ? 2 : 1;   // stages inside a lane
  static constexpr int L = RB + 6;
  static constexpr int P = D / 2;                              // pairs per stage
  static constexpr int TBL = L * P;                            // one expert's side table
  static constexpr int TAB_BYTES = TBL * 8;
  // fp32 H rows: 16 of them in the substrate staging array, 16 in the A
  // tile's (both dead once the product is done), D floats each. Rows r and
  // r + 4 (written by the two halves of a wave in the MFMA output layout)
  // land on opposite halves of the 64 banks: column c of row r is stored at
  // c ^ hswz(r).
  static constexpr int H_HALF_BYTES = (kSlots / 2) * D * 4;
  static __device__ __forceinline__ int hswz(int r) { return 32 * ((r >> 2) & 1); }
  static constexpr int WN = D / WG<D>::WAVES;  // substrate rows each wave copies to LDS
  // The product runs on the first eight waves, 32 rows x PWN columns each
  // (PFN 32x32 fragments): with sixteen waves, one 32-column fragment per
  // wave would read every A fragment sixteen times from LDS.
  static constexpr int PWAVES = WG<D>::WAVES < 8 ? WG<D>::WAVES : 8;
  static constexpr int PWN = D / PWAVES;
  static constexpr int PFN = PWN / 32;
  static constexpr int KS = 32;
  static constexpr int NSTEP = D / KS;
  static constexpr int ROUTE_BYTES = (WG<D>::WAVES * WG<D>::MAX_N + WG<D>::MAX_N + 16) * 4;
  // The packed substrate rows of one wave's output columns, copied to LDS
  // as they lie in memory (WN rows of D/4 bytes), 16-byte chunks permuted
  // within each row (see pw_chunk).
  static constexpr int ROWB = D / 4;
  static constexpr int CPR = ROWB / 16;               // 16-byte chunks per row
  static constexpr int PW_WAVE = WN * ROWB;
  static constexpr int PW_LOADS = PW_WAVE / 1024;     // 1 KiB per wave-wide copy
  // LDS, four arrays (distinct arrays let the compiler see that the global->
  // LDS copies into P cannot alias the other regions, so it does not wait for
  // them before unrelated LDS accesses):
  //   A: routing scratch and the input-side tables; once the A tile is
  //      complete, the output-side tables (written during the product);
  //   META: the tile's slot -> (expert, routed index);
  //   P: the packed substrate, then H rows 0..15;
  //   Z: the bf16 A tile, then H rows 16..31.
  static constexpr int OFF_ROUTE = 0;
  static constexpr int OFF_TIN = (ROUTE_BYTES + 255) / 256 * 256;
  static constexpr int OFF_TOUT = 0;
  static constexpr int A_BYTES = OFF_TIN + 2 * TAB_BYTES;
  static constexpr int META_BYTES = (3 * kSlots + 8) * 4;
  static constexpr int P_BYTES = WG<D>::WAVES * PW_WAVE;
  static constexpr int Z_BYTES = kSlots * D * 2;
  static constexpr int LDS_BYTES = A_BYTES + META_BYTES + P_BYTES + Z_BYTES;
  static_assert(P_BYTES >= H_HALF_BYTES && Z_BYTES >= H_HALF_BYTES, "H rows reuse P and Z");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  // Row R's chunk g sits at chunk g ^ pw_swz(R): a column of lanes reading
  // one word of 32 consecutive rows hits at most two lanes per bank.
  static __device__ __forceinline__ int pw_swz(int R) {
    return ((R & 7) ^ ((R >> 3) & 3)) & (CPR - 1);
  }
};

struct WaveArgs {
  int M, k, N;
  const uint16_t* x;
  const int32_t* ids;
  const float* gates;
  const float* theta;
  const float* phi;
  const uint32_t* wp;
  float alpha;  // scale for the +-2 substrate values
  uint16_t* u;
  RouteTables rt;
  int32_t* status;
  uint16_t* z;  // kZH: Z and H rows, bf16 [M][D] in sorted order
  uint16_t* h;
};

// What a launch writes: g * U rows (the forward), Z and H rows (kept for,
// or recomputed by, the backward), or both.
constexpr int kU = 1, kZH = 2;

// Which pairs a lane needs in stage s, and where a table keeps them.
//   in-lane stage (s < RB): the VPL/2 pairs (VPL/2) lane + u;
//   DPP stage (m = s - RB < 4): the VPL pairs p0(lane) + r of its elements,
//     shared with the partner lane (lane ^ 2^m);
//   swap stage (m = 4, 5): the VPL/2 pairs p0 + 2i, p0 the pair of element
//     VPL * (lane without bit m) + bit m.
// A table of one side of one expert stores, for each stage, exactly its D/2
// pairs in the order the lanes read them: 16-byte chunk i (two consecutive
// coefficients of one lane) of lane l at float4 s * D/4 + i * 64 + l, or, in a
// DPP stage, of compressed lane (l without bit m) at s * D/4 + i * 32 + that.
// Every wave-wide 16-byte read is then 64 (or 32, each read by two lanes)
// consecutive chunks: no bank conflicts.
template <int D>
__host__ __device__ constexpr int first_pair(int s, int lane) {
  using C = WCfg<D>;
  constexpr int VPL = C::VPL, RB = C::RB;
  if (s < RB) return (VPL / 2) * lane;
  const int m = s - RB;
  const int idx = m < 4 ? VPL * lane : VPL * (lane & ~(1 << m)) + ((lane >> m) & 1);
  return ((idx >> (s + 1)) << s) | (idx & ((1 << s) - 1));
}

// Pair of coefficient k of `lane` in stage s.
template <int D>
__host__ __device__ constexpr int pair_of(int s, int lane, int k) {
  const int m = s - WCfg<D>::RB;
  return first_pair<D>(s, lane) + (m >= 4 ? 2 * k : k);
}

// The pair a table keeps at float2 position k of stage s (the order the
// lanes read them in, above).
template <int D>
__host__ __device__ constexpr int table_pair(int s, int k) {
  using C = WCfg<D>;
  const int f = k / 2, h = k % 2;
  const int m = s - C::RB;
  if (s >= C::RB && m < 4) {
    const int i = f / 32, lam = f % 32;
    const int lane = ((lam >> m) << (m + 1)) | (lam & ((1 << m) - 1));
    return pair_of<D>(s, lane, 2 * i + h);
  }
  return pair_of<D>(s, f % 64, 2 * (f / 64) + h);
}

// Table position of every pair (the inverse of table_pair), fixed at compile
// time: pos[stage * D/2 + pair]. A thread that builds table entries reads the
// angles of four consecutive pairs with one 16-byte load and the positions
// of those four pairs with one 8-byte load, both coalesced across the wave.
template <int D>
struct TabPos {
  alignas(16) uint16_t v[WCfg<D>::TBL];
};
template <int D>
constexpr TabPos<D> make_tab_pos() {
  TabPos<D> t{};
  for (int s = 0; s < WCfg<D>::L; ++s)
    for (int k = 0; k < WCfg<D>::P; ++k)
      t.v[s * WCfg<D>::P + table_pair<D>(s, k)] = (uint16_t)k;
  return t;
}
// every stage's table order is a permutation of its pairs
template <int D>
constexpr bool table_order_is_permutation() {
  bool seen[WCfg<D>::TBL] = {};
  for (int s = 0; s < WCfg<D>::L; ++s)
    for (int k = 0; k < WCfg<D>::P; ++k) {
      const int p = table_pair<D>(s, k);
      if (p < 0 || p >= WCfg<D>::P || seen[s * WCfg<D>::P + p]) return false;
      seen[s * WCfg<D>::P + p] = true;
    }
  return true;
}
static_assert(table_order_is_permutation<256>() && table_order_is_permutation<512>(),
              "table positions invert the table order");
__device__ constexpr TabPos<256> kTabPos256 = make_tab_pos<256>();
__device__ constexpr TabPos<512> kTabPos512 = make_tab_pos<512>();
template <int D>
__device__ __forceinline__ const uint16_t* tab_pos() {
  if constexpr (D == 256) return kTabPos256.v;
  else return kTabPos512.v;
}

// Coefficients of one side of one expert from its LDS table.
template <int D>
struct TabSrc {
  static constexpr bool kPerRow = false;
  const float4* tab;
  template <int S, int N>
  __device__ __forceinline__ void get(float2 (&c)[N], int lane, int /*row*/) const {
    load<S, N>(tab, c, lane);
  }
  template <int S, int N>
  __device__ static __forceinline__ void load(const float4* tab, float2 (&c)[N], int lane) {
    using C = WCfg<D>;
    constexpr int M = S - C::RB;
    const float4* t = tab + S * (C::P / 2);
    int off = lane, stride = 64;
    if constexpr (S >= C::RB && M < 4) {
      off = ((lane >> (M + 1)) << M) | (lane & ((1 << M) - 1));
      stride = 32;
    }
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const float4 q = t[i * stride + off];
      c[2 * i] = make_float2(q.x, q.y);
      c[2 * i + 1] = make_float2(q.z, q.w);
    }
  }
};

// Each row its own expert's LDS table (a wave whose rows straddle the
// tile's expert boundary).
template <int D>
struct TabRowSrc {
  static constexpr bool kPerRow = true;
  const float4* tab[WG<D>::ROWS];
  template <int S, int N>
  __device__ __forceinline__ void get(float2 (&c)[N], int lane, int row) const {
    TabSrc<D>::template load<S, N>(tab[row], c, lane);
  }
};

// The same coefficients evaluated from the expert's angles in global memory
// (an expert without a table in this tile).
template <int D>
struct AngSrc {
  static constexpr bool kPerRow = false;
  const float* ang;
  template <int S, int N>
  __device__ __forceinline__ void get(float2 (&c)[N], int lane, int /*row*/) const {
#pragma unroll
    for (int i = 0; i < N; ++i) c[i] = tile_cos_sin(ang[S * WCfg<D>::P + pair_of<D>(S, lane, i)]);
  }
};

// One butterfly stage s on NR rows held VPL values per lane (element
// VPL*lane + r in v[.][r]). TR: the transposed side (angle negated).
template <int D, bool TR, int NR, int S, class Src>
__device__ __forceinline__ void stage(float (&v)[NR][D / 64], const Src& src, int lane) {
  using C = WCfg<D>;
  constexpr int VPL = C::VPL, RB = C::RB;
  constexpr int NC = Src::kPerRow ? NR : 1;  // coefficient sets: one per row, or shared
  if constexpr (S < RB) {
    // Both elements of every pair in this lane: pairs VPL/2 * lane + u.
    float2 cc[NC][VPL / 2];
#pragma unroll
    for (int q = 0; q < NC; ++q) src.template get<S, VPL / 2>(cc[q], lane, q);
#pragma unroll
    for (int u = 0; u < VPL / 2; ++u) {
      const int m = ((u >> S) << (S + 1)) | (u & ((1 << S) - 1)), n = m + (1 << S);
#pragma unroll
      for (int q = 0; q < NR; ++q) {
        const float2 c = cc[NC == 1 ? 0 : q][u];
        const float a = v[q][m], b = v[q][n];
        if (TR) {
          v[q][m] = c.x * a + c.y * b;
          v[q][n] = c.x * b - c.y * a;
        } else {
          v[q][m] = c.x * a - c.y * b;
          v[q][n] = c.y * a + c.x * b;
        }
      }
    }
  } else if constexpr (S < RB + 4) {
    // Partner in lane ^ 2^(S-RB): out = c * mine + sigma * s * partner, with
    // sigma = +1 for the lower element on the transposed side and -1 on the
    // forward side (and the opposite for the upper element).
    constexpr int M = S - RB;
    float2 cc[NC][VPL];
#pragma unroll
    for (int q = 0; q < NC; ++q) src.template get<S, VPL>(cc[q], lane, q);
    const int upper = (lane >> M) & 1;
    const int neg = TR ? upper : upper ^ 1;
#pragma unroll
    for (int r = 0; r < VPL; ++r) {
#pragma unroll
      for (int q = 0; q < NR; ++q) {
        const float2 c = cc[NC == 1 ? 0 : q][r];
        const float sn = fneg_if(c.y, neg);
        // the partner's DPP move folds into the multiply
        const float t = sn * lane_partner<M>(v[q][r]);
        v[q][r] = fmaf(c.x, v[q][r], t);
      }
    }
  } else {
    // Partner in lane ^ 16 or ^ 32: swap register pairs (r, r+1) so each lane
    // holds one whole pair (the lower lanes that of register r, the upper
    // lanes that of register r + 1), rotate, swap back.
    constexpr int M = S - RB;
    float2 c2[NC][VPL / 2];
#pragma unroll
    for (int q = 0; q < NC; ++q) src.template get<S, VPL / 2>(c2[q], lane, q);
#pragma unroll
    for (int q = 0; q < NR; ++q) {
#pragma unroll
      for (int r = 0; r < VPL; r += 2) {
        float a = v[q][r], b = v[q][r + 1];
        lane_swap<M>(a, b);
        const float cc = c2[NC == 1 ? 0 : q][r / 2].x, ss = c2[NC == 1 ? 0 : q][r / 2].y;
        float a2, b2;
        if (TR) {
          a2 = cc * a + ss * b;
          b2 = cc * b - ss * a;
        } else {
          a2 = cc * a - ss * b;
          b2 = ss * a + cc * b;
        }
        lane_swap<M>(a2, b2);
        v[q][r] = a2;
        v[q][r + 1] = b2;
      }
    }
  }
}

template <int D, bool TR, int NR, class Src, int... Ss>
__device__ __forceinline__ void stages(float (&v)[NR][D / 64], const Src& src, int lane,
                                       std::integer_sequence<int, Ss...>) {
  if constexpr (TR) {
    // B^T: S_{L-1}^T first
    (stage<D, TR, NR, WCfg<D>::L - 1 - Ss>(v, src, lane), ...);
  } else {
    (stage<D, TR, NR, Ss>(v, src, lane), ...);
  }
}

template <int D, bool TR, int NR, class Src>
__device__ __forceinline__ void butterfly(float (&v)[NR][D / 64], const Src& src, int lane) {
  stages<D, TR, NR>(v, src, lane, std::make_integer_sequence<int, WCfg<D>::L>{});
}

// Rotate this wave's four rows, row q by expert e[q]'s butterfly: all four
// in one pass when every row's expert has a table here (shared by the four in
// the usual case, per row where the tile's expert boundary falls inside the
// wave), else one row at a time. Each pass takes its coefficients from one
// kind of source, so its stages hold no branches.
template <int D, bool TR>
__device__ __forceinline__ void butterfly_rows(float (&v)[WG<D>::ROWS][D / 64],
                                               const int (&e)[WG<D>::ROWS], int e_first,
                                               int e_last, const float4* tab_first,
                                               const float4* tab_last, const float* ang,
                                               int lane) {
  using C = WCfg<D>;
  constexpr int VPL = C::VPL, NR = WG<D>::ROWS;
  auto table = [&](int ex) -> const float4* {
    return ex == e_first ? tab_first : ex == e_last ? tab_last : nullptr;
  };
  bool same = true, tables = true;
  TabRowSrc<D> rows;
#pragma unroll
  for (int q = 0; q < NR; ++q) {
    same = same && e[q] == e[0];
    rows.tab[q] = table(e[q]);
    tables = tables && rows.tab[q] != nullptr;
  }
  if (same && tables) {
    butterfly<D, TR, NR>(v, TabSrc<D>{rows.tab[0]}, lane);
    return;
  }
  if (tables) {
    // rows of the tile's first and last experts: one pass, per-row tables
    butterfly<D, TR, NR>(v, rows, lane);
    return;
  }
#pragma unroll 1
  for (int q = 0; q < NR; ++q) {
    // row q through selects (q is uniform; no dynamic register indexing)
    float one[1][VPL];
    int ex = e[0];
#pragma unroll
    for (int i = 1; i < NR; ++i) ex = q == i ? e[i] : ex;
#pragma unroll
    for (int r = 0; r < VPL; ++r) {
      one[0][r] = v[0][r];
#pragma unroll
      for (int i = 1; i < NR; ++i) one[0][r] = q == i ? v[i][r] : one[0][r];
    }
    const float4* tab = table(ex);
    if (tab) butterfly<D, TR, 1>(one, TabSrc<D>{tab}, lane);
    else butterfly<D, TR, 1>(one, AngSrc<D>{ang + (size_t)ex * C::TBL}, lane);
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
      for (int r = 0; r < VPL; ++r) v[i][r] = q == i ? one[0][r] : v[i][r];
  }
}

// The tables of the tile's first and last experts hold L stage blocks of
// D/2 pairs each; cut into chunks of four consecutive pairs of one stage,
// CPE chunks per expert, the two experts' 2 * CPE chunks are dealt to the
// threads in turn: chunk c = tid + THREADS * i is thread tid's i-th, so a
// wave reads 64 consecutive chunks (1 KiB of angles) at once.
template <int D>
struct TableJob {
  static constexpr int QPS = WCfg<D>::P / 4;                          // chunks per stage
  static constexpr int CPE = WCfg<D>::TBL / 4;                        // chunks per expert
  static constexpr int NTB = (2 * CPE + WG<D>::THREADS - 1) / WG<D>::THREADS;  // per thread
  static_assert(NTB <= WCfg<D>::NSTEP, "one output-side chunk per K-step");
  // chunk i of thread tid: expert (0 first, 1 last), stage, first pair;
  // false past the last chunk
  __device__ static __forceinline__ bool at(int i, int tid, int& ex, int& s, int& p0) {
    const int c = tid + WG<D>::THREADS * i;
    ex = c / CPE;
    s = (c % CPE) / QPS;
    p0 = 4 * (c % QPS);
    return c < 2 * CPE;
  }
};

// Chunk i of this thread's share of one side's tables (see TableJob), from
// its four angles and the four pairs' table positions; the last expert's
// chunks only when it differs from the first.
template <int D>
__device__ __forceinline__ void write_table_chunk(int i, float4 ang, uint2 pos, float2* tab,
                                                  bool two, int tid) {
  int ex, s, p0;
  if (!TableJob<D>::at(i, tid, ex, s, p0) || (ex == 1 && !two)) return;
  float2* t = tab + ex * WCfg<D>::TBL + s * WCfg<D>::P;
  t[pos.x & 0xFFFFu] = tile_cos_sin(ang.x);
  t[pos.x >> 16] = tile_cos_sin(ang.y);
  t[pos.y & 0xFFFFu] = tile_cos_sin(ang.z);
  t[pos.y >> 16] = tile_cos_sin(ang.w);
}

// ROUTE: the kernel routes its own rows (reads the ids, writes the routing
// tables and the status word); otherwise the rows' experts and routed
// indices come from the preparation kernel's tables (any M and N). OUT: kU,
// kZH or both (kZH only after prep; without kU the output side is skipped).
template <int D, bool ROUTE, int OUT = kU>
__global__ __launch_bounds__(WG<D>::THREADS) void fused_wave_kernel(WaveArgs a) {
  static_assert(!ROUTE || OUT == kU, "a routing launch writes U only");
  constexpr bool kOut = (OUT & kU) != 0;
  using C = WCfg<D>;
  using G = WG<D>;
  constexpr int VPL = C::VPL;
  constexpr int kThreadsW = G::THREADS, kWavesW = G::WAVES, kRowsW = G::ROWS, kIdsW = G::IDS;
  constexpr int kMaxNW = G::MAX_N;
  __shared__ __attribute__((aligned(1024))) char lds[C::A_BYTES];
  __shared__ __attribute__((aligned(16))) int meta[C::META_BYTES / 4];
  __shared__ __attribute__((aligned(1024))) char pst[C::P_BYTES];
  __shared__ __attribute__((aligned(1024))) char zt[C::Z_BYTES];
  int* const wcnt = reinterpret_cast<int*>(lds + C::OFF_ROUTE);  // [waves][N]
  int* const cnt = wcnt + kWavesW * kMaxNW;                        // [N + 1]
  int* const misc = cnt + kMaxNW + 4;                              // bad id; first, last expert
  float2* const tin = reinterpret_cast<float2*>(lds + C::OFF_TIN);    // first, last
  float2* const tout = reinterpret_cast<float2*>(lds + C::OFF_TOUT);  // first, last
  const float4* const tin_first = reinterpret_cast<const float4*>(tin);
  const float4* const tin_last = reinterpret_cast<const float4*>(tin + C::TBL);
  const float4* const tout_first = reinterpret_cast<const float4*>(tout);
  const float4* const tout_last = reinterpret_cast<const float4*>(tout + C::TBL);
  int* const sh_e = meta;
  int* const sh_r = sh_e + kSlots;
  // fp32 H row r (after the product): rows 0..15 in P, 16..31 in Z
  auto hrow = [&](int r) -> float* {
    return reinterpret_cast<float*>(r < kSlots / 2 ? pst : zt) + (r % (kSlots / 2)) * D;
  };
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int rl = row_lane(lane);  // this lane's position in a butterfly row
  char* const pwl = pst + wave * C::PW_WAVE;  // this wave's substrate rows
  // After prep, the last tiles (the many small experts of a skewed routing,
  // which take the slower per-row coefficient paths) go first, so they do
  // not form the last round of the grid.
  const int tile = ROUTE ? (int)blockIdx.x : (int)(gridDim.x - 1 - blockIdx.x);
  const int q0 = tile * kSlots;
  const int nr = min(kSlots, a.M - q0);
  const int N = a.N;

  // ---- routing of this tile's slots ---------------------------------------
  const int i0 = kIdsW * tid;
  const int nv = ROUTE ? max(0, min(kIdsW, a.M - i0)) : 0;
  int id[kIdsW];
  if constexpr (!ROUTE) {
#pragma unroll
    for (int j = 0; j < kIdsW; ++j) id[j] = 0;
  } else if (nv == kIdsW) {
#pragma unroll
    for (int j = 0; j < kIdsW / 4; ++j) {
      const int4 v = reinterpret_cast<const int4*>(a.ids + i0)[j];
      id[4 * j] = v.x; id[4 * j + 1] = v.y; id[4 * j + 2] = v.z; id[4 * j + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kIdsW; ++j) id[j] = j < nv ? a.ids[i0 + j] : 0;
  }

  // Table positions of this thread's table chunks (they do not depend on
  // the routing).
  constexpr int NTB = TableJob<D>::NTB;
  uint2 tpos[NTB];
#pragma unroll
  for (int i = 0; i < NTB; ++i) {
    int ex, s, p0;
    tpos[i] = make_uint2(0u, 0u);
    if (TableJob<D>::at(i, tid, ex, s, p0))
      tpos[i] = *reinterpret_cast<const uint2*>(tab_pos<D>() + s * C::P + p0);
  }
  // This wave's packed substrate rows (o = wave * WN ..), copied to LDS by
  // the global->LDS path in 1 KiB pieces: lane l of piece i fills LDS chunk
  // c = 64 i + l, which holds row c / CPR's global chunk (c % CPR) ^ swz.
  // Issued at the start: the compiler makes the first LDS access after a
  // global->LDS copy wait for it, so they land during the routing.
  {
    const char* wrows = reinterpret_cast<const char*>(a.wp) + (size_t)wave * C::PW_WAVE;
#pragma unroll
    for (int i = 0; i < C::PW_LOADS; ++i) {
      const int c = 64 * i + lane, R = c / C::CPR, g = (c % C::CPR) ^ C::pw_swz(R);
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(wrows + R * C::ROWB + 16 * g),
          (__attribute__((address_space(3))) void*)(pwl + 1024 * i), 16, 0, 0);
    }
  }
  if constexpr (!ROUTE) {
    // The preparation kernel's routing: slot -> (expert, routed index);
    // rows past the end repeat the last one.
    if (tid < kSlots) {
      const int q = q0 + min(tid, nr - 1);
      sh_e[tid] = a.rt.slot_e[q];
      sh_r[tid] = a.rt.perm[q];
    }
    if (tid == 0) {
      misc[1] = a.rt.slot_e[q0];
      misc[2] = a.rt.slot_e[q0 + nr - 1];
    }
    lds_barrier();
  } else {
    for (int e = tid; e < kWavesW * N; e += kThreadsW) wcnt[e] = 0;
    if (tid == 0) {
      misc[0] = 0;
      misc[1] = 0;
      misc[2] = 0;
    }
    if (tid < kSlots) {  // every valid slot is ranked below
      sh_e[tid] = 0;
      sh_r[tid] = 0;
    }
    lds_barrier();
    // The histogram needs the ids, and everything issued before them lands
    // first anyway. Waiting here visibly to the compiler keeps it from
    // waiting again at the ranking (each histogram add sits in its own
    // branch), where the angle loads issued in between would be waited for
    // too instead of landing during it.
    wait_vm_all();
    bool bad = false;
    int* const mine = wcnt + wave * N;
#pragma unroll
    for (int j = 0; j < kIdsW; ++j) {
      if (j < nv) {
        int e = id[j];
        if ((unsigned)e >= (unsigned)N) {
          bad = true;
          e = e < 0 ? 0 : N - 1;
        }
        id[j] = e;
        atomicAdd(&mine[e], 1);
      }
    }
    if (bad) misc[0] = 1;
    lds_barrier();
    // Wave 0: totals, each wave's exclusive prefix in place, the exclusive
    // offsets over experts, and the experts of the tile's first and last slot.
    if (wave == 0) {
      const int q_last = q0 + nr - 1;
      int carry = 0;
      for (int e0 = 0; e0 < N; e0 += kWave) {
        const int e = e0 + lane;
        int tot = 0;
        if (e < N) {
          // all eight counts read before any is overwritten, so the reads go
          // out together
          int cw[kWavesW];
#pragma unroll
          for (int w = 0; w < kWavesW; ++w) cw[w] = wcnt[w * N + e];
#pragma unroll
          for (int w = 0; w < kWavesW; ++w) {
            wcnt[w * N + e] = tot;
            tot += cw[w];
          }
        }
        const int incl = wave_incl_scan(tot);
        const int run = carry + incl - tot;
        if (e < N) {
          cnt[e] = run;
          if (tile == 0) a.rt.offsets[e] = run;
          if (run <= q0 && q0 < run + tot) misc[1] = e;
          if (run <= q_last && q_last < run + tot) misc[2] = e;
        }
        carry += __builtin_amdgcn_readlane(incl, kWave - 1);
      }
      if (lane == 0) {
        cnt[N] = a.M;
        if (tile == 0) {
          a.rt.offsets[N] = a.M;
          *a.status = misc[0] ? BMOE_E_EXPERT : BMOE_OK;
        }
      }
    }
    lds_barrier();
  }
  const int e_first = misc[1], e_last = misc[2];
  // Both sides' angles of the two tables, in flight during the ranking.
  const bool two = e_last != e_first;                    // a second table is needed
  float4 th[NTB], ph[NTB];
#pragma unroll
  for (int i = 0; i < NTB; ++i) {
    int ex, s, p0;
    th[i] = ph[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (TableJob<D>::at(i, tid, ex, s, p0) && (ex == 0 || two)) {
      const size_t src = (size_t)(ex ? e_last : e_first) * C::TBL + s * C::P + p0;
      th[i] = *reinterpret_cast<const float4*>(a.theta + src);
      if constexpr (kOut) ph[i] = *reinterpret_cast<const float4*>(a.phi + src);
    }
  }
  // Stable ranks of the tile's experts: an id's slot is its expert's offset,
  // plus that expert's ids in earlier waves, earlier lanes of this wave and
  // earlier positions of this thread.
  if constexpr (ROUTE) {
    for (int e = e_first; e <= e_last; ++e) {
      if (cnt[e + 1] == cnt[e]) continue;  // uniform: no ids of e
      const int w_lo = wcnt[wave * N + e];
      const int w_hi = wave + 1 < kWavesW ? wcnt[(wave + 1) * N + e] : cnt[e + 1] - cnt[e];
      if (w_hi <= q0 - cnt[e] || w_lo >= q0 + nr - cnt[e]) continue;  // uniform per wave
      int below = 0;
#pragma unroll
      for (int j = 0; j < kIdsW; ++j) {
        const uint64_t m = __ballot(j < nv && id[j] == e);
        below += __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                           __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
      }
      int q = cnt[e] + w_lo + below - q0;
#pragma unroll
      for (int j = 0; j < kIdsW; ++j) {
        if (j < nv && id[j] == e) {
          if ((unsigned)q < (unsigned)nr) {
            sh_e[q] = e;
            sh_r[q] = i0 + j;
          }
          ++q;
        }
      }
    }
    lds_barrier();  // ranks are in; the routing scratch is dead from here on
    if (tid < nr) {
      const int r = sh_r[tid];
      a.rt.perm[q0 + tid] = r;
      a.rt.inv[r] = q0 + tid;
      a.rt.slot_e[q0 + tid] = sh_e[tid];
    }
  }

  // ---- this wave's rows: x, gates -----------------------------------------
  int ew[kRowsW], rw[kRowsW];
  uint4 xraw[kRowsW];
  float gw[kRowsW];
#pragma unroll
  for (int i = 0; i < kRowsW; ++i) {
    const int q = wave * kRowsW + i;
    const int qq = q < nr ? q : nr - 1;  // rows past the end repeat the last one
    ew[i] = sh_e[qq];
    rw[i] = sh_r[qq];
    const uint16_t* xr = a.x + (size_t)(rw[i] / a.k) * D + VPL * rl;
    if constexpr (VPL == 8) {
      xraw[i] = *reinterpret_cast<const uint4*>(xr);
    } else {
      const uint2 t = *reinterpret_cast<const uint2*>(xr);
      xraw[i] = make_uint4(t.x, t.y, 0u, 0u);
    }
    gw[i] = kOut ? a.gates[rw[i]] : 0.f;
  }
  // Input-side tables of the tile's first and last experts (the output
  // side's are computed during the product).
#pragma unroll
  for (int i = 0; i < NTB; ++i) write_table_chunk<D>(i, th[i], tpos[i], tin, two, tid);
  lds_barrier();

  // ---- butterfly-in, Z rows into the A tile --------------------------------
  float v[kRowsW][VPL];
#pragma unroll
  for (int i = 0; i < kRowsW; ++i) {
    const uint32_t w4[4] = {xraw[i].x, xraw[i].y, xraw[i].z, xraw[i].w};
#pragma unroll
    for (int r = 0; r < VPL; r += 2) {
      v[i][r] = bf16_lo(w4[r / 2]);
      v[i][r + 1] = bf16_hi(w4[r / 2]);
    }
  }
  butterfly_rows<D, true>(v, ew, e_first, e_last, tin_first, tin_last, a.theta, rl);
  // Row q's 16-byte chunk c sits at chunk c ^ (q & 15) (conflict-free A reads).
  uint4 zpk[kRowsW];  // this lane's bf16 Z values of each row
#pragma unroll
  for (int i = 0; i < kRowsW; ++i) {
    const int q = wave * kRowsW + i;
    const int e0 = VPL * rl;
    char* dst = zt + q * (2 * D) + 16 * ((e0 / 8) ^ (q & 15)) + 2 * (e0 % 8);
    if constexpr (VPL == 8) {
      zpk[i] = make_uint4(pack_bf16x2(v[i][0], v[i][1]), pack_bf16x2(v[i][2], v[i][3]),
                          pack_bf16x2(v[i][4], v[i][5]), pack_bf16x2(v[i][6], v[i][7]));
      *reinterpret_cast<uint4*>(dst) = zpk[i];
    } else {
      zpk[i] = make_uint4(pack_bf16x2(v[i][0], v[i][1]), pack_bf16x2(v[i][2], v[i][3]), 0u, 0u);
      *reinterpret_cast<uint2*>(dst) = make_uint2(zpk[i].x, zpk[i].y);
    }
  }
  // This wave's substrate rows have landed (its own copies only: no other
  // wave reads them), and every wave's A rows are in.
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_barrier();
  if constexpr ((OUT & kZH) != 0) {
    // Z rows for the backward, stored while the product runs.
#pragma unroll
    for (int i = 0; i < kRowsW; ++i) {
      const int q = wave * kRowsW + i;
      if (q >= nr) continue;
      uint16_t* zg = a.z + (size_t)(q0 + q) * D + VPL * rl;
      if constexpr (VPL == 8) *reinterpret_cast<uint4*>(zg) = zpk[i];
      else *reinterpret_cast<uint2*>(zg) = make_uint2(zpk[i].x, zpk[i].y);
    }
  }

  // ---- substrate product: product wave w (w < PWAVES) computes all 32 rows
  // x columns [w * PWN, (w + 1) * PWN) on v_mfma_f32_32x32x16_bf16; the
  // other waves write their share of the output-side tables meanwhile.
  f32x16 acc[C::PFN];
  const int ra = lane & 31;
  if (wave < C::PWAVES) {
#pragma unroll
    for (int j = 0; j < C::PFN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
    // this wave's columns: the substrate rows copied by waves
    // (PWN / WN) w .., consecutive in P; each copy's chunk swizzle is by its
    // own row (R mod WN)
    const char* const pwp = pst + wave * C::PWN * C::ROWB;
    // B operand: lane l takes, in K-step ks, word 2 ks + (l >> 5) of W row
    // o = wave * PWN + 32 j + (l & 31) (K values 32 ks + 16 (l >> 5) .. + 15);
    // the step's two MFMAs take its low and high eight values, and their A
    // fragments the same K values.
#pragma unroll
    for (int ks = 0; ks < C::NSTEP; ++ks) {
      uint32_t pw[C::PFN];
#pragma unroll
      for (int j = 0; j < C::PFN; ++j) {
        const int R = 32 * j + ra, w = 2 * ks + (lane >> 5);
        pw[j] = *reinterpret_cast<const uint32_t*>(
            pwp + R * C::ROWB + 16 * ((w / 4) ^ C::pw_swz(R % C::WN)) + 4 * (w % 4));
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // K values 32 ks + 16 (lane >> 5) + 8 h .. + 7: 16-byte chunk ca of row ra
        const int ca = 4 * ks + 2 * (lane >> 5) + h;
        const bf16x8 av =
            *reinterpret_cast<const bf16x8*>(zt + ra * (2 * D) + 16 * (ca ^ (ra & 15)));
#pragma unroll
        for (int j = 0; j < C::PFN; ++j) {
          const bf16x8 b = unpack_frag(pw[j], h);
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b, acc[j], 0, 0, 0);
        }
      }
      // One chunk per K-step: VALU work beside the matrix cores (no one reads
      // this region before the barrier that follows the H rows).
      if constexpr (kOut) {
        if (ks < NTB) write_table_chunk<D>(ks, ph[ks], tpos[ks], tout, two, tid);
      }
    }
  } else if constexpr (kOut) {
#pragma unroll
    for (int i = 0; i < NTB; ++i) write_table_chunk<D>(i, ph[i], tpos[i], tout, two, tid);
  }
  lds_barrier();  // every wave is done with Z and P, which the H rows reuse
  // alpha * H -> fp32 rows (32x32 block layout: lane l, register r -> row
  // 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32).
  if (wave < C::PWAVES) {
#pragma unroll
    for (int j = 0; j < C::PFN; ++j) {
      const int col = wave * C::PWN + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        hrow(row)[col ^ C::hswz(row)] = a.alpha * acc[j][r];
      }
    }
  }
  lds_barrier();  // the H rows are complete

  // ---- butterfly-out, gate, g * U rows in routed order ---------------------
#pragma unroll
  for (int i = 0; i < kRowsW; ++i) {
    const int q = wave * kRowsW + i;
    const float* hr = hrow(q) + ((VPL * rl) ^ C::hswz(q));
#pragma unroll
    for (int r = 0; r < VPL; r += 4) {
      const float4 t = *reinterpret_cast<const float4*>(hr + r);
      v[i][r] = t.x;
      v[i][r + 1] = t.y;
      v[i][r + 2] = t.z;
      v[i][r + 3] = t.w;
    }
  }
  if constexpr ((OUT & kZH) != 0) {
    // H rows (alpha * the product, rounded to bf16) for the backward.
#pragma unroll
    for (int i = 0; i < kRowsW; ++i) {
      const int q = wave * kRowsW + i;
      if (q >= nr) continue;
      uint16_t* hg = a.h + (size_t)(q0 + q) * D + VPL * rl;
      if constexpr (VPL == 8) {
        *reinterpret_cast<uint4*>(hg) =
            make_uint4(pack_bf16x2(v[i][0], v[i][1]), pack_bf16x2(v[i][2], v[i][3]),
                       pack_bf16x2(v[i][4], v[i][5]), pack_bf16x2(v[i][6], v[i][7]));
      } else {
        *reinterpret_cast<uint2*>(hg) =
            make_uint2(pack_bf16x2(v[i][0], v[i][1]), pack_bf16x2(v[i][2], v[i][3]));
      }
    }
  }
  if constexpr (!kOut) return;
  butterfly_rows<D, false>(v, ew, e_first, e_last, tout_first, tout_last, a.phi, rl);
#pragma unroll
  for (int i = 0; i < kRowsW; ++i) {
    const int q = wave * kRowsW + i;
    if (q >= nr) continue;
    const float g = gw[i];
    uint16_t* dst = a.u + (size_t)rw[i] * D + VPL * rl;
    if constexpr (VPL == 8) {
      *reinterpret_cast<uint4*>(dst) =
          make_uint4(pack_bf16x2(g * v[i][0], g * v[i][1]), pack_bf16x2(g * v[i][2], g * v[i][3]),
                     pack_bf16x2(g * v[i][4], g * v[i][5]), pack_bf16x2(g * v[i][6], g * v[i][7]));
    } else {
      *reinterpret_cast<uint2*>(dst) =
          make_uint2(pack_bf16x2(g * v[i][0], g * v[i][1]), pack_bf16x2(g * v[i][2], g * v[i][3]));
    }
  }
}

template <int D, bool ROUTE, int OUT = kU>
hipError_t launch_w(const WaveArgs& a, hipStream_t s, const KernelTiming& t) {
  return launch_kernel(fused_wave_kernel<D, ROUTE, OUT>, dim3((a.M + kSlots - 1) / kSlots),
                       dim3(WG<D>::THREADS), 0, s, t, a);
}

}  // namespace

bool fused_supported(bmoe_dtype dt, int d) {
  return dt == BMOE_BF16 && (d == 256 || d == 512);
}

bool fused_wave_routes(bmoe_dtype dt, int M, int d, int N) {
  return dt == BMOE_BF16 && (d == 256 || d == 512) && M <= kMaxMW &&
         N <= (d == 512 ? WG<512>::MAX_N : WG<256>::MAX_N);
}

hipError_t launch_fused_wave(int M, int d, int k, int N, const void* x, const int32_t* ids,
                             const float* gates, const float* theta, const float* phi,
                             const uint32_t* wp, float alpha, void* u, const RouteTables& rt,
                             int32_t* status, hipStream_t s, const KernelTiming& t) {
  if (!fused_wave_routes(BMOE_BF16, M, d, N)) return hipErrorInvalidValue;
  WaveArgs a{};
  a.M = M;
  a.k = k;
  a.N = N;
  a.x = static_cast<const uint16_t*>(x);
  a.ids = ids;
  a.gates = gates;
  a.theta = theta;
  a.phi = phi;
  a.wp = wp;
  a.alpha = substrate_scale(alpha);
  a.u = static_cast<uint16_t*>(u);
  a.rt = rt;
  a.status = status;
  switch (d) {
    case 256: return launch_w<256, true>(a, s, t);
    case 512: return launch_w<512, true>(a, s, t);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fused_wave_prepped(int M, int d, int k, const void* x, const float* gates,
                                     const float* theta, const float* phi, const uint32_t* wp,
                                     float alpha, void* u, void* z, void* h,
                                     const RouteTables& rt, hipStream_t s,
                                     const KernelTiming& t) {
  if (M <= 0) return hipSuccess;
  if (!u && !(z && h)) return hipErrorInvalidValue;
  if (!z != !h) return hipErrorInvalidValue;
  WaveArgs a{};
  a.M = M;
  a.k = k;
  a.x = static_cast<const uint16_t*>(x);
  a.gates = gates;
  a.theta = theta;
  a.phi = phi;
  a.wp = wp;
  a.alpha = substrate_scale(alpha);
  a.u = static_cast<uint16_t*>(u);
  a.z = static_cast<uint16_t*>(z);
  a.h = static_cast<uint16_t*>(h);
  a.rt = rt;
  const int out = (u ? kU : 0) | (z ? kZH : 0);
  switch (d * 4 + out) {
    case 256 * 4 + kU: return launch_w<256, false, kU>(a, s, t);
    case 256 * 4 + kZH: return launch_w<256, false, kZH>(a, s, t);
    case 256 * 4 + (kU | kZH): return launch_w<256, false, kU | kZH>(a, s, t);
    case 512 * 4 + kU: return launch_w<512, false, kU>(a, s, t);
    case 512 * 4 + kZH: return launch_w<512, false, kZH>(a, s, t);
    case 512 * 4 + (kU | kZH): return launch_w<512, false, kU | kZH>(a, s, t);
  }
  return hipErrorInvalidValue;
}

}  // namespace bmoe
