// Fused ButterflyMoE expert forward for d <= 512 (bf16 activations), one
// workgroup per 32 consecutive sorted routed rows (ButterflyMoE gist.science
// summary, §2.3: rotate by B(theta_e)^T, ternary product with the shared
// W_base, rotate by B(phi_e); nothing per expert is ever materialised):
//
//   gather x rows -> LDS (fp32)        butterfly-in, register blocks of 3 stages
//   -> bf16 A tile in LDS              substrate GEMM on MFMA 32x32x16, the bf16
//                                      substrate of the last K-steps streamed
//                                      through a global->LDS ring
//   -> alpha * H back into LDS (fp32)  butterfly-out
//   -> g_r * row, bf16, in routed order (the combine kernel sums the k rows).
//
// LDS (160 KiB at d = 512): four stage arrays and the A tile, each its own
// array so the compiler can tell the stage being read from the stages the
// DMA is filling. The fp32 rows live inside stages 1..3 (14 rows per stage;
// they are used only before and after the GEMM). The ring uses stages 0..2;
// stage 3 keeps the last rows, the row metadata and, for a tile of more than
// one expert, the last expert's coefficient table. The first K-steps of the
// GEMM take the substrate from packed words in registers, which leaves time
// for the ring to fill after the rows are dead.
//
// Routed variant (no preparation launch, M <= 8192 and N <= 512): every
// workgroup reads all expert ids, builds the per-expert counts and offsets in
// LDS, and ranks only the rows of its own tile (stable: ascending routed
// index inside an expert). It computes the cos/sin tables of the tile's first
// expert (stage 0) and last expert (stage 3) itself, in-side before the first
// butterfly and out-side after it; rows of any expert in between take their
// coefficients straight from the angles. All K-steps then come from the
// packed words (there is no bf16 substrate copy). It writes the same routing
// tables as the preparation kernel.
#include "common.h"
#include "kernels.h"

namespace bmoe {
namespace {

constexpr int kThreads = 512;  // 8 waves: two per SIMD
constexpr int kWavesF = kThreads / 64;
constexpr int kBM = 32;
// Routed variant: ids per thread (M <= kRouteIds * kThreads) and experts.
constexpr int kRouteIds = 16;
constexpr int kRouteMaxM = kRouteIds * kThreads;
constexpr int kRouteMaxN = 512;

__device__ __forceinline__ int padi(int i) { return i + (i >> 3); }


// Sorted slot q of a tile lives in LDS row row_of_slot(q). The butterfly
// threads of phase p rotate rows p, p + 8, p + 16 and p + 24 (three-stage
// groups at d = 512), which then hold the four consecutive slots 4p .. 4p+3:
// the rows of one thread, and of one wave, stay inside one expert wherever
// the tile's expert boundary allows. Any permutation is correct; this one
// keeps each thread's slots ascending.
static_assert(kBM == 32, "the slot permutation is written for 32-row tiles");
__device__ __forceinline__ int row_of_slot(int q) { return 8 * (q % 4) + q / 4; }
__device__ __forceinline__ int slot_of_row(int l) { return 4 * (l % 8) + l / 8; }

template <int D>
struct FCfg {
  static constexpr int L = D == 128 ? 7 : D == 256 ? 8 : 9;
  static constexpr int PD = D + D / 8;              // padded fp32 row (floats)
  static constexpr int KS = 32;                     // K per GEMM step
  static constexpr int NSTEP = D / KS;
  // The first NP steps take B from the packed 2-bit words (registers, VALU
  // expansion); the last NR steps from the bf16 substrate via the ring.
  // Splitting K balances VALU against L2 bandwidth: with every CU streaming
  // the substrate at once, bf16 alone is L2-bound, packed alone VALU-bound.
  // At most three ring steps, so ring stage 3 is never used by the ring: it
  // keeps the last rows, the row metadata and one expert's coefficient table.
  static constexpr int NR = NSTEP / 4 < 3 ? NSTEP / 4 : 3;
  static constexpr int NP = NSTEP - NR;
  static constexpr int STAGE_BYTES = D * KS * 2;    // D rows of 64 bytes
  static constexpr int NSTAGE = 4;
  static constexpr int ZT_BYTES = kBM * D * 2;
  static constexpr int ROW_BYTES = PD * 4;
  static constexpr int RPS = STAGE_BYTES / ROW_BYTES;  // rows per stage array
  // Row metadata (expert, routed index) after the last row in stage 3.
  static constexpr int META_OFF = (kBM - 2 * RPS) * ROW_BYTES;
  // One side's cos/sin table of one expert (L * D/2 pairs), in stage 3 after
  // the metadata: the tile's last expert when the tile holds more than one.
  static constexpr int TAB_BYTES = L * (D / 2) * 8;
  static constexpr int TAB_OFF = (META_OFF + 2 * kBM * 4 + 1023) / 1024 * 1024;
  static constexpr int WN = D / kWavesF;            // output columns per wave
  static constexpr int FN = WN / 32;
  static constexpr int LPW = STAGE_BYTES / 1024 / kWavesF;  // 1 KiB wave loads per wave per stage
  static_assert(FN >= 1 && LPW >= 1, "d too small for this tiling");
  static_assert(3 * RPS >= kBM && 2 * RPS < kBM, "rows must end in ring stage 3");
  static_assert(NR >= 1 && NR <= 3, "ring steps must leave stage 3 free");
  static_assert(TAB_OFF + TAB_BYTES <= STAGE_BYTES && TAB_BYTES % 1024 == 0,
                "metadata and one coefficient table must fit in stage 3");
};

// fp32 row i inside ring stages 1..3.
template <int D>
struct RowMap {
  char* s1;
  char* s2;
  char* s3;
  __device__ __forceinline__ float* row(int i) const {
    using C = FCfg<D>;
    char* b = i < C::RPS ? s1 : (i < 2 * C::RPS ? s2 : s3);
    return reinterpret_cast<float*>(b + (i % C::RPS) * C::ROW_BYTES);
  }
};

// Stage groups of one butterfly side. Input side (transpose): stages from
// L-1 down in threes; output side: from 0 up.
template <int D, bool TR>
struct Groups {
  static constexpr int L = FCfg<D>::L;
  static constexpr int N = (L + 2) / 3;
  static constexpr int s_hi(int g) { return TR ? L - 1 - 3 * g : (3 * g + 2 < L ? 3 * g + 2 : L - 1); }
  static constexpr int s_lo(int g) { return TR ? (L - 3 - 3 * g > 0 ? L - 3 - 3 * g : 0) : 3 * g; }
  static constexpr int G(int g) { return s_hi(g) - s_lo(g) + 1; }
};

template <int G, bool TR>
__device__ __forceinline__ void rotate(float (&v)[8], const float2 (&c)[3][4]) {
#pragma unroll
  for (int tt = 0; tt < G; ++tt) {
    const int t = TR ? G - 1 - tt : tt;
#pragma unroll
    for (int u = 0; u < (1 << (G - 1)); ++u) {
      const int m = ((u >> t) << (t + 1)) | (u & ((1 << t) - 1));
      const int n = m + (1 << t);
      const float a = v[m], b = v[n];
      const float cc = c[t][u].x, ss = c[t][u].y;
      if (TR) {
        v[m] = cc * a + ss * b;
        v[n] = cc * b - ss * a;
      } else {
        v[m] = cc * a - ss * b;
        v[n] = ss * a + cc * b;
      }
    }
  }
}

// Coefficients of one block (base index) for stage group (s_lo, G) of expert e.
template <int D, int G>
__device__ __forceinline__ void load_coef(float2 (&c)[3][4], const float2* cs, int e, int s_lo,
                                          int base) {
  constexpr int L = FCfg<D>::L;
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

// The same coefficients from an expert's table copied to LDS (pair order).
template <int D, int G>
__device__ __forceinline__ void load_coef_lds(float2 (&c)[3][4], const float2* tab, int s_lo,
                                              int base) {
#pragma unroll
  for (int t = 0; t < G; ++t) {
    const int s = s_lo + t;
#pragma unroll
    for (int u = 0; u < (1 << (G - 1)); ++u) {
      const int m = ((u >> t) << (t + 1)) | (u & ((1 << t) - 1));
      c[t][u] = tab[s * (D / 2) + pair_index(base + (m << s_lo), s)];
    }
  }
}

// Expert e's table of one side (contiguous) -> LDS at dst, 1 KiB per wave
// instruction (global->LDS DMA; completion is tracked by vmcnt).
template <int D>
__device__ __forceinline__ void table_load(char* dst, const float2* cs, int e) {
  using C = FCfg<D>;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const char* src = reinterpret_cast<const char*>(cs + (size_t)e * C::L * (D / 2));
  for (int ch = wave; ch < C::TAB_BYTES / 1024; ch += kWavesF)
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)(src + ch * 1024 + lane * 16),
        (__attribute__((address_space(3))) void*)(dst + ch * 1024), 16, 0, 0);
}

// Butterfly side over the kBM rows in LDS. Each thread owns one block per
// group and every tpb-th row; its coefficients are fetched up front for the
// expert of its first row (prefetch) and reloaded only when the expert of a
// later row differs (rows are sorted by expert): from the LDS copy of expert
// e_tab's table when the row belongs to it, else from global memory.
template <int D, bool TR, bool RT = false>
struct BflyCoef {
  using Gr = Groups<D, TR>;
  float2 c[Gr::N][3][4];
  int e[Gr::N];
  // Routed variant: expert e_a's table in LDS at tab_a (the last expert's is
  // the e_tab table). The n_mid experts listed at mid (those of the tile
  // between its first and last) have no table: after each stage group's
  // main pass the workgroup writes that group's part of one of their tables
  // to `scratch` and rotates its rows from there.
  const float* ang = nullptr;
  const float2* tab_a = nullptr;
  int e_a = -1;
  const int* mid = nullptr;
  int n_mid = 0;
  float2* scratch = nullptr;

  // Coefficients of group g for expert ei: from the LDS table of e_tab, else
  // (prep path) the global tables cs, else (routed) e_a's table; a routed
  // expert without a table marks the group as holding none.
  template <int G>
  __device__ __forceinline__ void fetch(int g, int ei, const float2* cs, const float2* tab,
                                        int e_tab, int s_lo, int base) {
    if constexpr (RT) {
      if (ei == e_tab || ei == e_a) load_coef_lds<D, G>(c[g], ei == e_tab ? tab : tab_a, s_lo, base);
      else e[g] = -1;
    } else if (ei == e_tab) {
      load_coef_lds<D, G>(c[g], tab, s_lo, base);
    } else {
      load_coef<D, G>(c[g], cs, ei, s_lo, base);
    }
  }

  // Routed variant: as prefetch_from_lanes, from the LDS tables.
  __device__ __forceinline__ void prefetch_tables(int lane_e, const float2* tab, int e_tab) {
#pragma unroll
    for (int g = 0; g < Gr::N; ++g) {
      const int G = Gr::G(g), s_lo = Gr::s_lo(g);
      const int nb = D >> G;
      const int base = block_base(threadIdx.x % nb, s_lo, G);
      e[g] = __shfl(lane_e, threadIdx.x / nb, 64);
      if (G == 3) fetch<3>(g, e[g], nullptr, tab, e_tab, s_lo, base);
      else if (G == 2) fetch<2>(g, e[g], nullptr, tab, e_tab, s_lo, base);
      else fetch<1>(g, e[g], nullptr, tab, e_tab, s_lo, base);
    }
  }

  // Coefficients of every group for the expert of the thread's first row,
  // read from lane i's `lane_e` for row i.
  __device__ __forceinline__ void prefetch_from_lanes(const float2* cs, int lane_e) {
#pragma unroll
    for (int g = 0; g < Gr::N; ++g) {
      const int G = Gr::G(g), s_lo = Gr::s_lo(g);
      const int nb = D >> G;
      const int base = block_base(threadIdx.x % nb, s_lo, G);
      e[g] = __shfl(lane_e, threadIdx.x / nb, 64);
      if (G == 3) load_coef<D, 3>(c[g], cs, e[g], s_lo, base);
      else if (G == 2) load_coef<D, 2>(c[g], cs, e[g], s_lo, base);
      else load_coef<D, 1>(c[g], cs, e[g], s_lo, base);
    }
  }

  template <int G>
  __device__ __forceinline__ void rotate_rows(const RowMap<D>& rows, const int* sh_e,
                                              const float2* cs, const float2* tab, int e_tab,
                                              int g, int s_lo, int base,
                                              const int (&off)[8], int ph, int tpb) {
    const int rpt = kBM / tpb;
    const int first = ph, last = ph + (rpt - 1) * tpb;
    if (sh_e[first] == e[g] && sh_e[last] == e[g]) {
      // Every row of this thread shares the cached expert: batches of four
      // rows keep several LDS loads in flight.
      for (int j0 = 0; j0 < rpt; j0 += 4) {
        float v[4][8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (j0 + q < rpt) {
            const float* row = rows.row(ph + (j0 + q) * tpb);
#pragma unroll
            for (int m = 0; m < (1 << G); ++m) v[q][m] = row[off[m]];
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) rotate<G, TR>(v[q], c[g]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (j0 + q < rpt) {
            float* row = rows.row(ph + (j0 + q) * tpb);
#pragma unroll
            for (int m = 0; m < (1 << G); ++m) row[off[m]] = v[q][m];
          }
        }
      }
      return;
    }
    for (int j = 0; j < rpt; ++j) {
      const int i = ph + j * tpb;
      const int ei = sh_e[i];
      if constexpr (RT) {
        if (ei != e_a && ei != e_tab) continue;  // a middle expert: its own pass
      }
      if (ei != e[g]) {
        e[g] = ei;
        fetch<G>(g, ei, cs, tab, e_tab, s_lo, base);
      }
      float* row = rows.row(i);
      float v[8];
#pragma unroll
      for (int m = 0; m < (1 << G); ++m) v[m] = row[off[m]];
      rotate<G, TR>(v, c[g]);
#pragma unroll
      for (int m = 0; m < (1 << G); ++m) row[off[m]] = v[m];
    }
  }

  // Routed variant: middle expert em's table of stages s_lo .. s_lo+G-1 in
  // `scratch`, computed by the whole workgroup as the tile tables are.
  __device__ __forceinline__ void mid_table(int em, int s_lo, int G) {
    constexpr int L = FCfg<D>::L;
    lds_barrier();  // the previous pass is done with scratch
    for (int j = threadIdx.x; j < G * (D / 2); j += kThreads) {
      const int t = j / (D / 2), p = j % (D / 2);
      scratch[j] = tile_cos_sin(ang[((size_t)em * L + s_lo + t) * (D / 2) + p]);
    }
    lds_barrier();
  }

  // Routed variant: this thread's rows of middle expert em for stage group
  // g, from its group table in `scratch`.
  template <int G>
  __device__ __forceinline__ void rotate_mid(const RowMap<D>& rows, const int* sh_e, int g,
                                             int em, int s_lo, int base, const int (&off)[8],
                                             int ph, int tpb) {
    const int rpt = kBM / tpb;
    for (int j = 0; j < rpt; ++j) {
      const int i = ph + j * tpb;
      if (sh_e[i] != em) continue;
      if (e[g] != em) {
        e[g] = em;
        load_coef_lds<D, G>(c[g], scratch - s_lo * (D / 2), s_lo, base);
      }
      float* row = rows.row(i);
      float v[8];
#pragma unroll
      for (int m = 0; m < (1 << G); ++m) v[m] = row[off[m]];
      rotate<G, TR>(v, c[g]);
#pragma unroll
      for (int m = 0; m < (1 << G); ++m) row[off[m]] = v[m];
    }
  }

  __device__ __forceinline__ void apply(const RowMap<D>& rows, const float2* cs,
                                        const int* sh_e, const float2* tab, int e_tab) {
#pragma unroll
    for (int g = 0; g < Gr::N; ++g) {
      const int G = Gr::G(g), s_lo = Gr::s_lo(g);
      const int nb = D >> G;
      const int tpb = kThreads / nb;
      const int b = threadIdx.x % nb, ph = threadIdx.x / nb;
      const int base = block_base(b, s_lo, G);
      int off[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) off[m] = padi(base + ((m & ((1 << G) - 1)) << s_lo));
      if (G == 3) rotate_rows<3>(rows, sh_e, cs, tab, e_tab, g, s_lo, base, off, ph, tpb);
      else if (G == 2) rotate_rows<2>(rows, sh_e, cs, tab, e_tab, g, s_lo, base, off, ph, tpb);
      else rotate_rows<1>(rows, sh_e, cs, tab, e_tab, g, s_lo, base, off, ph, tpb);
      if constexpr (RT) {
        for (int mi = 0; mi < n_mid; ++mi) {
          const int em = mid[mi];
          mid_table(em, s_lo, G);
          if (G == 3) rotate_mid<3>(rows, sh_e, g, em, s_lo, base, off, ph, tpb);
          else if (G == 2) rotate_mid<2>(rows, sh_e, g, em, s_lo, base, off, ph, tpb);
          else rotate_mid<1>(rows, sh_e, g, em, s_lo, base, off, ph, tpb);
        }
      }
      lds_barrier();
    }
  }
};

template <int D>
__device__ __forceinline__ void ring_load(char* stage, const uint16_t* w16, int step) {
  // step: global K-step index (K offset step * KS)
  using C = FCfg<D>;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
  for (int j = 0; j < C::LPW; ++j) {
    const int blk = wave * C::LPW + j;           // 1 KiB = 16 rows of 64 bytes
    const int o = blk * 16 + lane / 4;
    const int chunk = (lane % 4) ^ ((o >> 2) & 3);
    const uint16_t* g = w16 + (size_t)o * D + step * C::KS + chunk * 8;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                     (__attribute__((address_space(3))) void*)(stage + blk * 1024),
                                     16, 0, 0);
  }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// Routed variant: one side's cos/sin tables of the tile's first expert (ta)
// and, when e_tab >= 0, its last expert (tb) from that side's angles, which
// thread holds in ang[i] (entry tid + i * kThreads).
template <int TBL, int NTB>
__device__ __forceinline__ void write_tables(const float (&ang)[NTB], float2* ta, float2* tb,
                                             int e_tab) {
#pragma unroll
  for (int i = 0; i < NTB; ++i) {
    const int j = threadIdx.x + i * kThreads;
    if (j < TBL || e_tab >= 0) (j < TBL ? ta : tb)[j < TBL ? j : j - TBL] = tile_cos_sin(ang[i]);
  }
}

struct FusedArgs {
  int M, k, N;
  const uint16_t* x;
  const float* gates;
  float alpha;  // the kernel's scale for the +-2 substrate values
  const uint32_t* wp;
  uint16_t* u;
  // Preparation path: routing and cos/sin tables from the prep kernel, and
  // the bf16 substrate the ring streams.
  const int32_t* perm;
  const int32_t* slot_e;
  const float2* cs_in;
  const float2* cs_out;
  const uint16_t* w16;
  // Routed variant: ids and angles in; routing tables and status out.
  const int32_t* ids;
  const float* theta;
  const float* phi;
  RouteTables rt;
  int32_t* status;
};

template <int D, bool RT>
__global__ __launch_bounds__(kThreads) void fused_kernel(FusedArgs a) {
  using C = FCfg<D>;
  constexpr int NR = RT ? 0 : C::NR;  // ring K-steps
  constexpr int NP = C::NSTEP - NR;   // K-steps from packed words
  // Packed K-steps requested before the first butterfly (the routed variant
  // requests the rest after it).
  constexpr int NPE = RT ? C::NSTEP / 2 : C::NP;
  // Routed variant: one side's table entries of the tile's two experts,
  // kThreads-strided over the threads.
  constexpr int TBL = C::L * (D / 2);
  constexpr int NTB = 2 * TBL / kThreads;
  static_assert(!RT || (2 * TBL) % kThreads == 0, "table entries must split over the threads");
  static_assert(!RT || (C::TAB_BYTES <= C::STAGE_BYTES &&
                        kWavesF * kRouteMaxN * 4 <= C::STAGE_BYTES &&
                        (kRouteMaxN + 16) * 4 <= C::STAGE_BYTES),
                "routing scratch and the first expert's table must fit in a stage");
  __shared__ __attribute__((aligned(1024))) char st0[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char st1[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char st2[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char st3[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char zt[C::ZT_BYTES];
  RowMap<D> rows;
  rows.s1 = st1;
  rows.s2 = st2;
  rows.s3 = st3;
  auto stage = [&](int i) -> char* { return i == 0 ? st0 : i == 1 ? st1 : i == 2 ? st2 : st3; };
  int* const sh_e = reinterpret_cast<int*>(st3 + C::META_OFF);
  int* const sh_r = sh_e + kBM;
  int* const sh_mid = sh_r + kBM;  // routed: the tile's middle experts, then their count
  static_assert(C::META_OFF + (3 * kBM + 1) * 4 <= C::TAB_OFF, "row metadata overlaps the table");
  // The last expert's table when the tile holds more than one (stage 3); in
  // the routed variant also the first expert's (stage 0).
  const float2* const tab = reinterpret_cast<const float2*>(st3 + C::TAB_OFF);
  const float2* const tab_a = reinterpret_cast<const float2*>(st0);

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int q0 = blockIdx.x * kBM;
  const int nr = min(kBM, a.M - q0);
  // Lane l < 32 of every wave keeps the (expert, routed index) of LDS row l,
  // that is of slot slot_of_row(l), in registers (an LDS copy serves the
  // butterflies). Rows of slots past the end repeat the last slot (computed,
  // never stored).
  int my_e, my_r, e_tab, e_first = -1, e_last = -1;
  float th[RT ? NTB : 1];
  if constexpr (RT) {
    // ---- routing of this tile's rows -------------------------------------
    // Per-wave counts, then each wave's count of the ids before it (stage
    // 1), and the offsets (stage 2).
    int* const wcnt = reinterpret_cast<int*>(st1);  // [kWavesF][N]
    int* const cnt = reinterpret_cast<int*>(st2);   // [N + 1]
    int* const misc = cnt + kRouteMaxN + 4;         // bad id; first, last expert
    const int N = a.N;
    // Thread t owns ids [kRouteIds * t, +kRouteIds), nv of them valid.
    const int i0 = kRouteIds * tid;
    const int nv = max(0, min(kRouteIds, a.M - i0));
    int id[kRouteIds];
    if (nv == kRouteIds) {
#pragma unroll
      for (int j = 0; j < kRouteIds / 4; ++j) {
        const int4 v = reinterpret_cast<const int4*>(a.ids + i0)[j];
        id[4 * j] = v.x; id[4 * j + 1] = v.y; id[4 * j + 2] = v.z; id[4 * j + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kRouteIds; ++j) id[j] = j < nv ? a.ids[i0 + j] : 0;
    }
    for (int e = tid; e < kWavesF * N; e += kThreads) wcnt[e] = 0;
    if (tid == 0) {
      misc[0] = 0;
      misc[1] = 0;
      misc[2] = 0;
      sh_mid[kBM] = 0;
    }
    if (tid < kBM) {  // every slot is ranked below; valid indices regardless
      sh_e[tid] = 0;
      sh_r[tid] = 0;
    }
    lds_barrier();
    // Per-wave counts (ids outside [0, N) are clamped for addressing and
    // reported).
    bool bad = false;
    int* const mine = wcnt + wave * N;
#pragma unroll
    for (int j = 0; j < kRouteIds; ++j) {
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
    // offsets over experts (expert u * 64 + lane in pass u), and the experts
    // of the tile's first and last rows (exactly one non-empty expert holds
    // each sorted slot).
    if (wave == 0) {
      const int q_last = q0 + nr - 1;
      int carry = 0;
      for (int e0 = 0; e0 < N; e0 += kWave) {
        const int e = e0 + lane;
        int tot = 0;
        if (e < N) {
#pragma unroll
          for (int w = 0; w < kWavesF; ++w) {
            const int c = wcnt[w * N + e];
            wcnt[w * N + e] = tot;
            tot += c;
          }
        }
        int incl = tot;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
          const int t = __shfl_up(incl, off, kWave);
          if (lane >= off) incl += t;
        }
        const int run = carry + incl - tot;
        if (e < N) {
          cnt[e] = run;
          if (blockIdx.x == 0) a.rt.offsets[e] = run;
          if (run <= q0 && q0 < run + tot) misc[1] = e;
          if (run <= q_last && q_last < run + tot) misc[2] = e;
        }
        carry += __shfl(incl, kWave - 1, kWave);
      }
      if (lane == 0) {
        cnt[N] = a.M;
        if (blockIdx.x == 0) {
          a.rt.offsets[N] = a.M;
          *a.status = misc[0] ? BMOE_E_EXPERT : BMOE_OK;
        }
      }
    }
    lds_barrier();
    e_first = misc[1];
    e_last = misc[2];
    e_tab = e_last != e_first ? e_last : -1;
    // The in-side angles of the two tables, in flight during the ranking.
#pragma unroll
    for (int i = 0; i < NTB; ++i) {
      const int j = tid + i * kThreads;
      th[i] = a.theta[j < TBL ? (size_t)e_first * TBL + j : (size_t)e_last * TBL + (j - TBL)];
    }
    // The non-empty experts strictly between the first and the last (all
    // their rows lie inside the tile), in any order.
    for (int e = e_first + 1 + tid; e < e_last; e += kThreads)
      if (cnt[e + 1] > cnt[e]) {
        const int at = atomicAdd(&sh_mid[kBM], 1);  // < nr - 2: each has a row here
        if (at < kBM) sh_mid[at] = e;
      }
    // Stable ranks of the tile's experts: the sorted slot of an id is its
    // expert's offset, plus that expert's ids in earlier waves, plus those in
    // earlier lanes of this wave and earlier positions of this thread.
    for (int e = e_first; e <= e_last; ++e) {
      if (cnt[e + 1] == cnt[e]) continue;  // uniform: no ids of e
      // This wave's ids of e rank in [w_lo, w_hi) within e; the tile needs
      // ranks [q0 - cnt[e], q0 + nr - cnt[e]). Waves outside skip (uniform
      // per wave).
      const int w_lo = wcnt[wave * N + e];
      const int w_hi = wave + 1 < kWavesF ? wcnt[(wave + 1) * N + e] : cnt[e + 1] - cnt[e];
      if (w_hi <= q0 - cnt[e] || w_lo >= q0 + nr - cnt[e]) continue;
      // ids of e held by lower lanes of this wave (every position)
      int below = 0;
#pragma unroll
      for (int j = 0; j < kRouteIds; ++j) {
        const uint64_t m = __ballot(j < nv && id[j] == e);
        below += __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                           __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
      }
      int q = cnt[e] + w_lo + below - q0;
#pragma unroll
      for (int j = 0; j < kRouteIds; ++j) {
        if (j < nv && id[j] == e) {
          if ((unsigned)q < (unsigned)nr) {
            sh_e[row_of_slot(q)] = e;
            sh_r[row_of_slot(q)] = i0 + j;
          }
          ++q;
        }
      }
    }
    lds_barrier();
    // Lane l < 32 holds LDS row l (slot sl); rows of slots past nr repeat
    // the last slot.
    const int sl = slot_of_row(lane & 31);
    const int li = sl < nr ? (lane & 31) : row_of_slot(nr - 1);
    my_e = sh_e[li];
    my_r = sh_r[li];
    if (tid < kBM) {
      if (sl < nr) {
        a.rt.perm[q0 + sl] = my_r;
        a.rt.inv[my_r] = q0 + sl;
        a.rt.slot_e[q0 + sl] = my_e;
      } else {
        sh_e[tid] = my_e;
        sh_r[tid] = my_r;
      }
    }
  } else {
    const int q_meta = q0 + min(slot_of_row(lane & 31), nr - 1);
    my_e = a.slot_e[q_meta];
    my_r = a.perm[q_meta];
    if (tid < kBM) {
      sh_e[tid] = my_e;
      sh_r[tid] = my_r;
    }
    // A tile holding more than one expert copies its last expert's tables to
    // LDS (each side before that side's butterfly), so the rows of that
    // expert reload their coefficients from LDS rather than from global
    // memory.
    e_tab = __shfl(my_e, 0, 64) != __shfl(my_e, kBM - 1, 64) ? __shfl(my_e, kBM - 1, 64) : -1;
    if (e_tab >= 0) table_load<D>(st3 + C::TAB_OFF, a.cs_in, e_tab);
    __asm__ volatile("" ::: "memory");
  }
  const int my_t = my_r / a.k;
  // Routed: lane i holds row i's gate, requested now (it is long in by the
  // stores).
  float my_g = 0.f;
  if constexpr (RT) my_g = a.gates[my_r];

  // Gather x rows (8 bf16 per 16-byte chunk) into registers and fetch the
  // butterfly-in coefficients. Token indices come from the lanes holding them
  // (no LDS round trip). Tail rows past nr repeat the last row: computed,
  // never stored.
  constexpr int CPR = D / 8;
  constexpr int XPT = kBM * CPR / kThreads;
  uint4 xv[XPT];
#pragma unroll
  for (int it = 0; it < XPT; ++it) {
    const int c = tid + it * kThreads;
    const int i = c / CPR, ch = c % CPR;
    const int t = __shfl(my_t, i, 64);
    xv[it] = *reinterpret_cast<const uint4*>(a.x + (size_t)t * D + ch * 8);
  }
  BflyCoef<D, true, RT> cin;
  if constexpr (RT) {
    // In-side tables: the first expert's in stage 0, the last expert's (if
    // different) in stage 3, in the prep kernel's layout and arithmetic.
    write_tables<TBL, NTB>(th, reinterpret_cast<float2*>(st0),
                           reinterpret_cast<float2*>(st3 + C::TAB_OFF), e_tab);
    lds_barrier();
    cin.ang = a.theta;
    cin.tab_a = tab_a;
    cin.e_a = e_first;
    cin.mid = sh_mid;
    cin.n_mid = sh_mid[kBM];
    cin.scratch = reinterpret_cast<float2*>(zt);  // free until the A tile is written
    cin.prefetch_tables(my_e, tab, e_tab);
  } else {
    cin.prefetch_from_lanes(a.cs_in, my_e);
  }
#pragma unroll
  for (int it = 0; it < XPT; ++it) {
    const int c = tid + it * kThreads;
    const int i = c / CPR, ch = c % CPR;
    float* dst = rows.row(i) + padi(ch * 8);
    const uint4 v = xv[it];
    dst[0] = bf16_lo(v.x); dst[1] = bf16_hi(v.x); dst[2] = bf16_lo(v.y); dst[3] = bf16_hi(v.y);
    dst[4] = bf16_lo(v.z); dst[5] = bf16_hi(v.z); dst[6] = bf16_lo(v.w); dst[7] = bf16_hi(v.w);
  }
  if (!RT && e_tab >= 0) wait_vm<0>();  // this wave's part of the table has landed
  __syncthreads();
  // The packed substrate words of the first NPE K-steps, for the GEMM (the
  // routed variant requests the rest after the first butterfly). Lane l needs W rows o = wave*WN + 32j + (l & 31), two words
  // per K-step.
  uint2 pw[NP][C::FN];
#pragma unroll
  for (int ks = 0; ks < NPE; ++ks)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int o = wave * C::WN + j * 32 + (lane & 31);
      pw[ks][j] = *reinterpret_cast<const uint2*>(a.wp + (size_t)o * (D / 16) + 2 * ks);
    }

  cin.apply(rows, a.cs_in, sh_e, tab, e_tab);

  // fp32 rows -> bf16 A tile, 16-byte chunk c of row r at chunk c ^ (r & 15).
#pragma unroll
  for (int it = 0; it < XPT; ++it) {
    const int c = tid + it * kThreads;
    const int r = c / CPR, ch = c % CPR;
    const float* s = rows.row(r) + padi(ch * 8);
    *reinterpret_cast<uint4*>(zt + r * (2 * D) + 16 * (ch ^ (r & 15))) =
        make_uint4(pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]), pack_bf16x2(s[4], s[5]),
                   pack_bf16x2(s[6], s[7]));
  }
  lds_barrier();  // rows are dead from here until the GEMM ends
  BflyCoef<D, false, RT> cout;
  float ph[RT ? NTB : 1];
  if constexpr (RT) {
    // The out-side angles of the two tables (their tables are computed
    // halfway through the GEMM) and the last packed K-steps.
#pragma unroll
    for (int i = 0; i < NTB; ++i) {
      const int j = tid + i * kThreads;
      ph[i] = a.phi[j < TBL ? (size_t)e_first * TBL + j : (size_t)e_last * TBL + (j - TBL)];
    }
#pragma unroll
    for (int ks = NPE; ks < NP; ++ks)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int o = wave * C::WN + j * 32 + (lane & 31);
        pw[ks][j] = *reinterpret_cast<const uint2*>(a.wp + (size_t)o * (D / 16) + 2 * ks);
      }
  } else {
    // Butterfly-out coefficients (for the expert of each thread's first row)
    // and then every ring stage are requested now; the packed K-steps run
    // while they land. Loads complete in issue order, so the coefficients go
    // first.
    cout.prefetch_from_lanes(a.cs_out, my_e);
    // The output side's table replaces the input side's (that butterfly is
    // done); it goes out before the ring, so it has landed once the ring has.
    if (e_tab >= 0) table_load<D>(st3 + C::TAB_OFF, a.cs_out, e_tab);
    __asm__ volatile("" ::: "memory");
    ring_load<D>(st0, a.w16, NP);
    if (NR > 1) ring_load<D>(st1, a.w16, NP + 1);
    if (NR > 2) ring_load<D>(st2, a.w16, NP + 2);
  }

  // ---- substrate GEMM: wave w computes rows 0..31 x columns [w*WN, (w+1)*WN)
  f32x16 acc[C::FN];
#pragma unroll
  for (int j = 0; j < C::FN; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;

  const int ra = lane & 31;
  // K-steps from the packed words.
#pragma unroll
  for (int ks = 0; ks < NP; ++ks) {
#pragma unroll
    for (int kk = 0; kk < C::KS; kk += 16) {
      const int ca = (ks * C::KS + kk) / 8 + (lane >> 5);
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(zt + ra * (2 * D) + 16 * (ca ^ (ra & 15)));
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const bf16x8 b = unpack_frag(kk == 0 ? pw[ks][j].x : pw[ks][j].y, lane >> 5);
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b, acc[j], 0, 0, 0);
      }
    }
    if constexpr (RT) {
      if (ks == NP / 2) {
        // Out-side tables in place of the in-side ones (that butterfly is
        // done), VALU work beside the other waves' MFMAs, then each thread's
        // butterfly-out coefficients for the rest of the GEMM to hide.
        write_tables<TBL, NTB>(ph, reinterpret_cast<float2*>(st0),
                               reinterpret_cast<float2*>(st3 + C::TAB_OFF), e_tab);
        lds_barrier();
        cout.ang = a.phi;
        cout.tab_a = tab_a;
        cout.e_a = e_first;
        cout.mid = sh_mid;
        cout.n_mid = sh_mid[kBM];
        cout.scratch = reinterpret_cast<float2*>(zt);  // free after the GEMM
        cout.prefetch_tables(my_e, tab, e_tab);
      }
    }
  }
  // K-steps from the bf16 ring.
#pragma unroll
  for (int rs = 0; rs < NR; ++rs) {
    // Stages requested after stage rs: rs+1 .. NR-1.
    const int after = NR - 1 - rs;
    if (after == 2) wait_vm<2 * C::LPW>();
    else if (after == 1) wait_vm<C::LPW>();
    else wait_vm<0>();
    lds_barrier();  // every wave's part of stage rs has landed
    const char* st = stage(rs);
    const int ks = NP + rs;
#pragma unroll
    for (int kk = 0; kk < C::KS; kk += 16) {
      const int ca = (ks * C::KS + kk) / 8 + (lane >> 5);
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(zt + ra * (2 * D) + 16 * (ca ^ (ra & 15)));
      const int cb = kk / 8 + (lane >> 5);
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int o = wave * C::WN + j * 32 + (lane & 31);
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(st + o * 64 + 16 * (cb ^ ((o >> 2) & 3)));
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b, acc[j], 0, 0, 0);
      }
    }
  }
  // Every wave is done with the ring: rows may be rewritten. (Without a ring
  // the GEMM reads only the A tile and the tables, which the rows do not
  // overlap.)
  if constexpr (!RT) __syncthreads();

  // alpha * H -> fp32 rows. 32x32 block layout: lane l, register r ->
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma unroll
  for (int j = 0; j < C::FN; ++j) {
    const int col = wave * C::WN + j * 32 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      rows.row(row)[padi(col)] = a.alpha * acc[j][r];
    }
  }
  // The rows are complete (the routed variant has no global loads left to
  // order here).
  if constexpr (RT) lds_barrier();
  else __syncthreads();

  cout.apply(rows, a.cs_out, sh_e, tab, e_tab);

  // g_r * row -> bf16, routed order.
#pragma unroll
  for (int it = 0; it < XPT; ++it) {
    const int c = tid + it * kThreads;
    const int i = c / CPR, ch = c % CPR;
    float g = 0.f;
    if constexpr (RT) g = __shfl(my_g, i, 64);
    if (slot_of_row(i) < nr) {
      const int r = sh_r[i];
      if constexpr (!RT) g = a.gates[r];
      const float* s = rows.row(i) + padi(ch * 8);
      *reinterpret_cast<uint4*>(a.u + (size_t)r * D + ch * 8) =
          make_uint4(pack_bf16x2(g * s[0], g * s[1]), pack_bf16x2(g * s[2], g * s[3]),
                     pack_bf16x2(g * s[4], g * s[5]), pack_bf16x2(g * s[6], g * s[7]));
    }
  }
}

template <int D, bool RT>
hipError_t launch_d(const FusedArgs& a, hipStream_t s, const KernelTiming& t) {
  return launch_kernel(fused_kernel<D, RT>, dim3((a.M + kBM - 1) / kBM), dim3(kThreads), 0, s, t,
                       a);
}

}  // namespace

bool fused_supported(bmoe_dtype dt, int d) {
  return dt == BMOE_BF16 && (d == 256 || d == 512);
}

bool fused_routes(bmoe_dtype dt, int M, int d, int N) {
  return fused_supported(dt, d) && M <= kRouteMaxM && N <= kRouteMaxN;
}

hipError_t launch_fused(int M, int d, int k, const void* x, const float* gates,
                        const RouteTables& rt, const float2* cs_in, const float2* cs_out,
                        const uint16_t* w16, const uint32_t* wp, float alpha, void* u,
                        hipStream_t s, const KernelTiming& t) {
  FusedArgs a{};
  a.M = M;
  a.k = k;
  a.x = static_cast<const uint16_t*>(x);
  a.gates = gates;
  a.alpha = substrate_scale(alpha);  // the kernel's substrate values are +-2
  a.wp = wp;
  a.u = static_cast<uint16_t*>(u);
  a.perm = rt.perm;
  a.slot_e = rt.slot_e;
  a.cs_in = cs_in;
  a.cs_out = cs_out;
  a.w16 = w16;
  switch (d) {
    case 256: return launch_d<256, false>(a, s, t);
    case 512: return launch_d<512, false>(a, s, t);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fused_routed(int M, int d, int k, int N, const void* x, const int32_t* ids,
                               const float* gates, const float* theta, const float* phi,
                               const uint32_t* wp, float alpha, void* u, const RouteTables& rt,
                               int32_t* status, hipStream_t s, const KernelTiming& t) {
  if (!fused_routes(BMOE_BF16, M, d, N)) return hipErrorInvalidValue;
  FusedArgs a{};
  a.M = M;
  a.k = k;
  a.N = N;
  a.x = static_cast<const uint16_t*>(x);
  a.gates = gates;
  a.alpha = substrate_scale(alpha);
  a.wp = wp;
  a.u = static_cast<uint16_t*>(u);
  a.ids = ids;
  a.theta = theta;
  a.phi = phi;
  a.rt = rt;
  a.status = status;
  switch (d) {
    case 256: return launch_d<256, true>(a, s, t);
    case 512: return launch_d<512, true>(a, s, t);
  }
  return hipErrorInvalidValue;
}

}  // namespace bmoe
