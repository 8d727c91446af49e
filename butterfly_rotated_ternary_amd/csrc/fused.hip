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
// This kernel runs after the preparation launch (routing and cos/sin tables),
// for batches the register-resident fused kernel does not route itself
// (M > 8192 or N > 512).
#include "common.h"
#include "kernels.h"

namespace bmoe {
namespace {

constexpr int kThreads = 512;  // 8 waves: two per SIMD
constexpr int kWavesF = kThreads / 64;
constexpr int kBM = 32;

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
template <int D, bool TR>
struct BflyCoef {
  using Gr = Groups<D, TR>;
  float2 c[Gr::N][3][4];
  int e[Gr::N];

  // Coefficients of group g for expert ei: from the LDS table of e_tab, else
  // the global tables cs.
  template <int G>
  __device__ __forceinline__ void fetch(int g, int ei, const float2* cs, const float2* tab,
                                        int e_tab, int s_lo, int base) {
    if (ei == e_tab) load_coef_lds<D, G>(c[g], tab, s_lo, base);
    else load_coef<D, G>(c[g], cs, ei, s_lo, base);
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

struct FusedArgs {
  int M, k;
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
};

template <int D>
__global__ __launch_bounds__(kThreads) void fused_kernel(FusedArgs a) {
  using C = FCfg<D>;
  constexpr int NR = C::NR;           // ring K-steps
  constexpr int NP = C::NSTEP - NR;   // K-steps from packed words
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
  static_assert(C::META_OFF + 2 * kBM * 4 <= C::TAB_OFF, "row metadata overlaps the table");
  // The last expert's table when the tile holds more than one (stage 3).
  const float2* const tab = reinterpret_cast<const float2*>(st3 + C::TAB_OFF);

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int q0 = blockIdx.x * kBM;
  const int nr = min(kBM, a.M - q0);
  // Lane l < 32 of every wave keeps the (expert, routed index) of LDS row l,
  // that is of slot slot_of_row(l), in registers (an LDS copy serves the
  // butterflies). Rows of slots past the end repeat the last slot (computed,
  // never stored).
  int my_e, my_r, e_tab;
  {
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
  BflyCoef<D, true> cin;
  cin.prefetch_from_lanes(a.cs_in, my_e);
#pragma unroll
  for (int it = 0; it < XPT; ++it) {
    const int c = tid + it * kThreads;
    const int i = c / CPR, ch = c % CPR;
    float* dst = rows.row(i) + padi(ch * 8);
    const uint4 v = xv[it];
    dst[0] = bf16_lo(v.x); dst[1] = bf16_hi(v.x); dst[2] = bf16_lo(v.y); dst[3] = bf16_hi(v.y);
    dst[4] = bf16_lo(v.z); dst[5] = bf16_hi(v.z); dst[6] = bf16_lo(v.w); dst[7] = bf16_hi(v.w);
  }
  if (e_tab >= 0) wait_vm<0>();  // this wave's part of the table has landed
  __syncthreads();
  // The packed substrate words of the packed K-steps, for the GEMM. Lane l
  // needs W rows o = wave*WN + 32j + (l & 31), two words per K-step.
  uint2 pw[NP][C::FN];
#pragma unroll
  for (int ks = 0; ks < NP; ++ks)
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
  BflyCoef<D, false> cout;
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
  // Every wave is done with the ring: rows may be rewritten.
  __syncthreads();

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
  // The rows are complete.
  __syncthreads();

  cout.apply(rows, a.cs_out, sh_e, tab, e_tab);

  // g_r * row -> bf16, routed order.
#pragma unroll
  for (int it = 0; it < XPT; ++it) {
    const int c = tid + it * kThreads;
    const int i = c / CPR, ch = c % CPR;
    if (slot_of_row(i) < nr) {
      const int r = sh_r[i];
      const float g = a.gates[r];
      const float* s = rows.row(i) + padi(ch * 8);
      *reinterpret_cast<uint4*>(a.u + (size_t)r * D + ch * 8) =
          make_uint4(pack_bf16x2(g * s[0], g * s[1]), pack_bf16x2(g * s[2], g * s[3]),
                     pack_bf16x2(g * s[4], g * s[5]), pack_bf16x2(g * s[6], g * s[7]));
    }
  }
}

template <int D>
hipError_t launch_d(const FusedArgs& a, hipStream_t s, const KernelTiming& t) {
  return launch_kernel(fused_kernel<D>, dim3((a.M + kBM - 1) / kBM), dim3(kThreads), 0, s, t, a);
}

}  // namespace

bool fused_supported(bmoe_dtype dt, int d) {
  return dt == BMOE_BF16 && (d == 256 || d == 512);
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
    case 256: return launch_d<256>(a, s, t);
    case 512: return launch_d<512>(a, s, t);
  }
  return hipErrorInvalidValue;
}

}  // namespace bmoe
