// Substrate gradient dW = alpha * dH^T Z (ButterflyMoE gist.science summary,
// §2.1 and §2.4: the shared ternary W_base is trained through its latent
// full-precision copy, whose gradient is the sum over every routed row of
// the outer product of the product's output gradient dH and its input Z).
//
// dH and Z are [M][d] bf16, rows in sorted order; dW is [d][d] fp32, row o
// (output), column c (input): dW[o][c] = alpha * sum_q dH[q][o] Z[q][c].
// The reduction index q is the row index of both operands, so both MFMA
// operands need 8 consecutive q per lane: each K-step's 32 rows of dH and Z
// go to LDS by DMA with their 16-byte chunks XOR-swizzled by row, and gfx950's
// transposing LDS read (ds_read_b64_tr_b16) gathers a lane's 4 q values of
// one column in one instruction.
//
// Tiles of 128 x 128 outputs (4 waves of 64 x 64) up to d = 1024 and of
// 256 x 256 (8 waves of 128 x 64) above, v_mfma_f32_32x32x16_bf16
// fragments, for d = 128 .. 4096. The rows are split into S equal ranges
// (multiples of 32) so the grid fills the CUs; split s writes its fp32
// partial product to part[s], and the backward's closing kernel adds the S
// slices in order, so the result does not depend on scheduling.
#include "common.h"
#include "kernels.h"

namespace bmoe {
namespace {

constexpr int kDwRows = 32;  // rows of dH and Z per K-step

// BM x BN outputs per workgroup, WM x WN waves of TM x TN each.
template <int BM_, int BN_, int WM_, int WN_>
struct DwCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int WAVES = WM * WN, THREADS = 64 * WAVES;
  static constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  static constexpr int A_BYTES = kDwRows * BM * 2, B_BYTES = kDwRows * BN * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES, NSTAGE = 4;
  static constexpr int A_LOADS = A_BYTES / 1024 / WAVES, B_LOADS = B_BYTES / 1024 / WAVES;
  static constexpr int V = A_LOADS + B_LOADS;  // DMA instructions per wave and K-step
  static_assert(A_LOADS >= 1 && B_LOADS >= 1 && 2 * V <= 63, "DMA counts");
  static_assert(NSTAGE * STAGE <= 160 * 1024, "LDS budget");
};

// 16-byte chunk position of chunk ch in LDS row r: rows r..r+3 of a
// transposing read land on four different 64-byte bank ranges.
__device__ __forceinline__ int dw_swz(int r, int ch) { return ch ^ ((r & 3) << 2); }

// Sixteen zero bytes: the DMA source of rows past the end of a range.
__device__ const uint4 kZero16 = {0u, 0u, 0u, 0u};

// Issue K-step rows [q, q + 32) of dH (columns o0 .. o0 + BM) and Z (columns
// c0 .. c0 + BN) into stage `stg`; rows at or past q_end read zeros.
template <class C>
__device__ __forceinline__ void dw_load(char* stg, const uint16_t* dH, const uint16_t* Z, int d,
                                        int q, int q_end, int o0, int c0, int lane, int wave) {
  constexpr int ACH = C::BM / 8, BCH = C::BN / 8;  // 16-byte chunks per LDS row
#pragma unroll
  for (int j = 0; j < C::A_LOADS; ++j) {
    const int blk = wave * C::A_LOADS + j;  // 1 KiB of the A region
    const int e = blk * 64 + lane;          // 16-byte slot
    const int r = e / ACH, slot = e % ACH;
    const int ch = dw_swz(r, slot);
    const void* g = q + r < q_end ? (const void*)(dH + (size_t)(q + r) * d + o0 + ch * 8)
                                  : (const void*)&kZero16;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                     (__attribute__((address_space(3))) void*)(stg + blk * 1024),
                                     16, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < C::B_LOADS; ++j) {
    const int blk = wave * C::B_LOADS + j;
    const int e = blk * 64 + lane;
    const int r = e / BCH, slot = e % BCH;
    const int ch = dw_swz(r, slot);
    const void* g = q + r < q_end ? (const void*)(Z + (size_t)(q + r) * d + c0 + ch * 8)
                                  : (const void*)&kZero16;
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)g,
        (__attribute__((address_space(3))) void*)(stg + C::A_BYTES + blk * 1024), 16, 0, 0);
  }
}

// LDS byte offset (within a region of WIDTH columns) of this lane's first
// transposing read for the 32 columns from col, K-slice 0. In each 16-lane
// group, lane 4j + q points at row kb + j, columns 4q .. 4q + 3 of the
// group's 16 (kb = 8 for lanes 32..63); the read hands lane i the group's
// column i of those 4 rows. Rows kb + 4 .. kb + 7 and K-slice kk (rows
// + 16 kk) keep the row's swizzle, so they sit 4 and 16 kk rows further on.
template <int WIDTH>
__device__ __forceinline__ uint32_t dw_frag_offset(int col, int lane) {
  const int gr = lane >> 4, L = lane & 15;
  const int c = col + 16 * (gr & 1) + 4 * (L & 3);
  const int r0 = 8 * (gr >> 1) + (L >> 2);
  return (uint32_t)(r0 * (WIDTH * 2) + dw_swz(r0, c >> 3) * 16 + (c & 7) * 2);
}

typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
typedef short dw_v4s __attribute__((ext_vector_type(4)));

// The FM + FN MFMA operands of K-slice KK of stage `stg`: lane l gets column
// l % 32 of each, rows 16 KK + 8 (l / 32) + 0..7, two transposing reads per
// operand. The stages are separate arrays, so the compiler can tell the stage
// read here from the stages the DMA still fills, and waits only for these
// reads, where their results are used (one slice's reads overlap the other
// slice's MFMAs).
template <class C, int KK>
__device__ __forceinline__ void dw_read(bf16x8 (&fa)[C::FM], bf16x8 (&fb)[C::FN],
                                        const char* stg, const uint32_t (&offA)[C::FM],
                                        const uint32_t (&offB)[C::FN]) {
  constexpr int LO_A = KK * 16 * C::BM * 2, HI_A = LO_A + 4 * C::BM * 2;
  constexpr int LO_B = KK * 16 * C::BN * 2, HI_B = LO_B + 4 * C::BN * 2;
  typedef __attribute__((address_space(3))) dw_v4s lds_v4s;
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const char* p = stg + offA[i];
    const dw_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + LO_A));
    const dw_v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + HI_A));
    const u64x2 x = {__builtin_bit_cast(uint64_t, lo), __builtin_bit_cast(uint64_t, hi)};
    fa[i] = __builtin_bit_cast(bf16x8, x);
  }
#pragma unroll
  for (int j = 0; j < C::FN; ++j) {
    const char* p = stg + C::A_BYTES + offB[j];
    const dw_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + LO_B));
    const dw_v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + HI_B));
    const u64x2 x = {__builtin_bit_cast(uint64_t, lo), __builtin_bit_cast(uint64_t, hi)};
    fb[j] = __builtin_bit_cast(bf16x8, x);
  }
}

template <int N>
__device__ __forceinline__ void dw_wait() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// K-step kt in ring stage S (compile-time). Every step issues its DMA
// unconditionally (steps past the range load zeros), so each wave has the
// same count of DMA instructions in flight per step and the wait counts
// below are exact.
template <class C, int S>
__device__ __forceinline__ void dw_step(f32x16 (&acc)[C::FM][C::FN], char* const (&ring)[4],
                                        const uint32_t (&offA)[C::FM],
                                        const uint32_t (&offB)[C::FN], const uint16_t* dH,
                                        const uint16_t* Z, int d, int kt, int q_begin,
                                        int q_end, int o0, int c0, int lane, int wave) {
  // This wave's loads of step kt have landed once only those of the two
  // later steps already issued are outstanding.
  __asm__ volatile("" ::: "memory");
  dw_wait<2 * C::V>();
  // Every wave's part of step kt has landed, and every wave is done with
  // step kt - 1, whose stage the next DMA overwrites.
  lds_barrier();
  dw_load<C>(ring[(S + 3) & 3], dH, Z, d, q_begin + (kt + 3) * kDwRows, q_end, o0, c0, lane, wave);
  __asm__ volatile("" ::: "memory");
  bf16x8 fa[C::FM], fb[C::FN], ga[C::FM], gb[C::FN];
  dw_read<C, 0>(fa, fb, ring[S], offA, offB);
  dw_read<C, 1>(ga, gb, ring[S], offA, offB);
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
#pragma unroll
  for (int i = 0; i < C::FM; ++i) fa[i] = ga[i];
#pragma unroll
  for (int j = 0; j < C::FN; ++j) fb[j] = gb[j];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
}

// One workgroup: one output tile and one row range of the S. Work item w
// = split * tiles + t; when the grid is a multiple of 8, XCD x (workgroups
// dealt round-robin) takes the contiguous items [x * n/8, (x+1) * n/8), so
// the workgroups sharing rows of dH and Z share that XCD's L2. Tiles run in
// panels of four tile rows. out: dW (S == 1) or part + split * d * d.
template <class C>
__global__ __launch_bounds__(C::THREADS) void dw_kernel(const uint16_t* dH, const uint16_t* Z,
                                                         int M, int d, int rows_per_split,
                                                         float alpha, float* out) {
  __shared__ __attribute__((aligned(1024))) char st0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char st2[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char st3[C::STAGE];
  char* const ring[4] = {st0, st1, st2, st3};

  const int tn = d / C::BN, tm = d / C::BM, tiles = tm * tn;
  const int n = gridDim.x;
  const int w = n % 8 == 0 ? (blockIdx.x % 8) * (n / 8) + blockIdx.x / 8 : blockIdx.x;
  const int split = w / tiles, t = w % tiles;
  const int P = tm < 4 ? tm : 4;  // tile rows per panel (tm is a power of two)
  const int o0 = (P * (t / (P * tn)) + t % P) * C::BM;
  const int c0 = ((t / P) % tn) * C::BN;
  const int q_begin = split * rows_per_split;
  const int q_end = min(M, q_begin + rows_per_split);
  // K-steps rounded up to a multiple of 4 (the extra ones hold zero rows).
  const int nsteps = q_end > q_begin ? (q_end - q_begin + 4 * kDwRows - 1) / (4 * kDwRows) * 4 : 0;
  float* dst = out + (size_t)split * d * d;

  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int wm = wave / C::WN, wn = wave % C::WN;
  uint32_t offA[C::FM], offB[C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i) offA[i] = dw_frag_offset<C::BM>(wm * C::TM + 32 * i, lane);
#pragma unroll
  for (int j = 0; j < C::FN; ++j) offB[j] = dw_frag_offset<C::BN>(wn * C::TN + 32 * j, lane);

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Steps 0..2 in flight before the loop.
  dw_load<C>(st0, dH, Z, d, q_begin, q_end, o0, c0, lane, wave);
  __asm__ volatile("" ::: "memory");
  dw_load<C>(st1, dH, Z, d, q_begin + kDwRows, q_end, o0, c0, lane, wave);
  __asm__ volatile("" ::: "memory");
  dw_load<C>(st2, dH, Z, d, q_begin + 2 * kDwRows, q_end, o0, c0, lane, wave);
  __asm__ volatile("" ::: "memory");
  for (int kt = 0; kt < nsteps; kt += 4) {
    dw_step<C, 0>(acc, ring, offA, offB, dH, Z, d, kt, q_begin, q_end, o0, c0,
                  lane, wave);
    dw_step<C, 1>(acc, ring, offA, offB, dH, Z, d, kt + 1, q_begin, q_end, o0, c0,
                  lane, wave);
    dw_step<C, 2>(acc, ring, offA, offB, dH, Z, d, kt + 2, q_begin, q_end, o0, c0,
                  lane, wave);
    dw_step<C, 3>(acc, ring, offA, offB, dH, Z, d, kt + 3, q_begin, q_end, o0, c0,
                  lane, wave);
  }
  dw_wait<0>();  // no DMA may land in LDS after the workgroup ends

  // 32x32 block layout: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4,
  // column l%32.
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int col = c0 + wn * C::TN + 32 * j + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = o0 + wm * C::TM + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        dst[(size_t)row * d + col] = alpha * acc[i][j][r];
      }
    }
}

template <class C>
hipError_t launch_dw_cfg(int M, int d, const uint16_t* dh, const uint16_t* z, float alpha,
                         float* dw, float* part, int S, hipStream_t s, const KernelTiming& t) {
  const int tiles = (d / C::BM) * (d / C::BN);
  const int rows = ((M + S - 1) / S + kDwRows - 1) / kDwRows * kDwRows;
  float* out = S == 1 ? dw : part;
  return launch_kernel(dw_kernel<C>, dim3(tiles * S), dim3(C::THREADS), 0, s, t, dh, z, M, d, rows,
                       alpha, out);
}

// ---------------------------------------------------------------------------
// The same gradient for fp32 activations (any d) and for bf16 below d = 128,
// on v_mfma_f32_32x32x2_f32. Its A operand (32 x 2) gives lane l element
// (l % 32, l / 32) and its B operand (2 x 32) element (l / 32, l % 32): with
// A[o][q] = dH[q][o] and B[q][c] = Z[q][c], lanes 0-31 read 32 consecutive
// columns of row q and lanes 32-63 the same columns of row q + 1, straight
// from memory (bf16 widened exactly to fp32). One wave per output tile of
// WT x WT (WT = 64, or 32 when d < 64; outputs past d are masked) and row
// range; accumulation in fp32 like the bf16 kernel.
constexpr int kF32Unroll = 8;  // K-steps (two rows each) loaded ahead

template <typename T>
__device__ __forceinline__ float ld_f32(const T* p) {
  if constexpr (sizeof(T) == 2) return bf16_lo(*reinterpret_cast<const uint16_t*>(p));
  else return *p;
}

template <typename T, int WT>
__global__ __launch_bounds__(kWave) void dw_f32_kernel(const T* dH, const T* Z, int M, int d,
                                                       int rows_per_split, float alpha,
                                                       float* out) {
  constexpr int F = WT / 32;  // 32 x 32 blocks per side
  const int tn = (d + WT - 1) / WT, tiles = tn * tn;
  const int split = blockIdx.x / tiles, t = blockIdx.x % tiles;
  const int o0 = (t / tn) * WT, c0 = (t % tn) * WT;
  const int q_begin = split * rows_per_split;
  const int q_end = min(M, q_begin + rows_per_split);
  float* dst = out + (size_t)split * d * d;
  const int lane = threadIdx.x, col = lane & 31, kq = lane >> 5;
  bool okA[F], okB[F];
#pragma unroll
  for (int i = 0; i < F; ++i) {
    okA[i] = o0 + 32 * i + col < d;
    okB[i] = c0 + 32 * i + col < d;
  }
  f32x16 acc[F][F];
#pragma unroll
  for (int i = 0; i < F; ++i)
#pragma unroll
    for (int j = 0; j < F; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  for (int q0 = q_begin; q0 < q_end; q0 += 2 * kF32Unroll) {
    float a[kF32Unroll][F], b[kF32Unroll][F];
#pragma unroll
    for (int u = 0; u < kF32Unroll; ++u) {
      const int q = q0 + 2 * u + kq;
      const bool row_ok = q < q_end;
#pragma unroll
      for (int i = 0; i < F; ++i) {
        a[u][i] = row_ok && okA[i] ? ld_f32(dH + (size_t)q * d + o0 + 32 * i + col) : 0.f;
        b[u][i] = row_ok && okB[i] ? ld_f32(Z + (size_t)q * d + c0 + 32 * i + col) : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kF32Unroll; ++u)
#pragma unroll
      for (int i = 0; i < F; ++i)
#pragma unroll
        for (int j = 0; j < F; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[u][i], b[u][j], acc[i][j], 0, 0, 0);
  }
  // 32x32 block layout: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4,
  // column l%32.
#pragma unroll
  for (int i = 0; i < F; ++i)
#pragma unroll
    for (int j = 0; j < F; ++j) {
      const int c = c0 + 32 * j + col;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int o = o0 + 32 * i + 8 * (r >> 2) + 4 * kq + (r & 3);
        if (o < d && c < d) dst[(size_t)o * d + c] = alpha * acc[i][j][r];
      }
    }
}

int f32_tile(int d) { return d >= 64 ? 64 : 32; }

}  // namespace

int dw_f32_splits(int M, int d) {
  const int wt = f32_tile(d), tn = (d + wt - 1) / wt, tiles = tn * tn;
  int S = (2048 + tiles - 1) / tiles;
  const int max_s = M / 256;  // at least 256 rows per split
  if (S > max_s) S = max_s;
  return S < 1 ? 1 : S;
}

hipError_t launch_dw_f32(bmoe_dtype dt, int M, int d, const void* dh, const void* z,
                         float alpha, float* dw, float* part, hipStream_t s,
                         const KernelTiming& t) {
  const int S = dw_f32_splits(M, d);
  const int wt = f32_tile(d), tn = (d + wt - 1) / wt;
  const int rows = ((M + S - 1) / S + 2 * kF32Unroll - 1) / (2 * kF32Unroll) * (2 * kF32Unroll);
  float* out = S == 1 ? dw : part;
  const dim3 grid(tn * tn * S), block(kWave);
  if (dt == BMOE_BF16) {
    const uint16_t* a = static_cast<const uint16_t*>(dh);
    const uint16_t* b = static_cast<const uint16_t*>(z);
    return wt == 64 ? launch_kernel(dw_f32_kernel<uint16_t, 64>, grid, block, 0, s, t, a, b, M, d,
                                    rows, alpha, out)
                    : launch_kernel(dw_f32_kernel<uint16_t, 32>, grid, block, 0, s, t, a, b, M, d,
                                    rows, alpha, out);
  }
  const float* a = static_cast<const float*>(dh);
  const float* b = static_cast<const float*>(z);
  return wt == 64 ? launch_kernel(dw_f32_kernel<float, 64>, grid, block, 0, s, t, a, b, M, d, rows,
                                  alpha, out)
                  : launch_kernel(dw_f32_kernel<float, 32>, grid, block, 0, s, t, a, b, M, d, rows,
                                  alpha, out);
}

// 128 x 128 tiles of four waves up to d = 1024; from d = 2048, 256 x 256 tiles
// of eight waves (128 x 64 each), which read half as many operand bytes per
// MFMA: the smaller tile needs L2 bandwidth at the per-CU limit to keep its
// MFMAs busy.
using DwSmall = DwCfg<128, 128, 2, 2>;
using DwLarge = DwCfg<256, 256, 2, 4>;

int dw_kernel_splits(int M, int d) {
  if (d < 128 || d > 4096) return 0;
  const int bm = d >= 2048 ? DwLarge::BM : DwSmall::BM;
  const int tiles = (d / bm) * (d / bm);
  int S = (256 + tiles - 1) / tiles;
  const int max_s = M / (16 * kDwRows);  // at least 16 K-steps per split
  if (S > max_s) S = max_s;
  return S < 1 ? 1 : S;
}

hipError_t launch_dw(int M, int d, const uint16_t* dh, const uint16_t* z, float alpha, float* dw,
                     float* part, hipStream_t s, const KernelTiming& t) {
  const int S = dw_kernel_splits(M, d);
  if (S == 0) return hipErrorInvalidValue;
  if (d >= 2048) return launch_dw_cfg<DwLarge>(M, d, dh, z, alpha, dw, part, S, s, t);
  return launch_dw_cfg<DwSmall>(M, d, dh, z, alpha, dw, part, S, s, t);
}

}  // namespace bmoe
