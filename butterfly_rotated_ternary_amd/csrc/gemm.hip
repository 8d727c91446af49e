// Shared-substrate product H = alpha * Z W_base^T over every routed row at
// once (ButterflyMoE gist.science summary, §2.3 step 2: one ternary W_base
// serves all experts, so the contraction is a single dense GEMM over all
// routed rows, whatever their expert).
//
// bf16 MFMA (v_mfma_f32_32x32x16_bf16) with fp32 accumulation. The packed
// 2-bit substrate is expanded to exact bf16 {-2,0,+2} (twice the weights, one
// shift and one mask per value pair), so every product is exact, and the
// accumulator is scaled by alpha / 2. For fp32 activations each Z value is
// split into three bf16 terms (hi + mid + lo represent it to within 2^-24
// relative) and the three partial products accumulate in fp32.
//
// Generic tiling (the kernels below the large-tile one): BM x BN output tile
// per workgroup, K in steps of 64, LDS double buffered (global loads for step
// k+1 are in flight while step k runs on the matrix cores; one barrier per
// step). Tiles are ordered so that the workgroups one XCD runs at a time share
// their rows of Z in that XCD's L2.
#include "common.h"
#include "kernels.h"

namespace bmoe {
namespace {

constexpr int BK = 64;
constexpr int LDK = BK + 8;  // bf16 per LDS row; the pad spreads rows over banks

__device__ __forceinline__ void split3(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = f32_to_bf16_bits(x);
  const float r1 = x - __uint_as_float(hi << 16);
  mid = f32_to_bf16_bits(r1);
  const float r2 = r1 - __uint_as_float(mid << 16);
  lo = f32_to_bf16_bits(r2);
}

template <int BM_, int BN_, int WM_, int WN_, bool F32A_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr bool F32A = F32A_;
  static constexpr int SPL = F32A ? 3 : 1;
  static constexpr int THREADS = 64 * WM * WN;
  static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  static constexpr int FM = TM / 32, FN = TN / 32;  // 32x32 MFMA blocks per wave
  // A tile: BM rows x BK. bf16 A: 16-byte chunks (8 values); fp32 A: 16-byte
  // chunks of 4 values.
  static constexpr int A_VALS = F32A ? 4 : 8;
  static constexpr int A_CHUNKS = BM * BK / A_VALS;
  static constexpr int A_PER_THREAD = A_CHUNKS / THREADS;
  // B tile: BN rows x BK = BN * BK/16 packed words.
  static constexpr int B_WORDS = BN * (BK / 16);
  static constexpr int B_PER_THREAD = (B_WORDS + THREADS - 1) / THREADS;
  static constexpr int A_LDS = SPL * BM * LDK;  // bf16 elements per buffer
  static constexpr int B_LDS = BN * LDK;
  static constexpr size_t LDS_BYTES = 2 * (A_LDS + B_LDS) * sizeof(uint16_t);
  static_assert(A_CHUNKS % THREADS == 0, "A tile must split evenly");
};

template <class C>
struct Stage {
  uint4 a[C::A_PER_THREAD];
  uint32_t b[C::B_PER_THREAD];
};

template <class C>
__device__ __forceinline__ void load_stage(Stage<C>& st, const void* zv, const uint32_t* wp, int M,
                                           int d, int m0, int n0, int k0) {
  const int tid = threadIdx.x;
  constexpr int CPR = BK / C::A_VALS;  // chunks per row
#pragma unroll
  for (int i = 0; i < C::A_PER_THREAD; ++i) {
    const int c = tid + i * C::THREADS;
    const int row = c / CPR, kc = (c % CPR) * C::A_VALS;
    const int gr = m0 + row;
    uint4 v = {0u, 0u, 0u, 0u};
    if (gr < M && k0 + kc < d) {
      if constexpr (C::F32A)
        v = *reinterpret_cast<const uint4*>(static_cast<const float*>(zv) + (size_t)gr * d + k0 + kc);
      else
        v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(zv) + (size_t)gr * d + k0 + kc);
    }
    st.a[i] = v;
  }
  const int G = d / 16;
#pragma unroll
  for (int i = 0; i < C::B_PER_THREAD; ++i) {
    const int wi = tid + i * C::THREADS;
    const int o = wi / (BK / 16), g = wi % (BK / 16);
    const int go = n0 + o, c0 = k0 + g * 16;
    uint32_t w = 0;
    if (wi < C::B_WORDS && go < d && c0 < d) w = wp[(size_t)go * G + c0 / 16];
    st.b[i] = w;
  }
}

template <class C>
__device__ __forceinline__ void store_stage(const Stage<C>& st, uint16_t* As, uint16_t* Bs) {
  const int tid = threadIdx.x;
  constexpr int CPR = BK / C::A_VALS;
#pragma unroll
  for (int i = 0; i < C::A_PER_THREAD; ++i) {
    const int c = tid + i * C::THREADS;
    const int row = c / CPR, kc = (c % CPR) * C::A_VALS;
    if constexpr (C::F32A) {
      uint32_t h[4], m[4], l[4];
      split3(__uint_as_float(st.a[i].x), h[0], m[0], l[0]);
      split3(__uint_as_float(st.a[i].y), h[1], m[1], l[1]);
      split3(__uint_as_float(st.a[i].z), h[2], m[2], l[2]);
      split3(__uint_as_float(st.a[i].w), h[3], m[3], l[3]);
      *reinterpret_cast<uint2*>(&As[(0 * C::BM + row) * LDK + kc]) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      *reinterpret_cast<uint2*>(&As[(1 * C::BM + row) * LDK + kc]) = make_uint2(m[0] | (m[1] << 16), m[2] | (m[3] << 16));
      *reinterpret_cast<uint2*>(&As[(2 * C::BM + row) * LDK + kc]) = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
    } else {
      *reinterpret_cast<uint4*>(&As[row * LDK + kc]) = st.a[i];
    }
  }
#pragma unroll
  for (int i = 0; i < C::B_PER_THREAD; ++i) {
    const int wi = tid + i * C::THREADS;
    if (wi < C::B_WORDS) {
      const int o = wi / (BK / 16), g = wi % (BK / 16);
      const uint32_t w = st.b[i];
      uint4 lo4, hi4;
      lo4.x = unpack_pair(w, 0); lo4.y = unpack_pair(w, 1);
      lo4.z = unpack_pair(w, 2); lo4.w = unpack_pair(w, 3);
      hi4.x = unpack_pair(w, 4); hi4.y = unpack_pair(w, 5);
      hi4.z = unpack_pair(w, 6); hi4.w = unpack_pair(w, 7);
      *reinterpret_cast<uint4*>(&Bs[o * LDK + g * 16]) = lo4;
      *reinterpret_cast<uint4*>(&Bs[o * LDK + g * 16 + 8]) = hi4;
    }
  }
}

template <class C, typename OutT>
__global__ __launch_bounds__(C::THREADS) void gemm_kernel(const void* zv, const uint32_t* wp,
                                                          OutT* H, int M, int d, float alpha,
                                                          int tiles_m, int tiles_n) {
  extern __shared__ uint4 lds_raw[];
  uint16_t* const lds = reinterpret_cast<uint16_t*>(lds_raw);
  constexpr int BUF = C::A_LDS + C::B_LDS;  // bf16 elements per buffer

  // XCD-aware order: workgroup b runs on XCD b % 8; give each XCD a
  // contiguous range of tiles (row-block major) so concurrently resident
  // tiles on one XCD share their rows of Z.
  const int ntiles = tiles_m * tiles_n;
  const int b = blockIdx.x;
  int tile = b;
  if (ntiles % 8 == 0) tile = (b % 8) * (ntiles / 8) + b / 8;
  const int m0 = (tile / tiles_n) * C::BM, n0 = (tile % tiles_n) * C::BN;

  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int wm = wave / C::WN, wn = wave % C::WN;

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  Stage<C> st;
  load_stage<C>(st, zv, wp, M, d, m0, n0, 0);
  store_stage<C>(st, lds, lds + C::A_LDS);
  __syncthreads();

  const int nk = (d + BK - 1) / BK;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_stage<C>(st, zv, wp, M, d, m0, n0, (kt + 1) * BK);
    const uint16_t* A = lds + cur * BUF;
    const uint16_t* B = lds + cur * BUF + C::A_LDS;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 bf[C::FN];
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        bf[j] = *reinterpret_cast<const bf16x8*>(
            &B[(wn * C::TN + j * 32 + (lane & 31)) * LDK + kk + 8 * (lane >> 5)]);
#pragma unroll
      for (int sp = 0; sp < C::SPL; ++sp) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
          const bf16x8 af = *reinterpret_cast<const bf16x8*>(
              &A[((C::SPL - 1 - sp) * C::BM + wm * C::TM + i * 32 + (lane & 31)) * LDK + kk +
                 8 * (lane >> 5)]);
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[j], acc[i][j], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < nk) store_stage<C>(st, lds + (cur ^ 1) * BUF, lds + (cur ^ 1) * BUF + C::A_LDS);
    __syncthreads();
  }

  // 32x32 block layout: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4,
  // column l%32.
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int col = n0 + wn * C::TN + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * C::TM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < M && col < d) {
          const float v = alpha * acc[i][j][r];
          if constexpr (sizeof(OutT) == 2)
            H[(size_t)row * d + col] = (OutT)f32_to_bf16_bits(v);
          else
            H[(size_t)row * d + col] = v;
        }
      }
    }
}

template <class C, typename OutT>
hipError_t launch_cfg(const void* z, const uint32_t* wp, OutT* h, int M, int d, float alpha,
                      hipStream_t s, const KernelTiming& t) {
  const int tm = (M + C::BM - 1) / C::BM, tn = (d + C::BN - 1) / C::BN;
  auto kern = gemm_kernel<C, OutT>;
  if (C::LDS_BYTES > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)C::LDS_BYTES);
    if (e != hipSuccess) return e;
  }
  return launch_kernel(kern, dim3(tm * tn), dim3(C::THREADS), (uint32_t)C::LDS_BYTES, s, t, z, wp,
                       h, M, d, alpha, tm, tn);
}


// ---------------------------------------------------------------------------
// Pipelined bf16 kernel for d % 128 == 0 and d % BN == 0.
//
// Z tiles go straight from global memory into LDS (global_load_lds_dwordx4:
// lane l of a wave lands in 16-byte slot l of a 1 KiB LDS block), so they
// occupy no registers. LDS rows are 128 bytes (64 bf16 of K) with their eight
// 16-byte chunks XOR-swizzled by (row >> 1) & 7, which keeps the 16-lane
// phases of the fragment reads on distinct banks. Packed substrate words come
// through registers two steps ahead and are expanded to bf16 in LDS in four
// slices between the MFMA groups of the current step. Z rows past M are
// clamped (computed, then dropped at the store), so nothing is predicated.
constexpr int kRowBytes = 128;  // one LDS row: BK = 64 bf16

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + 16 * (chunk ^ ((row >> 1) & 7));
}

template <int BM_, int BN_, int WM_, int WN_>
struct DCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int WAVES = WM * WN, THREADS = 64 * WAVES;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int A_BYTES = BM * kRowBytes, B_BYTES = BN * kRowBytes;
  static constexpr int A_LOADS = A_BYTES / 1024 / WAVES;  // 1 KiB wave loads per wave
  static constexpr int B_PER = BN * (BK / 16) / THREADS;  // packed words per thread
  static_assert(A_LOADS >= 1 && B_PER >= 1, "tile too small for the thread count");
};

// vmcnt(n) with expcnt / lgkmcnt left unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

template <class C>
__device__ __forceinline__ void d_load_a(char* abuf, const uint16_t* Z, int M, int d, int m0,
                                         int k0) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
  for (int j = 0; j < C::A_LOADS; ++j) {
    const int blk = wave * C::A_LOADS + j;    // 1 KiB block = 8 rows
    const int row = blk * 8 + lane / 8;
    const int chunk = (lane % 8) ^ ((row >> 1) & 7);  // slot lane%8 holds this chunk
    const int grow = min(m0 + row, M - 1);
    const uint16_t* g = Z + (size_t)grow * d + k0 + chunk * 8;
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)g,
        (__attribute__((address_space(3))) void*)(abuf + blk * 1024), 16, 0, 0);
  }
}

// Where the substrate of the dl kernel comes from: the packed 2-bit words
// (one register per word), or the base-3 stream (five ternary digits per
// byte, row-major entries), decoded into the same words as they are written
// to LDS. Both give exactly the same bf16 B tiles.
// REGS: registers per word in flight; VMEM: vector-memory instructions per
// word, which the step-end wait counts.
struct Packed2Src {
  static constexpr int REGS = 1, VMEM = 1;
  const uint32_t* wp;
  __device__ __forceinline__ void load(uint32_t* r, int o, int d, int k0, int g) const {
    r[0] = wp[(size_t)o * (d / 16) + k0 / 16 + g];
  }
  __device__ __forceinline__ uint32_t word(const uint32_t* r, int, int, int, int,
                                           const uint16_t*) const {
    return r[0];
  }
};

typedef uint64_t u64_dw_aligned __attribute__((aligned(4)));

struct Base3Src {
  static constexpr int REGS = 2, VMEM = 1;
  const uint8_t* w3;
  // The word's 16 entries e0 .. e0+15 (e0 = o d + k0 + 16 g) lie in bytes
  // e0/5 .. e0/5 + 3: the 8 bytes from the dword boundary (e0/5) & ~3 hold
  // them, read as one 8-byte load. For the stream's last words it reaches up
  // to 7 bytes past its end (the caller's buffer extends 8 bytes beyond it;
  // those bytes are never decoded), so every lane issues the same load.
  __device__ __forceinline__ void load(uint32_t* r, int o, int d, int k0, int g) const {
    const size_t e0 = (size_t)o * d + k0 + 16 * g, a = (e0 / 5) & ~(size_t)3;
    const uint64_t v = *reinterpret_cast<const u64_dw_aligned*>(w3 + a);
    r[0] = (uint32_t)v;
    r[1] = (uint32_t)(v >> 32);
  }
  // lut[b]: the five digits of byte b as 2-bit codes in entry order (digit 0,
  // 1, 2 -> code 3, 0, 1, i.e. -1, 0, +1).
  __device__ __forceinline__ uint32_t word(const uint32_t* r, int o, int d, int k0, int g,
                                           const uint16_t* lut) const {
    const size_t e0 = (size_t)o * d + k0 + 16 * g, b0 = e0 / 5;
    const int pos = (int)(e0 - 5 * b0), sh = 8 * (int)(b0 & 3);
    const uint64_t pair = ((uint64_t)r[1] << 32) | r[0];
    uint64_t seq = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      seq |= (uint64_t)(lut[(uint32_t)(pair >> (sh + 8 * i)) & 0xFFu] & 0x3FFu) << (10 * i);
    const uint32_t x = (uint32_t)(seq >> (2 * pos));  // entry v's code at bits 2v, 2v+1
    // even entries (columns 2j) to the low half, odd ones to the high half
    uint32_t ev = x & 0x33333333u, od = (x >> 2) & 0x33333333u;
    ev = (ev | (ev >> 2)) & 0x0F0F0F0Fu;
    od = (od | (od >> 2)) & 0x0F0F0F0Fu;
    ev = (ev | (ev >> 4)) & 0x00FF00FFu;
    od = (od | (od >> 4)) & 0x00FF00FFu;
    ev = (ev | (ev >> 8)) & 0x0000FFFFu;
    od = (od | (od >> 8)) & 0x0000FFFFu;
    return ev | (od << 16);
  }
};

template <class C, class Src>
__device__ __forceinline__ void d_load_b(uint32_t (&rb)[C::B_PER * Src::REGS], const Src& src,
                                         int d, int n0, int k0) {
#pragma unroll
  for (int i = 0; i < C::B_PER; ++i) {
    const int wi = threadIdx.x + i * C::THREADS;
    src.load(rb + i * Src::REGS, n0 + wi / (BK / 16), d, k0, wi % (BK / 16));
  }
}

// Expand slice `part` (of 4) of the words into bf16 LDS rows.
template <class C, class Src>
__device__ __forceinline__ void d_write_b(const uint32_t (&rb)[C::B_PER * Src::REGS],
                                          const Src& src, const uint16_t* lut, char* bbuf,
                                          int d, int n0, int k0, int part) {
#pragma unroll
  for (int i = 0; i < C::B_PER; ++i) {
    if ((i * 4) / C::B_PER != part) continue;
    const int wi = threadIdx.x + i * C::THREADS;
    const int o = wi / (BK / 16), g = wi % (BK / 16);
    const uint32_t w = src.word(rb + i * Src::REGS, n0 + o, d, k0, g, lut);
    *reinterpret_cast<uint4*>(bbuf + swz(o, 2 * g)) =
        make_uint4(unpack_pair(w, 0), unpack_pair(w, 1), unpack_pair(w, 2), unpack_pair(w, 3));
    *reinterpret_cast<uint4*>(bbuf + swz(o, 2 * g + 1)) =
        make_uint4(unpack_pair(w, 4), unpack_pair(w, 5), unpack_pair(w, 6), unpack_pair(w, 7));
  }
}

template <class C>
struct DFrags {
  bf16x8 a[C::FM];
  bf16x8 b[C::FN];
};

template <class C>
__device__ __forceinline__ void d_read(DFrags<C>& f, const char* abuf, const char* bbuf, int wm,
                                       int wn, int lane, int kk) {
  const int chunk = kk / 8 + (lane >> 5);
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
    f.a[i] = *reinterpret_cast<const bf16x8*>(abuf + swz(wm * C::TM + i * 32 + (lane & 31), chunk));
#pragma unroll
  for (int j = 0; j < C::FN; ++j)
    f.b[j] = *reinterpret_cast<const bf16x8*>(bbuf + swz(wn * C::TN + j * 32 + (lane & 31), chunk));
}

template <class C>
__device__ __forceinline__ void d_mfma(f32x16 (&acc)[C::FM][C::FN], const DFrags<C>& f) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// One K-step on (acur, bcur). LOAD: start step kt+1's Z tile into anxt and
// step kt+2's substrate words into rl. WRITE: expand rn (step kt+1's words)
// into bnxt. Ends with every Z load of this step landed and a barrier.
template <class C, class Src, bool LOAD, bool WRITE>
__device__ __forceinline__ void d_step(f32x16 (&acc)[C::FM][C::FN], const char* acur,
                                       const char* bcur, char* anxt, char* bnxt,
                                       uint32_t (&rn)[C::B_PER * Src::REGS],
                                       uint32_t (&rl)[C::B_PER * Src::REGS], const Src& src,
                                       const uint16_t* lut, const uint16_t* Z, int M, int d,
                                       int m0, int n0, int kt, int wm, int wn, int lane) {
  if constexpr (LOAD) {
    d_load_a<C>(anxt, Z, M, d, m0, (kt + 1) * BK);
    // The step-end wait counts the substrate loads as the newest vector
    // memory ops: keep the compiler from issuing them before the DMA.
    __asm__ volatile("" ::: "memory");
    d_load_b<C>(rl, src, d, n0, (kt + 2) * BK);
  }
  const int kw = (kt + 1) * BK;  // K offset of the words being written
  DFrags<C> f0, f1;
  d_read<C>(f0, acur, bcur, wm, wn, lane, 0);
  d_read<C>(f1, acur, bcur, wm, wn, lane, 16);
  d_mfma<C>(acc, f0);
  if constexpr (WRITE) d_write_b<C>(rn, src, lut, bnxt, d, n0, kw, 0);
  d_read<C>(f0, acur, bcur, wm, wn, lane, 32);
  d_mfma<C>(acc, f1);
  if constexpr (WRITE) d_write_b<C>(rn, src, lut, bnxt, d, n0, kw, 1);
  d_read<C>(f1, acur, bcur, wm, wn, lane, 48);
  d_mfma<C>(acc, f0);
  if constexpr (WRITE) d_write_b<C>(rn, src, lut, bnxt, d, n0, kw, 2);
  d_mfma<C>(acc, f1);
  if constexpr (WRITE) d_write_b<C>(rn, src, lut, bnxt, d, n0, kw, 3);
  if constexpr (LOAD) wait_vmcnt<C::B_PER * Src::VMEM>();  // Z tile of kt+1 has landed
  else wait_vmcnt<0>();
  lds_barrier();
}

template <class C, class Src>
__global__ __launch_bounds__(C::THREADS) void gemm_dl_kernel(const uint16_t* Z, Src src,
                                                             uint16_t* H, int M, int d,
                                                             float alpha, int tiles_m,
                                                             int tiles_n) {
  __shared__ __attribute__((aligned(1024))) char a0[C::A_BYTES];
  __shared__ __attribute__((aligned(1024))) char a1[C::A_BYTES];
  __shared__ __attribute__((aligned(1024))) char b0[C::B_BYTES];
  __shared__ __attribute__((aligned(1024))) char b1[C::B_BYTES];
  constexpr bool kB3 = Src::REGS == 2;
  __shared__ uint16_t lut[kB3 ? 256 : 1];
  if constexpr (kB3) {
    // byte value -> its five digits as 2-bit codes (values above 242 do not
    // occur in a stream written by the pack step)
    for (int v = threadIdx.x; v < 256; v += C::THREADS) {
      uint32_t codes = 0, rest = (uint32_t)v;
      for (int i = 0; i < 5; ++i) {
        const uint32_t t = rest % 3u;
        rest /= 3u;
        codes |= (t == 0 ? 3u : t == 2 ? 1u : 0u) << (2 * i);
      }
      lut[v] = (uint16_t)codes;
    }
    __syncthreads();
  }

  const int ntiles = tiles_m * tiles_n;
  const int bid = blockIdx.x;
  int tile = bid;
  if (ntiles % 8 == 0) tile = (bid % 8) * (ntiles / 8) + bid / 8;
  const int m0 = (tile / tiles_n) * C::BM, n0 = (tile % tiles_n) * C::BN;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int wm = wave / C::WN, wn = wave % C::WN;

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = d / BK;  // even
  uint32_t r0[C::B_PER * Src::REGS], r1[C::B_PER * Src::REGS];
  d_load_a<C>(a0, Z, M, d, m0, 0);
  d_load_b<C>(r0, src, d, n0, 0);
  d_load_b<C>(r1, src, d, n0, BK);
  wait_vmcnt<0>();
#pragma unroll
  for (int part = 0; part < 4; ++part) d_write_b<C>(r0, src, lut, b0, d, n0, 0, part);
  __syncthreads();

  int kt = 0;
  for (; kt + 2 < nk; kt += 2) {
    d_step<C, Src, true, true>(acc, a0, b0, a1, b1, r1, r0, src, lut, Z, M, d, m0, n0, kt, wm,
                               wn, lane);
    d_step<C, Src, true, true>(acc, a1, b1, a0, b0, r0, r1, src, lut, Z, M, d, m0, n0, kt + 1,
                               wm, wn, lane);
  }
  // kt = nk - 2: its Z tile for nk-1 still has to be fetched.
  d_load_a<C>(a1, Z, M, d, m0, (kt + 1) * BK);
  d_step<C, Src, false, true>(acc, a0, b0, a1, b1, r1, r0, src, lut, Z, M, d, m0, n0, kt, wm,
                              wn, lane);
  // (the barrier inside d_step<.., false, ..> needs the Z loads landed first)
  d_step<C, Src, false, false>(acc, a1, b1, a0, b0, r0, r1, src, lut, Z, M, d, m0, n0, kt + 1,
                               wm, wn, lane);

#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int col = n0 + wn * C::TN + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * C::TM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < M) H[(size_t)row * d + col] = (uint16_t)f32_to_bf16_bits(alpha * acc[i][j][r]);
      }
    }
}

template <class C, class Src>
hipError_t launch_dl(const uint16_t* z, const Src& src, uint16_t* h, int M, int d, float alpha,
                     hipStream_t s, const KernelTiming& t) {
  const int tm = (M + C::BM - 1) / C::BM, tn = d / C::BN;
  return launch_kernel(gemm_dl_kernel<C, Src>, dim3(tm * tn), dim3(C::THREADS), 0, s, t, z, src,
                       h, M, d, alpha, tm, tn);
}

// The dl kernel's tile choice: 64x128 tiles when 128x128 gives fewer than
// two tiles per CU (same per-element accumulation order, so the same bits).
template <class Src>
hipError_t launch_dl_auto(const uint16_t* z, const Src& src, uint16_t* h, int M, int d,
                          float alpha, hipStream_t s, const KernelTiming& t) {
  if ((long long)((M + 127) / 128) * (d / 128) < 512)
    return launch_dl<DCfg<64, 128, 2, 2>>(z, src, h, M, d, alpha, s, t);
  return launch_dl<DCfg<128, 128, 2, 2>>(z, src, h, M, d, alpha, s, t);
}

// ---------------------------------------------------------------------------
// Large-tile kernel (the large product, d a multiple of its BN): BM x BN
// output tiles, WM x WN waves, each owning a TM x TN block of 32x32
// fragments (FM x FN accumulator blocks). The configuration in use is below
// (LargeCfg).
//
// Both operands stream global->LDS with global_load_lds_dwordx4 through a
// 4-stage ring, three K-steps ahead: a stage holds the Z tile (BM rows x 64
// bf16, XOR-swizzled) and the packed substrate words of the step (BN output
// columns x 16 bytes). The substrate stays packed in LDS. In the MFMA B
// layout lane l holds output column l % 32 of a fragment and K half l / 32 of
// each 16-wide slice, so a lane reads the 16 bytes of its column once per
// step and expands the 8 bf16 of a slice in registers (unpack_pair: two VALU
// ops per bf16 pair) right before the MFMAs that use them; each expanded
// fragment feeds FM MFMAs.
//
// One barrier per step, before the last slice's MFMAs: all waves are done
// reading the step's stage (the DMA issued next step may overwrite it) and the
// next stage has landed, so the next step's first reads overlap this step's
// last MFMAs. sched_group_barrier fixes the order inside each slice: the next
// slice's LDS reads go out one per MFMA at the start, the expansion VALU ops
// are spread between MFMAs.
template <int BM_, int BN_, int WM_, int WN_>
struct RbCfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WM = WM_, WN = WN_, WAVES = WM * WN, THREADS = 64 * WAVES;
  static constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  static constexpr int NSTAGE = 4, AHEAD = NSTAGE - 1;
  static constexpr int A_BYTES = BM * kRowBytes;       // Z: BM rows x 64 bf16
  static constexpr int B_BYTES = BN * 16;              // packed words: BN columns x 16 B
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_LOADS = A_BYTES / 1024 / WAVES;  // 1 KiB DMA blocks per wave
  static constexpr int B_LOADS = B_BYTES / 1024 / WAVES;
  static constexpr int VM_PER_STEP = A_LOADS + B_LOADS;
  static constexpr int OUT_BYTES = 16 * TN * 2;        // per-wave epilogue staging: 16 rows
  // Global stores of one tile's epilogue per wave (16-byte row segments).
  static constexpr int STORES = FM * 2 * (16 * TN * 2 / 16 / 64);
  static_assert(WAVES * FM * FN * 32 * 32 == BM * BN, "the waves cover the tile");
  static_assert(FM * FN * 16 <= 256, "accumulators fit the AGPRs");
  static_assert(A_LOADS >= 1 && B_LOADS >= 1, "whole DMA blocks per wave");
  static_assert(NSTAGE * STAGE + WAVES * OUT_BYTES <= 160 * 1024, "LDS budget");
};

template <int N>
struct RbFrag {
  bf16x8 v[N];
};

// Issue step kt's DMA into `stg`: first this wave's blocks of packed words
// (each one contiguous KiB of the tile-major copy wt: 64 columns x 16 B),
// then its share of the Z tile.
// Addresses: a wave-uniform base (scalar registers) plus a 32-bit offset
// per lane, so the DMA uses the scalar-base form and a lane keeps one
// 32-bit register per load rather than a 64-bit address.
template <class C>
__device__ __forceinline__ void rb_load(char* stg, const uint16_t* Z, const uint32_t* wt, int M,
                                        int d, int m0, int n0, int kt, int lane, int wave) {
  const char* wbase = reinterpret_cast<const char*>(wt) +
                      ((size_t)(n0 / C::BN) * (d / BK) + kt) * C::BN * 16;
#pragma unroll
  for (int b = 0; b < C::B_LOADS; ++b) {
    const int blk = wave * C::B_LOADS + b;  // 64 columns
    const char* g = wbase + blk * 1024 + (uint32_t)(lane * 16);
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                     (__attribute__((address_space(3))) void*)(stg + C::A_BYTES +
                                                                              blk * 1024),
                                     16, 0, 0);
  }
  __asm__ volatile("" ::: "memory");
  const char* zbase = reinterpret_cast<const char*>(Z) + ((size_t)m0 * d + kt * BK) * 2;
  const int last = M - 1 - m0;  // rows past the end repeat the last row
#pragma unroll
  for (int j = 0; j < C::A_LOADS; ++j) {
    const int blk = wave * C::A_LOADS + j;  // 8 rows
    const int row = blk * 8 + lane / 8;
    const int chunk = (lane % 8) ^ ((row >> 1) & 7);
    const uint32_t off = (uint32_t)(min(row, last) * d * 2 + chunk * 16);
    const char* z = zbase + off;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)z,
                                     (__attribute__((address_space(3))) void*)(stg + blk * 1024),
                                     16, 0, 0);
  }
}

// A fragments of slice kk (0..3) for this wave's rows.
template <class C>
__device__ __forceinline__ void rb_read_a(RbFrag<C::FM>& a, const char* stg, int wm, int lane,
                                          int kk) {
  const int chunk = 2 * kk + (lane >> 5);
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
    a.v[i] = *reinterpret_cast<const bf16x8*>(stg + swz(wm * C::TM + i * 32 + (lane & 31), chunk));
}

// Packed words of this lane's columns for the whole step.
template <class C>
__device__ __forceinline__ void rb_read_w(uint4 (&w)[C::FN], const char* stg, int wn, int lane) {
#pragma unroll
  for (int j = 0; j < C::FN; ++j)
    w[j] = *reinterpret_cast<const uint4*>(stg + C::A_BYTES +
                                           16 * (wn * C::TN + j * 32 + (lane & 31)));
}

// B fragments of slice kk from the packed words (shifted by this lane's half).
template <class C>
__device__ __forceinline__ void rb_expand_b(RbFrag<C::FN>& b, const uint4 (&w)[C::FN], int hshift,
                                            int kk) {
#pragma unroll
  for (int j = 0; j < C::FN; ++j) {
    const uint32_t word = (kk == 0 ? w[j].x : kk == 1 ? w[j].y : kk == 2 ? w[j].z : w[j].w) >> hshift;
    u32x4 u;
    u[0] = unpack_pair(word, 0);
    u[1] = unpack_pair(word, 1);
    u[2] = unpack_pair(word, 2);
    u[3] = unpack_pair(word, 3);
    b.v[j] = __builtin_bit_cast(bf16x8, u);
  }
}

// INIT: start the accumulators from zero (the tile's first slice), so they
// are not live across tiles.
template <class C, bool INIT = false>
__device__ __forceinline__ void rb_mfma(f32x16 (&acc)[C::FM][C::FN], const RbFrag<C::FM>& a,
                                        const RbFrag<C::FN>& b) {
  const f32x16 zero = {};
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v[i], b.v[j], INIT ? zero : acc[i][j],
                                                          0, 0, 0);
}

// Order inside one slice section: the FM*FN MFMAs, with `nds` LDS reads and
// `nvm` DMA issues one per MFMA from the start, VALU ops spread between them.
// The closing sched_barrier keeps sections apart.
template <class C>
__device__ __forceinline__ void rb_interleave(int nds, int nvm) {
  constexpr int NMF = C::FM * C::FN;
#pragma unroll
  for (int i = 0; i < NMF; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA
    if (i < nds) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // DS read
    if (i < nvm) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);     // VMEM read
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);                  // VALU
  }
  __builtin_amdgcn_sched_barrier(0);
}

// What a step issues at its start.
enum RbLoad { kNoLoad = 0, kOwnStep = 1, kNextTile = 2 };

struct RbTile {
  int m0, n0;
};

// One K-step in ring slot S. On entry `a` holds slice 0 and `w` the packed
// words of this step. LOAD kOwnStep: issue step kt+3 of this tile into slot
// S+3; kNextTile: issue step kt+3-nk of the next tile `nt` there instead (the
// ring runs on across the tile boundary). WAIT: vector memory ops allowed in
// flight once step kt+1 has landed; `strict` (runtime, uniform) adds a wait
// down to WSTRICT first. NEXT: after the barrier, read slice 0 and the packed
// words of the following step.
template <class C, int S, int LOAD, int WAIT, bool NEXT, bool INIT = false, int WSTRICT = WAIT>
__device__ __forceinline__ void rb_step(f32x16 (&acc)[C::FM][C::FN], RbFrag<C::FM>& a,
                                        uint4 (&w)[C::FN], char* const (&ring)[C::NSTAGE],
                                        const uint16_t* Z, const uint32_t* wt, int M, int d,
                                        RbTile tl, RbTile nt, int kt, int wm, int wn, int lane,
                                        int wave, int hshift, bool strict = false) {
  const char* cur = ring[S];
  if constexpr (LOAD == kOwnStep) {
    rb_load<C>(ring[(S + C::AHEAD) % C::NSTAGE], Z, wt, M, d, tl.m0, tl.n0, kt + C::AHEAD, lane,
               wave);
  } else if constexpr (LOAD == kNextTile) {
    rb_load<C>(ring[(S + C::AHEAD) % C::NSTAGE], Z, wt, M, d, nt.m0, nt.n0,
               kt + C::AHEAD - d / BK, lane, wave);
  }
  constexpr int NVM = LOAD != kNoLoad ? C::VM_PER_STEP : 0;
  RbFrag<C::FN> b0, b1;
  RbFrag<C::FM> a1;
  rb_expand_b<C>(b0, w, hshift, 0);
  rb_read_a<C>(a1, cur, wm, lane, 1);
  rb_mfma<C, INIT>(acc, a, b0);
  rb_interleave<C>(C::FM, NVM);
  rb_expand_b<C>(b1, w, hshift, 1);
  rb_read_a<C>(a, cur, wm, lane, 2);
  rb_mfma<C>(acc, a1, b1);
  rb_interleave<C>(C::FM, 0);
  rb_expand_b<C>(b0, w, hshift, 2);
  rb_read_a<C>(a1, cur, wm, lane, 3);
  rb_mfma<C>(acc, a, b0);
  rb_interleave<C>(C::FM, 0);
  rb_expand_b<C>(b1, w, hshift, 3);
  // The last expansion happens before the barrier, so this step's packed
  // words are dead before the next step reloads their registers.
#pragma unroll
  for (int j = 0; j < C::FN; ++j) __asm__ volatile("" : "+v"(b1.v[j]));
  if constexpr (NEXT) {
    if constexpr (WSTRICT != WAIT) {
      if (strict) wait_vmcnt<WSTRICT>();
    }
    wait_vmcnt<WAIT>();
    lds_barrier();
    const char* nxt = ring[(S + 1) % C::NSTAGE];
    rb_read_w<C>(w, nxt, wn, lane);
    rb_read_a<C>(a, nxt, wm, lane, 0);
  }
  rb_mfma<C>(acc, a1, b1);
  rb_interleave<C>(NEXT ? C::FM + C::FN : 0, 0);
}

// Epilogue of one tile: alpha * acc -> bf16 H through this wave's staging
// LDS, 16 rows at a time (registers 8h .. 8h+7 of a 32x32 block are its rows
// 16h .. 16h+15), so the global stores are 16 bytes per lane over whole row
// segments of TN columns (8 stores per 32 rows).
template <class C>
__device__ __forceinline__ void rb_store(const f32x16 (&acc)[C::FM][C::FN], char* stg,
                                         uint16_t* H, int M, int d, RbTile tl, int wm, int wn,
                                         int lane, float alpha) {
  constexpr int PITCH = C::TN * 2, CHUNKS = C::TN / 8, RPQ = 64 / CHUNKS;
  static_assert((CHUNKS & (CHUNKS - 1)) == 0 && CHUNKS <= 64, "chunk swizzle");
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // 16 rows x TN bf16; 16-byte chunks XOR-swizzled by row.
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int r = 8 * h; r < 8 * h + 8; ++r) {
          const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3) - 16 * h;
          const int col = j * 32 + (lane & 31);
          const int off = row * PITCH + 16 * ((col >> 3) ^ (row & (CHUNKS - 1))) + 2 * (col & 7);
          *reinterpret_cast<uint16_t*>(stg + off) =
              (uint16_t)f32_to_bf16_bits(alpha * acc[i][j][r]);
        }
#pragma unroll
      for (int q = 0; q < 16 / RPQ; ++q) {
        const int row = q * RPQ + lane / CHUNKS, ch = lane % CHUNKS;
        const uint4 v =
            *reinterpret_cast<const uint4*>(stg + row * PITCH + 16 * (ch ^ (row & (CHUNKS - 1))));
        const int grow = tl.m0 + wm * C::TM + i * 32 + 16 * h + row;
        if (grow < M)
          *reinterpret_cast<uint4*>(H + (size_t)grow * d + tl.n0 + wn * C::TN + ch * 8) = v;
      }
    }
}

// Persistent: one workgroup per CU walks every nw-th tile of its XCD's
// contiguous tile range. The next tile's first three K-steps are issued in the
// current tile's last K-step (ring slots 0..2 are free once every wave has
// passed step nk-2's barrier), so they land while the epilogue stores run.
template <class C>
__global__ __launch_bounds__(C::THREADS) void gemm_rb_kernel(const uint16_t* Z,
                                                             const uint32_t* wt, uint16_t* H,
                                                             int M, int d, float alpha,
                                                             int tiles_m, int tiles_n) {
  // One array per stage: the compiler can then tell a stage being read from
  // the stages the DMA still writes, and does not wait for all loads.
  __shared__ __attribute__((aligned(1024))) char st0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char st2[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char st3[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char stage_out[C::WAVES * C::OUT_BYTES];
  static_assert(C::NSTAGE == 4, "four stage arrays");
  char* ring[4];
  ring[0] = st0;
  ring[1] = st1;
  ring[2] = st2;
  ring[3] = st3;

  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int hshift = 8 * (lane >> 5);  // K half of the slice -> its 4 code pairs

  // Workgroups are dealt round-robin to the 8 XCDs (gridDim.x is a multiple
  // of 8): XCD x owns tiles [t0, t1) and its nw workgroups interleave on them.
  const int ntiles = tiles_m * tiles_n;
  const int xcd = blockIdx.x % 8, nw = gridDim.x / 8;
  const int per = ntiles / 8, extra = ntiles % 8;
  const int t0 = xcd * per + min(xcd, extra), t1 = t0 + per + (xcd < extra ? 1 : 0);
  int tile = t0 + blockIdx.x / 8;
  if (tile >= t1) return;  // whole workgroup
  RbTile tl;
  tl.m0 = (tile / tiles_n) * C::BM;
  tl.n0 = (tile % tiles_n) * C::BN;

  const int nk = d / BK;  // multiple of 4, at least 8
#pragma unroll
  for (int s = 0; s < C::AHEAD; ++s) {
    rb_load<C>(ring[s], Z, wt, M, d, tl.m0, tl.n0, s, lane, wave);
    __asm__ volatile("" ::: "memory");
  }
  wait_vmcnt<(C::AHEAD - 1) * C::VM_PER_STEP>();
  lds_barrier();
  uint4 w[C::FN];
  RbFrag<C::FM> a;
  rb_read_w<C>(w, ring[0], wn, lane);
  rb_read_a<C>(a, ring[0], wm, lane, 0);

  // Steady state: steps kt+2, kt+3 in flight. A tile's first two steps also
  // have the previous tile's epilogue stores (8 per 32 rows) in flight; the
  // first tile has none, so it waits strictly there.
  constexpr int W3 = 2 * C::VM_PER_STEP;
  constexpr int WS = W3 + C::STORES;
  static_assert(WS <= 63, "vmcnt range");
  bool first = true;
  for (;;) {
    const int next = tile + nw;
    const bool has_next = next < t1;
    // Without a next tile the last steps re-issue this tile's first steps (a
    // few wasted loads, no branch around the accumulators); they are drained
    // before the workgroup exits.
    const int nx = has_next ? next : tile;
    RbTile nt;
    nt.m0 = (nx / tiles_n) * C::BM;
    nt.n0 = (nx % tiles_n) * C::BN;

    f32x16 acc[C::FM][C::FN];
    // The first four steps (the first slice sets the accumulators).
    rb_step<C, 0, kOwnStep, WS, true, true, W3>(acc, a, w, ring, Z, wt, M, d, tl, nt, 0, wm, wn,
                                                lane, wave, hshift, first);
    rb_step<C, 1, kOwnStep, WS, true, false, W3>(acc, a, w, ring, Z, wt, M, d, tl, nt, 1, wm, wn,
                                                 lane, wave, hshift, first);
    rb_step<C, 2, kOwnStep, W3, true>(acc, a, w, ring, Z, wt, M, d, tl, nt, 2, wm, wn, lane, wave,
                                      hshift);
    rb_step<C, 3, kOwnStep, W3, true>(acc, a, w, ring, Z, wt, M, d, tl, nt, 3, wm, wn, lane, wave,
                                      hshift);
    int kt = 4;
    for (; kt + 4 < nk; kt += 4) {
      rb_step<C, 0, kOwnStep, W3, true>(acc, a, w, ring, Z, wt, M, d, tl, nt, kt, wm, wn, lane,
                                        wave, hshift);
      rb_step<C, 1, kOwnStep, W3, true>(acc, a, w, ring, Z, wt, M, d, tl, nt, kt + 1, wm, wn,
                                        lane, wave, hshift);
      rb_step<C, 2, kOwnStep, W3, true>(acc, a, w, ring, Z, wt, M, d, tl, nt, kt + 2, wm, wn,
                                        lane, wave, hshift);
      rb_step<C, 3, kOwnStep, W3, true>(acc, a, w, ring, Z, wt, M, d, tl, nt, kt + 3, wm, wn,
                                        lane, wave, hshift);
    }
    // Last four steps: the ring runs on into the next tile's steps 0..2.
    rb_step<C, 0, kOwnStep, W3, true>(acc, a, w, ring, Z, wt, M, d, tl, nt, kt, wm, wn, lane,
                                      wave, hshift);
    rb_step<C, 1, kNextTile, W3, true>(acc, a, w, ring, Z, wt, M, d, tl, nt, kt + 1, wm, wn, lane,
                                       wave, hshift);
    rb_step<C, 2, kNextTile, W3, true>(acc, a, w, ring, Z, wt, M, d, tl, nt, kt + 2, wm, wn, lane,
                                       wave, hshift);
    rb_step<C, 3, kNextTile, W3, true>(acc, a, w, ring, Z, wt, M, d, tl, nt, kt + 3, wm, wn, lane,
                                       wave, hshift);

    rb_store<C>(acc, stage_out + wave * C::OUT_BYTES, H, M, d, tl, wm, wn, lane, alpha);
    if (!has_next) {
      wait_vmcnt<0>();  // no DMA may land in LDS after the workgroup ends
      break;
    }
    tile = next;
    tl = nt;
    first = false;
  }
}

template <class C>
hipError_t launch_rb(const uint16_t* z, const uint32_t* wt, uint16_t* h, int M, int d,
                     float alpha, hipStream_t s, const KernelTiming& t) {
  const int tm = (M + C::BM - 1) / C::BM, tn = d / C::BN;
  // One workgroup per CU (the LDS use allows no second one), a multiple of 8.
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        n >= 8)
      cus = n;
    else
      cus = 256;
  }
  int grid = tm * tn < cus ? tm * tn : cus;
  grid = (grid + 7) / 8 * 8;
  return launch_kernel(gemm_rb_kernel<C>, dim3(grid), dim3(C::THREADS), 0, s, t, z, wt, h, M, d,
                       alpha, tm, tn);
}

}  // namespace

// Eight waves, two per SIMD, each a 128 x 64 block (8 accumulator blocks):
// one wave's LDS reads and expansion overlap the other's MFMAs (measured
// against four waves of 128 x 128: 1556 against 1492-1529 TFLOP/s at d = 4096).
using LargeCfg = RbCfg<128, 512, 1, 8>;

int gemm_tiled_w_block(bmoe_dtype dt, int M, int d) {
  if (dt != BMOE_BF16 || d % LargeCfg::BN != 0) return 0;
  const long long tiles = (long long)((M + LargeCfg::BM - 1) / LargeCfg::BM) * (d / LargeCfg::BN);
  return tiles >= 512 ? LargeCfg::BN : 0;
}

hipError_t launch_gemm(bmoe_dtype dt, int M, int d, const void* z, const uint32_t* w_packed,
                       const uint32_t* wt, float alpha, void* h, hipStream_t s,
                       const KernelTiming& t) {
  alpha = substrate_scale(alpha);  // the expanded substrate holds +-2
  if (dt == BMOE_F32)
    return launch_cfg<Cfg<64, 64, 2, 2, true>, float>(z, w_packed, static_cast<float*>(h), M, d,
                                                      alpha, s, t);
  uint16_t* hb = static_cast<uint16_t*>(h);
  const uint16_t* zb = static_cast<const uint16_t*>(z);
  // Large problems: 128x512 tiles (8 waves of 128x64, tile-major substrate
  // copy). Smaller ones: 128x128 or 64x128 tiles so that the grid still
  // covers the CUs.
  if (gemm_tiled_w_block(dt, M, d)) {
    if (!wt) return hipErrorInvalidValue;
    return launch_rb<LargeCfg>(zb, wt, hb, M, d, alpha, s, t);
  }
  if (d >= 128) return launch_dl_auto(zb, Packed2Src{w_packed}, hb, M, d, alpha, s, t);
  return launch_cfg<Cfg<64, 64, 2, 2, false>, uint16_t>(z, w_packed, hb, M, d, alpha, s, t);
}

hipError_t launch_product(int M, int d, const uint16_t* z, const void* w, bmoe_wformat fmt,
                          float alpha, uint16_t* h, hipStream_t s, const KernelTiming& t) {
  alpha = substrate_scale(alpha);
  if (fmt == BMOE_W_BASE3)
    return launch_dl_auto(z, Base3Src{static_cast<const uint8_t*>(w)}, h, M, d, alpha, s, t);
  return launch_dl_auto(z, Packed2Src{static_cast<const uint32_t*>(w)}, h, M, d, alpha, s, t);
}

}  // namespace bmoe
