// Router in front of the expert layer: logits = x W_r^T, top-k experts per
// token, softmax gates over the k chosen logits. The pages describe the layer
// as a top-k mixture of experts (ButterflyMoE abstract; gist.science summary,
// §2.3) without a router formula; this is the usual top-k gate, with its
// readings stated in the C header.
//
//   logits[t][e] = sum_c x[t][c] * w_r[e][c]          (fp32 accumulation)
//   ids[t][0..k)  = experts by descending logit, ties to the lower id
//   gates[t][j]   = exp(l_j - l_0) / sum_i exp(l_i - l_0)
#include "common.h"
#include "kernels.h"

namespace bmoe {
namespace {

// ---- logits, bf16: MFMA --------------------------------------------------------
// A wave computes 32 tokens x 32G experts (G fragments of
// v_mfma_f32_32x32x16_bf16 sharing each A operand). Lane l feeds row / column
// l & 31 and, of each 64-wide k chunk, the contiguous half l >> 5: the order
// of the k terms inside a dot product is free as long as A and B agree.
// SPLIT = false: the 4 waves take 4 consecutive 32-token groups (their expert
// rows coincide, so those loads meet in L1). SPLIT = true: the 4 waves take
// the 4 quarters of k for one 32-token group, and their partial sums are added
// through LDS in wave order (more waves for small problems, and a quarter of
// the dependent load chain).
template <int G, bool SPLIT>
__global__ __launch_bounds__(256) void logits_mfma_kernel(const uint16_t* x, const uint16_t* w,
                                                          int T, int d, int N, float* logits) {
  __shared__ f32x16 part[SPLIT ? 3 * G * 64 : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = SPLIT ? blockIdx.x * 32 : blockIdx.x * 128 + wave * 32;
  const int e0 = blockIdx.y * 32 * G;
  const int row = lane & 31, half = lane >> 5;
  const int t = min(t0 + row, T - 1);
  const int kq = SPLIT ? d / 4 : d;                 // this wave's k range
  const int kbeg = SPLIT ? wave * kq : 0;
  const uint4* xa = reinterpret_cast<const uint4*>(x + (size_t)t * d + kbeg + half * 32);
  const uint4* wb[G];
  bool ok[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int e = e0 + 32 * g + row;
    ok[g] = e < N;
    wb[g] = reinterpret_cast<const uint4*>(w + (size_t)(ok[g] ? e : 0) * d + kbeg + half * 32);
  }
  const int steps = kq / 64;
  f32x16 acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = f32x16{};
  uint4 a[4], b[G][4], na[4], nb[G][4];
  const uint4 zero = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    a[u] = xa[u];
#pragma unroll
    for (int g = 0; g < G; ++g) b[g][u] = ok[g] ? wb[g][u] : zero;
  }
  for (int s = 0; s < steps; ++s) {
    const bool more = s + 1 < steps;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      na[u] = more ? xa[(s + 1) * 8 + u] : zero;
#pragma unroll
      for (int g = 0; g < G; ++g) nb[g][u] = (more && ok[g]) ? wb[g][(s + 1) * 8 + u] : zero;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int g = 0; g < G; ++g)
        acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[u]),
                                                         __builtin_bit_cast(bf16x8, b[g][u]),
                                                         acc[g], 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] = na[u];
#pragma unroll
      for (int g = 0; g < G; ++g) b[g][u] = nb[g][u];
    }
  }
  if (SPLIT) {
    if (wave > 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) part[((wave - 1) * G + g) * 64 + lane] = acc[g];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
      for (int g = 0; g < G; ++g) acc[g] += part[(q * G + g) * 64 + lane];
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (!ok[g]) continue;
    const int e = e0 + 32 * g + row;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tt = t0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (tt < T) logits[(size_t)tt * N + e] = acc[g][r];
    }
  }
}

// Large problems: BM x BN tiles staged through LDS. Coalesced 16-byte loads
// of 64-wide k chunks go to registers, then to an XOR-swizzled LDS tile (the
// 16-byte chunk c of row r sits at slot c ^ (r & 7)). AHEAD register sets
// keep that many chunks in flight; LDS is double-buffered, with one barrier
// per chunk. 4 waves in a 2 x 2 grid, each owning (BM/2) x (BN/2) as 32 x 32
// fragments. blockIdx.x walks the expert tiles, so the workgroups sharing a
// token tile run together and read it from L2.
template <int BM, int BN>
struct LdsTile {
  static constexpr int FM = BM / 64, FN = BN / 64;
  static constexpr int AL = BM * 8 / 256, BL = BN * 8 / 256;  // 16-byte loads per thread
};

template <int BM, int BN>
__device__ __forceinline__ void lt_load(const uint16_t* x, const uint16_t* w, int T, int d, int N,
                                        int m0, int n0, int s, int tid,
                                        uint4 (&ra)[LdsTile<BM, BN>::AL],
                                        uint4 (&rb)[LdsTile<BM, BN>::BL]) {
  using C = LdsTile<BM, BN>;
#pragma unroll
  for (int i = 0; i < C::AL; ++i) {
    const int u = tid + i * 256, r = u >> 3, c = u & 7;
    const int t = min(m0 + r, T - 1);
    ra[i] = *reinterpret_cast<const uint4*>(x + (size_t)t * d + s * 64 + c * 8);
  }
#pragma unroll
  for (int i = 0; i < C::BL; ++i) {
    const int u = tid + i * 256, r = u >> 3, c = u & 7;
    const int e = n0 + r;
    rb[i] = e < N ? *reinterpret_cast<const uint4*>(w + (size_t)e * d + s * 64 + c * 8)
                  : make_uint4(0, 0, 0, 0);
  }
}

template <int BM, int BN>
__device__ __forceinline__ void lt_store(uint4* As, uint4* Bs, int tid,
                                         const uint4 (&ra)[LdsTile<BM, BN>::AL],
                                         const uint4 (&rb)[LdsTile<BM, BN>::BL]) {
  using C = LdsTile<BM, BN>;
#pragma unroll
  for (int i = 0; i < C::AL; ++i) {
    const int u = tid + i * 256, r = u >> 3, c = u & 7;
    As[r * 8 + (c ^ (r & 7))] = ra[i];
  }
#pragma unroll
  for (int i = 0; i < C::BL; ++i) {
    const int u = tid + i * 256, r = u >> 3, c = u & 7;
    Bs[r * 8 + (c ^ (r & 7))] = rb[i];
  }
}

template <int BM, int BN>
__device__ __forceinline__ void lt_mfma(const uint4* As, const uint4* Bs, int lane, int wm, int wn,
                                        f32x16 (&acc)[LdsTile<BM, BN>::FM][LdsTile<BM, BN>::FN]) {
  using C = LdsTile<BM, BN>;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int c = 2 * kk + (lane >> 5);  // 16-byte chunk holding this lane's 8 k values
    bf16x8 af[C::FM], bfr[C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      const int r = wm * (BM / 2) + i * 32 + (lane & 31);
      af[i] = __builtin_bit_cast(bf16x8, As[r * 8 + (c ^ (r & 7))]);
    }
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int r = wn * (BN / 2) + j * 32 + (lane & 31);
      bfr[j] = __builtin_bit_cast(bf16x8, Bs[r * 8 + (c ^ (r & 7))]);
    }
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
  }
}

template <int BM, int BN, int AHEAD>
__global__ __launch_bounds__(256) void logits_lds_kernel(const uint16_t* x, const uint16_t* w,
                                                         int T, int d, int N, float* logits) {
  using C = LdsTile<BM, BN>;
  __shared__ uint4 As[2][BM * 8];
  __shared__ uint4 Bs[2][BN * 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int steps = d / 64;

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x16{};

  // register set j holds the chunks c with c % AHEAD == j
  uint4 ra[AHEAD][C::AL], rb[AHEAD][C::BL];
  lt_load<BM, BN>(x, w, T, d, N, m0, n0, 0, tid, ra[0], rb[0]);
  lt_store<BM, BN>(As[0], Bs[0], tid, ra[0], rb[0]);
#pragma unroll
  for (int j = 1; j < AHEAD; ++j)
    if (j < steps) lt_load<BM, BN>(x, w, T, d, N, m0, n0, j, tid, ra[j], rb[j]);
  __syncthreads();
  for (int s0 = 0; s0 < steps; s0 += AHEAD) {
#pragma unroll
    for (int j = 0; j < AHEAD; ++j) {
      const int s = s0 + j;
      if (s < steps) {
        // chunk s + AHEAD reuses the set of chunk s, already in LDS
        if (s + AHEAD < steps) lt_load<BM, BN>(x, w, T, d, N, m0, n0, s + AHEAD, tid, ra[j], rb[j]);
        lt_mfma<BM, BN>(As[s & 1], Bs[s & 1], lane, wm, wn, acc);
        const int jn = (j + 1) % AHEAD;  // a constant once the loop is unrolled
        if (s + 1 < steps) lt_store<BM, BN>(As[(s + 1) & 1], Bs[(s + 1) & 1], tid, ra[jn], rb[jn]);
        __syncthreads();
      }
    }
  }
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int e = n0 + wn * (BN / 2) + j * 32 + (lane & 31);
      if (e >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = m0 + wm * (BM / 2) + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (t < T) logits[(size_t)t * N + e] = acc[i][j][r];
      }
    }
}

// d < 64: one 16- or 32-wide chunk; lane half h takes k = h*KC/2 .. +KC/2.
template <int KC>
__global__ __launch_bounds__(64) void logits_mfma_narrow_kernel(const uint16_t* x,
                                                                const uint16_t* w, int T, int d,
                                                                int N, float* logits) {
  constexpr int NU = KC / 16;
  const int lane = threadIdx.x;
  const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
  const int row = lane & 31, half = lane >> 5;
  const int t = min(t0 + row, T - 1), e = e0 + row;
  const bool ok = e < N;
  const uint4* xa = reinterpret_cast<const uint4*>(x + (size_t)t * d + half * (KC / 2));
  const uint4* wb = reinterpret_cast<const uint4*>(w + (size_t)(ok ? e : 0) * d + half * (KC / 2));
  f32x16 acc = {};
#pragma unroll
  for (int u = 0; u < NU; ++u)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(bf16x8, xa[u]),
        __builtin_bit_cast(bf16x8, ok ? wb[u] : make_uint4(0, 0, 0, 0)), acc, 0, 0, 0);
  if (!ok) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int tt = t0 + 8 * (r >> 2) + 4 * half + (r & 3);
    if (tt < T) logits[(size_t)tt * N + e] = acc[r];
  }
}

// ---- logits, fp32: FMA ---------------------------------------------------------
// 64 x 64 outputs per workgroup, 4 x 4 per thread, k in chunks of 32 via LDS.
__global__ __launch_bounds__(256) void logits_f32_kernel(const float* x, const float* w, int T,
                                                         int d, int N, float* logits) {
  __shared__ float xs[32][65];
  __shared__ float ws_[32][65];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  const int kc = d < 32 ? d : 32;
  for (int k0 = 0; k0 < d; k0 += kc) {
    for (int u = tid; u < 64 * kc; u += 256) {
      const int r = u / kc, c = u % kc;
      const int tt = min(t0 + r, T - 1), ee = e0 + r;
      xs[c][r] = x[(size_t)tt * d + k0 + c];
      ws_[c][r] = ee < N ? w[(size_t)ee * d + k0 + c] : 0.f;
    }
    __syncthreads();
    for (int c = 0; c < kc; ++c) {
      float xv[4], wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xv[i] = xs[c][ty + 16 * i];
        wv[i] = ws_[c][tx + 16 * i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xv[i], wv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tt = t0 + ty + 16 * i, ee = e0 + tx + 16 * j;
      if (tt < T && ee < N) logits[(size_t)tt * N + ee] = acc[i][j];
    }
}

// ---- top-k + softmax -------------------------------------------------------------
// One wave per token. Lane l holds logits l, l + 64, ... (PER of them). Each
// round takes the wave's largest not-yet-chosen logit (ties to the lower id);
// pick j stays in lane j.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

template <int PER>
__global__ __launch_bounds__(256) void topk_kernel(const float* logits, int T, int N, int k,
                                                   int32_t* ids, float* gates) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave
  const float* lt = logits + (size_t)t * N;
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < N ? lt[e] : -INFINITY;
  }
  uint64_t taken = 0u;
  float mine_v = -INFINITY;
  int mine_i = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + 64 * i;
      if (e < N && !(taken >> i & 1u) && better(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1ull << (bi >> 6);
    if (lane == j) {
      mine_v = bv;
      mine_i = bi;
    }
  }
  const float top = __shfl(mine_v, 0, 64);
  const float ex = lane < k ? expf(mine_v - top) : 0.f;
  float sum = ex;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
  if (lane < k) {
    ids[(size_t)t * k + lane] = mine_i;
    gates[(size_t)t * k + lane] = ex / sum;
  }
}

template <int PER>
hipError_t launch_topk_per(const float* logits, int T, int N, int k, int32_t* ids, float* gates,
                           hipStream_t s, const KernelTiming& tm) {
  return launch_kernel(topk_kernel<PER>, dim3((T + 3) / 4), dim3(256), 0, s, tm, logits, T, N, k,
                       ids, gates);
}

}  // namespace

hipError_t launch_router_logits(bmoe_dtype dt, int T, int d, int N, const void* x,
                                const void* w, float* logits, hipStream_t s,
                                const KernelTiming& tm) {
  if (dt == BMOE_F32)
    return launch_kernel(logits_f32_kernel, dim3((T + 63) / 64, (N + 63) / 64), dim3(256), 0, s, tm,
                         static_cast<const float*>(x), static_cast<const float*>(w), T, d, N,
                         logits);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* wb = static_cast<const uint16_t*>(w);
  if (d < 64) {
    const dim3 g2((T + 31) / 32, (N + 31) / 32);
    if (d == 32)
      return launch_kernel(logits_mfma_narrow_kernel<32>, g2, dim3(64), 0, s, tm, xb, wb, T, d, N,
                           logits);
    return launch_kernel(logits_mfma_narrow_kernel<16>, g2, dim3(64), 0, s, tm, xb, wb, T, d, N,
                         logits);
  }
  // Many experts and many token tiles: the LDS-tiled kernel. Two chunks in
  // flight measured fastest at d = 512 and one at d = 4096 (where the extra
  // registers cost occupancy). With N <= 64 the register kernel below is
  // faster at every measured size.
  if (d >= 64 && N > 64 && (long long)((T + 127) / 128) * ((N + 127) / 128) >= 256) {
    const dim3 gl((N + 127) / 128, (T + 127) / 128);
    if (d >= 2048)
      return launch_kernel(logits_lds_kernel<128, 128, 1>, gl, dim3(256), 0, s, tm, xb, wb, T, d,
                           N, logits);
    return launch_kernel(logits_lds_kernel<128, 128, 2>, gl, dim3(256), 0, s, tm, xb, wb, T, d, N,
                         logits);
  }
  // experts per wave: 32G with G up to 4; four 32-token waves per workgroup
  // when that already gives at least 512 workgroups, else a 4-way k split.
  const int G = N > 64 ? 4 : N > 32 ? 2 : 1;
  const int ny = (N + 32 * G - 1) / (32 * G);
  const bool split = d >= 256 && (long long)((T + 127) / 128) * ny < 512;
  const dim3 gr(split ? (T + 31) / 32 : (T + 127) / 128, ny);
#define BMOE_LOGITS(GG, SS) \
  launch_kernel(logits_mfma_kernel<GG, SS>, gr, dim3(256), 0, s, tm, xb, wb, T, d, N, logits)
  if (G == 4) return split ? BMOE_LOGITS(4, true) : BMOE_LOGITS(4, false);
  if (G == 2) return split ? BMOE_LOGITS(2, true) : BMOE_LOGITS(2, false);
  return split ? BMOE_LOGITS(1, true) : BMOE_LOGITS(1, false);
#undef BMOE_LOGITS
}

hipError_t launch_topk(const float* logits, int T, int N, int k, int32_t* ids, float* gates,
                       hipStream_t s, const KernelTiming& tm) {
  if (N <= 64) return launch_topk_per<1>(logits, T, N, k, ids, gates, s, tm);
  if (N <= 128) return launch_topk_per<2>(logits, T, N, k, ids, gates, s, tm);
  if (N <= 256) return launch_topk_per<4>(logits, T, N, k, ids, gates, s, tm);
  if (N <= 512) return launch_topk_per<8>(logits, T, N, k, ids, gates, s, tm);
  if (N <= 1024) return launch_topk_per<16>(logits, T, N, k, ids, gates, s, tm);
  if (N <= 2048) return launch_topk_per<32>(logits, T, N, k, ids, gates, s, tm);
  return launch_topk_per<64>(logits, T, N, k, ids, gates, s, tm);
}

}  // namespace bmoe
