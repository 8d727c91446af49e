// Per-call preparation, one launch:
//  * (fused path) the packed substrate expanded to bf16 rows once per call,
//    or (large-tile product) copied into tile-major order;
//  * (backward) the expert-aligned row tiles and the packed W_base^T;
//  * routing: per-expert histogram, exclusive scan and a stable scatter of
//    routed rows r = t*k + j grouped by expert (ascending r inside a group);
//  * the cos/sin tables of both rotation sides, computed once per call so no
//    row ever evaluates a trigonometric function.
// Rows are grouped so that consecutive rows share one expert's rotation
// coefficients (ButterflyMoE gist.science summary, §2.3: every routed token is
// rotated by its own expert's butterflies around the shared substrate).
#include "common.h"
#include "kernels.h"

namespace bmoe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTrig = 4;  // angles per thread in the cos/sin role

struct PrepParams {
  const int32_t* ids;
  int M, N, nbits;
  int chunk, n_route_blocks;
  RouteTables rt;
  int32_t* status;
  const float* theta;
  const float* phi;
  float2* cs_in;
  float2* cs_out;
  long long n_ang;  // angles per side: N * L * d/2
  // Optional per-call copy of the packed substrate (both NULL: none): bf16
  // expansion [d][d], or tile-major packed words.
  const uint32_t* w_packed;
  uint32_t* wt;
  int wt_block;
  int d, n_trig_blocks, n_w_blocks, n_wt_blocks;
  BwdSetup bs;
};

// 2-bit code position of column v within a packed word (column 2j at bit
// 2j, column 2j+1 at bit 16 + 2j).
__device__ __forceinline__ int code_pos(int v) { return (v & 1) ? 16 + 2 * (v >> 1) : 2 * (v >> 1); }

// Backward tile list from the routing offsets (one 256-thread block).
__device__ void tiles_role(const int32_t* offsets, int N, int tr, int4* tiles, int32_t* tile_base,
                           int max_tiles) {
  __shared__ int scan[kThreads];
  __shared__ int carry;
  const int tid = threadIdx.x;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int e0 = 0; e0 < N; e0 += kThreads) {
    const int e = e0 + tid;
    const int cnt = e < N ? offsets[e + 1] - offsets[e] : 0;
    const int nt = (cnt + tr - 1) / tr;
    scan[tid] = nt;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
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
        tiles[base + i] = make_int4(e, q0 + i * tr, min(q0 + (i + 1) * tr, q0 + cnt), 0);
    }
    __syncthreads();
    if (tid == kThreads - 1) carry += scan[kThreads - 1];
    __syncthreads();
  }
  const int total = carry;
  if (tid == 0) tile_base[N] = total;
  for (int i = total + tid; i < max_tiles; i += kThreads) tiles[i] = make_int4(-1, 0, 0, 0);
}

__device__ __forceinline__ int clamp_expert(int e, int N, bool& bad) {
  if ((unsigned)e >= (unsigned)N) {
    bad = true;
    return e < 0 ? 0 : N - 1;
  }
  return e;
}

// Exclusive prefix sum of one int per thread over the 256-thread block.
__device__ int block_exclusive_scan(int v, int* scratch) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int incl = wave_incl_scan(v);
  if (lane == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += scratch[w];
  __syncthreads();
  return before + incl - v;
}

__global__ __launch_bounds__(kThreads) void prep_kernel(PrepParams p) {
  const int b_w = p.n_route_blocks + p.n_trig_blocks, b_wt = b_w + p.n_w_blocks;
  if ((int)blockIdx.x >= b_wt) {
    // ---- packed W_base^T: one thread per word (row c of W^T holds the codes
    // of column c of W, 16 per word; word g covers rows o = 16g .. 16g+15) --
    const int G = p.d / 16;
    const size_t n = (size_t)p.d * G;
    for (size_t u = (size_t)(blockIdx.x - b_wt) * kThreads + threadIdx.x; u < n;
         u += (size_t)p.n_wt_blocks * kThreads) {
      const int c = (int)(u / G), g = (int)(u % G);
      const int cw = c / 16, cpos = code_pos(c % 16);
      uint32_t out = 0u;
#pragma unroll
      for (int o16 = 0; o16 < 16; ++o16) {
        const uint32_t code = (p.w_packed[(size_t)(g * 16 + o16) * G + cw] >> cpos) & 3u;
        out |= code << code_pos(o16);
      }
      p.bs.wpt[(size_t)c * G + g] = out;
      if (p.bs.wtt_block > 0) {
        const int cb = p.bs.wtt_block, nk = p.d / 64;
        p.bs.wtt[(((size_t)(c / cb) * nk + g / 4) * cb + c % cb) * 4 + g % 4] = out;
      }
    }
    return;
  }
  if ((int)blockIdx.x >= b_w && p.wt) {
    // ---- packed substrate -> tile-major order ---------------------------
    // Destination-ordered: uint4 u = (ob * nk + kt) * CB + oo holds the 16
    // bytes of row ob * CB + oo for K-step kt.
    const int nk = p.d / 64;
    const size_t cb = (size_t)p.wt_block;
    const size_t n = (size_t)p.d * nk;
    const int b = blockIdx.x - b_w, nb = p.n_w_blocks;
    for (size_t u = (size_t)b * kThreads + threadIdx.x; u < n; u += (size_t)nb * kThreads) {
      const size_t oo = u % cb, rest = u / cb;
      const size_t kt = rest % nk, ob = rest / nk;
      const size_t o = ob * cb + oo;
      reinterpret_cast<uint4*>(p.wt)[u] =
          *reinterpret_cast<const uint4*>(p.w_packed + o * (p.d / 16) + kt * 4);
    }
    return;
  }
  if ((int)blockIdx.x >= p.n_route_blocks) {
    // ---- cos/sin tables -------------------------------------------------
    // A thread's angles are kTrig grid strides apart; all of their loads are
    // issued before the first sincosf, so a wave waits on memory once per
    // kTrig angles rather than once per angle.
    const long long total = p.phi ? 2 * p.n_ang : p.n_ang;  // no phi: input side only
    const long long stride = (long long)p.n_trig_blocks * kThreads;
    for (long long i0 = (long long)(blockIdx.x - p.n_route_blocks) * kThreads + threadIdx.x;
         i0 < total; i0 += kTrig * stride) {
      float a[kTrig];
#pragma unroll
      for (int u = 0; u < kTrig; ++u) {
        const long long i = i0 + u * stride;
        a[u] = i < total ? (i >= p.n_ang ? p.phi[i - p.n_ang] : p.theta[i]) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kTrig; ++u) {
        const long long i = i0 + u * stride;
        if (i < total) {
          float s, c;
          sincosf(a[u], &s, &c);
          if (i >= p.n_ang) p.cs_out[i - p.n_ang] = make_float2(c, s);
          else p.cs_in[i] = make_float2(c, s);
        }
      }
    }
    return;
  }

  // ---- routing ----------------------------------------------------------
  extern __shared__ int sh[];
  const int N = p.N, M = p.M;
  int* cnt = sh;                 // [N] counts from this chunk on, then totals, then offsets
  int* before = sh + N;          // [N] counts of rows before this chunk, then bases
  int* wcur = sh + 2 * N;        // [kWaves][N] per-wave counts, then cursors
  int* cid = sh + (2 + kWaves) * N;  // [chunk] this chunk's expert ids (clamped)
  __shared__ int scratch[kWaves];

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int r0 = blockIdx.x * p.chunk;
  const int r1 = min(M, r0 + p.chunk);

  for (int i = tid; i < (2 + kWaves) * N; i += kThreads) sh[i] = 0;
  __syncthreads();

  // Histogram of every id (all blocks need the global offsets), 4 ids per
  // load, a whole batch of loads in flight per thread (one round trip for
  // M <= 4 * kBatch * kThreads): rows before this block's chunk count into
  // `before`, the others into `cnt` (one LDS atomic per id). The ids of this
  // block's chunk go to LDS from the same loads.
  bool bad = false;
  const int M4 = M / 4;
  const int4* ids4 = reinterpret_cast<const int4*>(p.ids);
  constexpr int kBatch = 16;
  for (int i0 = 0; i0 < M4; i0 += kBatch * kThreads) {
    int4 v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = i0 + tid + j * kThreads;
      v[j] = i < M4 ? ids4[i] : make_int4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = i0 + tid + j * kThreads;
      if (i >= M4) break;
      const int r = 4 * i;
      const int e0 = clamp_expert(v[j].x, N, bad), e1 = clamp_expert(v[j].y, N, bad);
      const int e2 = clamp_expert(v[j].z, N, bad), e3 = clamp_expert(v[j].w, N, bad);
      int* h = r < r0 ? before : cnt;  // chunks start at multiples of 4
      atomicAdd(&h[e0], 1); atomicAdd(&h[e1], 1);
      atomicAdd(&h[e2], 1); atomicAdd(&h[e3], 1);
      if (r >= r0 && r < r1) {  // r1 - r0 is a multiple of 4 except at M
        cid[r - r0] = e0; cid[r - r0 + 1] = e1; cid[r - r0 + 2] = e2; cid[r - r0 + 3] = e3;
      }
    }
  }
  for (int r = 4 * M4 + tid; r < M; r += kThreads) {  // the last M % 4 ids
    const int e = clamp_expert(p.ids[r], N, bad);
    atomicAdd(r < r0 ? &before[e] : &cnt[e], 1);
    if (r >= r0 && r < r1) cid[r - r0] = e;
  }
  __syncthreads();
  for (int e = tid; e < N; e += kThreads) cnt[e] += before[e];  // totals
  __syncthreads();

  // Exclusive scan of the counts: each thread owns a contiguous segment.
  const int per = (N + kThreads - 1) / kThreads;
  const int lo = min(N, tid * per), hi = min(N, lo + per);
  int seg = 0;
  for (int e = lo; e < hi; ++e) seg += cnt[e];
  int run = block_exclusive_scan(seg, scratch);
  for (int e = lo; e < hi; ++e) {
    const int c = cnt[e];
    cnt[e] = run;
    run += c;
  }
  const bool any_bad = __syncthreads_or(bad);
  if (blockIdx.x == 0) {
    for (int e = tid; e < N; e += kThreads) p.rt.offsets[e] = cnt[e];
    if (tid == 0) {
      p.rt.offsets[N] = M;
      *p.status = any_bad ? BMOE_E_EXPERT : BMOE_OK;
    }
  }
  for (int e = tid; e < N; e += kThreads) before[e] += cnt[e];

  // Each wave owns a contiguous quarter of the chunk.
  const int len = r1 - r0;
  const int quarter = (len + kWaves - 1) / kWaves;
  const int wb = min(len, wave * quarter), we = min(len, wb + quarter);
  int* mycur = wcur + wave * N;
  for (int r = wb + lane; r < we; r += kWave) atomicAdd(&mycur[cid[r]], 1);
  __syncthreads();
  for (int e = tid; e < N; e += kThreads) {
    int c0 = before[e];
    for (int w = 0; w < kWaves; ++w) {
      const int c = wcur[w * N + e];
      wcur[w * N + e] = c0;
      c0 += c;
    }
  }
  __syncthreads();

  // Stable ranks inside each 64-row step: lanes holding the same expert are
  // found with one ballot per key bit; their order is the lane order.
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int base = wb; base < we; base += kWave) {
    const int rl = base + lane;
    const bool valid = rl < we;
    const int e = valid ? cid[rl] : 0;
    uint64_t mask = __ballot(valid);
    for (int b = 0; b < p.nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(bit);
      mask &= bit ? bal : ~bal;
    }
    const int rank = __popcll(mask & lt);
    const int grp = __popcll(mask);
    int cur = 0;
    if (valid) cur = mycur[e];
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      const int q = cur + rank;
      const int r = r0 + rl;
      p.rt.perm[q] = r;
      p.rt.inv[r] = q;
      p.rt.slot_e[q] = e;
      if (rank == grp - 1) mycur[e] = cur + grp;
    }
    __builtin_amdgcn_wave_barrier();
  }

  if (blockIdx.x == 0 && p.bs.tiles) {
    __syncthreads();  // this block wrote the offsets above
    tiles_role(p.rt.offsets, N, p.bs.tile_rows, p.bs.tiles, p.bs.tile_base, p.bs.max_tiles);
  }
}

}  // namespace

hipError_t launch_prep(const int32_t* ids, int M, int N, const float* theta, const float* phi,
                       int d, RouteTables rt, float2* cs_in, float2* cs_out, int32_t* status,
                       const uint32_t* w_packed, uint32_t* wt, int wt_block,
                       hipStream_t s, const KernelTiming& t, const BwdSetup& bs) {
  int L = 0;
  while ((1 << L) < d) ++L;
  PrepParams p;
  p.ids = ids;
  p.M = M;
  p.N = N;
  p.nbits = 0;
  while ((1 << p.nbits) < N) ++p.nbits;
  p.chunk = M <= 8192 ? 1024 : 2048;
  p.n_route_blocks = (M + p.chunk - 1) / p.chunk;
  if (p.n_route_blocks < 1) p.n_route_blocks = 1;
  p.rt = rt;
  p.status = status;
  p.theta = theta;
  p.phi = phi;
  p.cs_in = cs_in;
  p.cs_out = cs_out;
  p.n_ang = (long long)N * L * (d / 2);
  long long trig_blocks = ((phi ? 2 : 1) * p.n_ang + kThreads * kTrig - 1) / (kThreads * kTrig);
  if (trig_blocks > 65536) trig_blocks = 65536;
  if (!theta) trig_blocks = 0;  // no tables wanted
  p.n_trig_blocks = (int)trig_blocks;
  p.w_packed = w_packed;
  p.wt = (wt_block <= 0 || d % wt_block != 0) ? nullptr : wt;
  p.wt_block = wt_block;
  p.d = d;
  int w_blocks = 0;
  if (p.wt) {
    const long long quads = (long long)d * (d / 64);
    w_blocks = (int)((quads + kThreads * 4 - 1) / (kThreads * 4));
  }
  p.n_w_blocks = w_blocks;
  p.bs = bs;
  p.n_wt_blocks = 0;
  if (bs.tiles) {
    const long long words = (long long)d * (d / 16);
    p.n_wt_blocks = (int)((words + kThreads * 4 - 1) / (kThreads * 4));
  }
  const size_t shmem = sizeof(int) * ((size_t)(2 + kWaves) * N + p.chunk);
  if (shmem > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(prep_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  return launch_kernel(prep_kernel,
                       dim3(p.n_route_blocks + p.n_trig_blocks + w_blocks + p.n_wt_blocks),
                       dim3(kThreads), (uint32_t)shmem, s, t, p);
}

}  // namespace bmoe
