// Internal launchers of the ButterflyMoE kernels (host side, not exported).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bmoe.h"

namespace bmoe {

// Optional start/stop events recorded by a kernel's own dispatch.
struct KernelTiming {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Launch `kernel`; with timing events set, the dispatch itself records them.
template <typename F, typename... Args>
hipError_t launch_kernel(F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t s,
                         const KernelTiming& t, Args... args) {
  hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, t.start, t.stop, 0u, args...);
  return hipGetLastError();
}

struct RouteTables {
  int32_t* offsets;  // [N+1]
  int32_t* perm;     // [M] sorted slot -> routed index
  int32_t* inv;      // [M] routed index -> sorted slot
  int32_t* slot_e;   // [M] sorted slot -> expert
};

// What the backward needs besides the forward's tables: expert-aligned row
// tiles (tiles[i] = (expert, first sorted row, end row, 0), at most
// tile_rows rows each; tile_base[e] = first tile of expert e, tile_base[N] =
// number of tiles; entries up to max_tiles past the last get expert -1) and
// the packed W_base^T, row-major (wpt) and, when wtt_block > 0, in the
// large-tile GEMM's tile-major order (wtt). tiles == NULL: none.
struct BwdSetup {
  int4* tiles = nullptr;
  int32_t* tile_base = nullptr;
  int max_tiles = 0, tile_rows = 0;
  uint32_t* wpt = nullptr;
  uint32_t* wtt = nullptr;
  int wtt_block = 0;
};

// Routing (histogram, scan, stable scatter), the per-call cos/sin tables of
// both rotation sides (none with theta NULL; the input side only with phi
// NULL), optionally a per-call tile-major copy of the packed substrate for
// the large-tile GEMM (wt) and optionally the backward's setup, in one
// launch.
hipError_t launch_prep(const int32_t* ids, int M, int N, const float* theta, const float* phi,
                       int d, RouteTables rt, float2* cs_in, float2* cs_out, int32_t* status,
                       const uint32_t* w_packed, uint32_t* wt, int wt_block,
                       hipStream_t s, const KernelTiming& t = {}, const BwdSetup& bs = {});

// Column block CB of the tile-major substrate copy `wt` the large-tile GEMM
// reads, or 0 when launch_gemm does not use that kernel. For output-column
// block ob = o / CB and K-step kt (64 columns), the 16 bytes of row o sit at
// uint4 index (ob * (d/64) + kt) * CB + o % CB of `wt`.
int gemm_tiled_w_block(bmoe_dtype dt, int M, int d);

// Routed fused forward with wave-resident rows (bf16, d = 256 or 512, M <=
// 8192 routed rows, N <= 512 experts): routing and cos/sin tables computed
// inside (each workgroup ranks its own 32 sorted rows from all M ids, stable,
// and writes their entries of rt: perm, inv, slot_e; workgroup 0 also
// offsets[0..N] and *status, BMOE_E_EXPERT for an id outside [0, N)), then
// both butterflies, the product and the gate for those rows, U in routed
// order.
bool fused_wave_routes(bmoe_dtype dt, int M, int d, int N);
// The same kernel after the preparation launch (any M and N): the rows'
// experts and routed indices from rt (perm, slot_e), nothing of rt written.
// Writes the g * U rows to u, and/or (z and h both non-NULL) the bf16 Z rows
// and H = alpha * Z W_base^T rows in sorted order, as the backward reads
// them; with u NULL the output side is skipped.
hipError_t launch_fused_wave_prepped(int M, int d, int k, const void* x, const float* gates,
                                     const float* theta, const float* phi, const uint32_t* wp,
                                     float alpha, void* u, void* z, void* h,
                                     const RouteTables& rt, hipStream_t s,
                                     const KernelTiming& t = {});
hipError_t launch_fused_wave(int M, int d, int k, int N, const void* x, const int32_t* ids,
                             const float* gates, const float* theta, const float* phi,
                             const uint32_t* wp, float alpha, void* u, const RouteTables& rt,
                             int32_t* status, hipStream_t s, const KernelTiming& t = {});

// H = alpha Z W^T (bf16) with the substrate in either storage format (the dl
// product kernel; d a multiple of 128; a base-3 buffer extends 8 bytes past
// the stream).
hipError_t launch_product(int M, int d, const uint16_t* z, const void* w, bmoe_wformat fmt,
                          float alpha, uint16_t* h, hipStream_t s, const KernelTiming& t = {});

// Whole forward for d in {2, 4, 8}: one thread per token, its k routed rows
// in ascending j (rotations with the prep kernel's cos/sin tables, the
// ternary product, the gate and the fp32 sum), written straight to y.
hipError_t launch_small(bmoe_dtype dt, int T, int d, int k, int N, const void* x,
                        const int32_t* ids, const float* gates, const float2* cs_in,
                        const float2* cs_out, const uint32_t* w_packed, float alpha, void* y,
                        hipStream_t s, const KernelTiming& t = {});

// Whether the fused d <= 512 path handles this shape (launch_fused_wave when
// fused_wave_routes also holds, else launch_fused_wave_prepped after prep).
bool fused_supported(bmoe_dtype dt, int d);

// Z[q] = B(theta_e)^T x[t]   (t = perm[q] / k, e = slot_e[q]).
// routed_out: row perm[q] of z instead of row q (routed order).
hipError_t launch_bfly_in(bmoe_dtype dt, int M, int d, int k, const void* x,
                          const RouteTables& rt, const float2* cs_in, void* z, hipStream_t s,
                          const KernelTiming& t = {}, bool routed_out = false);

// Register-resident butterflies for bf16 at d = 1024, 2048, 4096 (what
// launch_bfly_in / launch_bfly_out use there): in_side: dst = B(theta_e)^T of
// src row perm[q] / k, into row q (or perm[q] with routed_out); otherwise
// dst[perm[q]] = gates[perm[q]] * B(phi_e) src[q]. cs: that side's [N][L][d/2]
// (cos, sin).
bool bfly_wave_supported(bmoe_dtype dt, int d);
hipError_t launch_bfly_wave(bool in_side, int M, int d, int k, const RouteTables& rt,
                            const float2* cs, const void* src, void* dst, const float* gates,
                            bool routed_out, hipStream_t s, const KernelTiming& t = {});

// H = alpha * Z W_base^T over all M sorted rows (H bf16 on the bf16 path,
// fp32 on the fp32 path; Z likewise).
hipError_t launch_gemm(bmoe_dtype dt, int M, int d, const void* z, const uint32_t* w_packed,
                       const uint32_t* wt, float alpha, void* h, hipStream_t s,
                       const KernelTiming& t = {});

// U[r] = g_r * B(phi_e) H[q] for r = perm[q], written in routed order.
hipError_t launch_bfly_out(bmoe_dtype dt, int M, int d, const void* h, const float* gates,
                           const RouteTables& rt, const float2* cs_out, void* u,
                           hipStream_t s, const KernelTiming& t = {});

// y[t] = sum_j U[t*k + j], ascending j.
hipError_t launch_combine(bmoe_dtype dt, int T, int d, int k, const void* u, void* y,
                          hipStream_t s, const KernelTiming& t = {});

// Base-3 storage: five ternary digits per byte over the row-major entries
// (ceil(d*d/5) bytes), and its decoding into the 2-bit words launch_pack
// writes. Both reset *status first and set BMOE_E_TERNARY on a bad entry or a
// byte above 242.
hipError_t launch_pack_b3(const int8_t* w, int d, uint8_t* packed3, int32_t* status,
                          hipStream_t s);
hipError_t launch_unpack_b3(const uint8_t* packed3, int d, uint32_t* packed, int32_t* status,
                            hipStream_t s, const KernelTiming& t = {});
hipError_t launch_pack(const int8_t* w, int d, uint32_t* packed, int32_t* status,
                       hipStream_t s);

// ---- backward ----------------------------------------------------------------
// Upper bound on the expert-aligned row tiles of the backward kernels, and
// the rows per tile (BwdSetup::tile_rows).
int bwd_max_tiles(int M, int N, int d);
int bwd_tile_rows_for(int d);
// Register-resident variant of launch_bfly_bwd for bf16 d = 256 and 512 (same
// arguments and results; the tiles must have 16 rows).
bool bwd_wave_supported(bmoe_dtype dt, int d);
hipError_t launch_bfly_bwd_wave(bool in_side, int d, int k, const int4* tiles, int max_tiles,
                                const int32_t* perm, const float2* cs, const float* gates,
                                const void* src, const void* grad, void* dst, float* dgates,
                                float* partial, hipStream_t s, const KernelTiming& t);
// Butterfly backward over the tiles. Output side (in_side = false): src = H
// (sorted), grad = dy (token rows) -> dst = dH (sorted), dgates, partials of
// dphi. Input side: src = x (token rows), grad = dZ (sorted) -> dst = dX
// (routed order), partials of dtheta. partial: [max_tiles][L][d/2].
hipError_t launch_bfly_bwd(bool in_side, bmoe_dtype dt, int M, int d, int k, const int4* tiles,
                           int max_tiles, const int32_t* perm, const float2* cs,
                           const float* gates, const void* src, const void* grad, void* dst,
                           float* dgates, float* partial, hipStream_t s, const KernelTiming& t = {});
// dW [d][d] fp32 = alpha * dH^T Z for bf16 dH, Z [M][d] (128 <= d <= 4096):
// bf16 MFMA tiles over row ranges. With dw_kernel_splits(M, d) = S > 1 the
// ranges' partial products go to part [S][d][d] (launch_bwd_finish sums
// them), else straight to dw. 0 splits: d outside that range.
int dw_kernel_splits(int M, int d);
hipError_t launch_dw(int M, int d, const uint16_t* dh, const uint16_t* z, float alpha, float* dw,
                     float* part, hipStream_t s, const KernelTiming& t = {});
// The same for fp32 dH, Z (any d) or bf16 below d = 128, on fp32 MFMA; its
// row ranges: dw_f32_splits(M, d) (always >= 1), same slice convention.
int dw_f32_splits(int M, int d);
hipError_t launch_dw_f32(bmoe_dtype dt, int M, int d, const void* dh, const void* z,
                         float alpha, float* dw, float* part, hipStream_t s,
                         const KernelTiming& t = {});
// The backward's closing sums in one launch: dx[t] = sum_j dxr[t k + j]
// (ascending j, fp32; dtype dt); dphi / dtheta [N][L][d/2] = sums over each
// expert's tiles of the output / input side partials [tiles][L][d/2], in tile
// order; and, when slices > 1 and dw is set, dw [d][d] = sum over the slices
// of dw_part [slices][d][d], in order. status (may be NULL): set to BMOE_OK.
hipError_t launch_bwd_finish(bmoe_dtype dt, int T, int d, int k, const void* dxr, void* dx,
                             const float* part_out, const float* part_in,
                             const int32_t* tile_base, int N, float* dphi, float* dtheta,
                             const float* dw_part, int slices, float* dw, int32_t* status,
                             hipStream_t s, const KernelTiming& t = {});

// ---- outlier measurement ---------------------------------------------------------
// Per row of src [rows][d] (dtype dt): err = ||v - q|| / ||v|| with
// q = s * clip(rint(v / s), -m, m), s = max|v| / m (mode 0) or mean|v|
// (mode 1); crest (optional) = max|v| / rms(v). Zero rows give 0.
hipError_t launch_quant_error(bmoe_dtype dt, int rows, int d, const void* src, int m, int mode,
                              float* err, float* crest, hipStream_t s,
                              const KernelTiming& t = {});

// ---- router ------------------------------------------------------------------
// logits[t][e] = sum_c x[t][c] w[e][c] (fp32), x [T][d] and w [N][d] of dtype dt.
hipError_t launch_router_logits(bmoe_dtype dt, int T, int d, int N, const void* x,
                                const void* w, float* logits, hipStream_t s,
                                const KernelTiming& t = {});
// Top-k (k <= 64) of each logits row, ties to the lower id; softmax gates over
// the chosen logits.
hipError_t launch_topk(const float* logits, int T, int N, int k, int32_t* ids, float* gates,
                       hipStream_t s, const KernelTiming& t = {});

}  // namespace bmoe
