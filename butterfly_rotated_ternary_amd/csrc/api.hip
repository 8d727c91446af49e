// C ABI of libbmoe.so: host-side validation, workspace carving and the
// launch sequence of the forward. Every step of the forward runs in the HIP
// kernels of this library; nothing here touches element data.
#include <climits>
#include <mutex>


#include "common.h"
#include "kernels.h"

namespace bmoe {
namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// The forward and the pack step take d = 2 .. 8192; everything else (the
// backward, the router, the input-side rotation, the quantisation error and
// the base-3 storage) needs whole 16-column words per row: d >= 16.
bool valid_d(int d) { return d >= 2 && d <= 8192 && (d & (d - 1)) == 0; }
bool valid_d16(int d) { return d >= 16 && valid_d(d); }
// d in {2, 4, 8}: the one-thread-per-token forward.
bool small_d(int d) { return d < 16; }

int log2i(int d) {
  int L = 0;
  while ((1 << L) < d) ++L;
  return L;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct FwdLayout {
  size_t status, offsets, perm, inv, slot_e, cs_in, cs_out, z, h, u, wt, tiles, tile_base,
      wpt, wtt, total;
  int max_tiles;
};

bool shape_ok(bmoe_dtype dt, int T, int d, int N, int k) {
  if (dt != BMOE_F32 && dt != BMOE_BF16) return false;
  if (!valid_d(d) || N < 1 || N > kMaxExperts || k < 1 || k > N || T < 0) return false;
  if ((long long)T * k > INT_MAX) return false;
  return true;
}

// keep: the unfused path, with Z and H left in the workspace (with the
// routing and cos/sin tables, and the backward's row tiles and packed
// W_base^T) for a later bmoe_backward_kept.
FwdLayout fwd_layout(bmoe_dtype dt, int T, int d, int N, int k, bool keep = false) {
  FwdLayout l{};
  const size_t M = (size_t)T * k;
  const size_t L = (size_t)log2i(d);
  const size_t zel = dt == BMOE_BF16 ? 2 : 4;
  size_t off = 0;
  l.status = off;  off = align_up(off + sizeof(int32_t));
  l.offsets = off; off = align_up(off + sizeof(int32_t) * (N + 1));
  l.perm = off;    off = align_up(off + sizeof(int32_t) * M);
  l.inv = off;     off = align_up(off + sizeof(int32_t) * M);
  l.slot_e = off;  off = align_up(off + sizeof(int32_t) * M);
  const bool fused = !keep && fused_supported(dt, d);
  // The fused kernel evaluates its own tiles' coefficient tables from the
  // angles and reads the packed substrate words.
  l.cs_in = off;   if (!fused) off = align_up(off + sizeof(float2) * N * L * (d / 2));
  l.cs_out = off;  if (!fused) off = align_up(off + sizeof(float2) * N * L * (d / 2));
  // The fused path keeps Z and H on chip; only U lives in the workspace.
  const bool small = small_d(d);
  l.z = off;       if (!fused && !small) off = align_up(off + zel * M * d);
  l.h = off;       if (!fused && !small) off = align_up(off + zel * M * d);
  l.u = off;       if (!small) off = align_up(off + zel * M * d);
  // Tile-major copy of the packed substrate for the large-tile product.
  l.wt = off;
  const bool wt_copy = gemm_tiled_w_block(dt, (int)M, d) != 0;
  if (wt_copy) off = align_up(off + sizeof(uint32_t) * (size_t)d * (d / 16));
  l.max_tiles = keep ? bwd_max_tiles((int)M, N, d) : 0;
  l.tiles = off;     if (keep) off = align_up(off + sizeof(int4) * l.max_tiles);
  l.tile_base = off; if (keep) off = align_up(off + sizeof(int32_t) * (N + 1));
  l.wpt = off;       if (keep) off = align_up(off + sizeof(uint32_t) * (size_t)d * (d / 16));
  l.wtt = off;       if (keep && wt_copy) off = align_up(off + sizeof(uint32_t) * (size_t)d * (d / 16));
  l.total = off;
  return l;
}

// Workspace of bmoe_rotate_in: the routing tables and the input-side cos/sin.
struct RotLayout {
  size_t status, offsets, perm, inv, slot_e, cs_in, total;
};

RotLayout rot_layout(int T, int d, int N, int k) {
  RotLayout l{};
  const size_t M = (size_t)T * k;
  size_t off = 0;
  l.status = off;  off = align_up(off + sizeof(int32_t));
  l.offsets = off; off = align_up(off + sizeof(int32_t) * (N + 1));
  l.perm = off;    off = align_up(off + sizeof(int32_t) * M);
  l.inv = off;     off = align_up(off + sizeof(int32_t) * M);
  l.slot_e = off;  off = align_up(off + sizeof(int32_t) * M);
  l.cs_in = off;   off = align_up(off + sizeof(float2) * N * log2i(d) * (d / 2));
  l.total = off;
  return l;
}

struct BwdLayout {
  size_t status, offsets, perm, inv, slot_e, cs_in, cs_out, z, h, dh, dx, wt, wpt, wtt, tiles,
      tile_base, part_in, part_out, dw_part, total;
  int max_tiles, wt_block;
};

// The substrate gradient's kernel: bf16 with 128 <= d <= 4096 on bf16 MFMA
// (launch_dw), otherwise (fp32, small d) on fp32 MFMA (launch_dw_f32). Both
// may split the reduction over the M routed rows into row ranges whose fp32
// partial products the backward's closing kernel sums in a fixed order.
bool dw_own_kernel(bmoe_dtype dt, int d) { return dt == BMOE_BF16 && d >= 128 && d <= 4096; }
int dw_slots(bmoe_dtype dt, int M, int d) {
  const int S = dw_own_kernel(dt, d) ? dw_kernel_splits(M, d) : dw_f32_splits(M, d);
  return S > 1 ? S : 0;
}

BwdLayout bwd_layout(bmoe_dtype dt, int T, int d, int N, int k) {
  BwdLayout l{};
  const size_t M = (size_t)T * k;
  const size_t L = (size_t)log2i(d);
  const size_t zel = dt == BMOE_BF16 ? 2 : 4;
  const size_t wwords = (size_t)d * (d / 16);
  l.wt_block = gemm_tiled_w_block(dt, (int)M, d);
  l.max_tiles = bwd_max_tiles((int)M, N, d);
  size_t off = 0;
  l.status = off;    off = align_up(off + sizeof(int32_t));
  l.offsets = off;   off = align_up(off + sizeof(int32_t) * (N + 1));
  l.perm = off;      off = align_up(off + sizeof(int32_t) * M);
  l.inv = off;       off = align_up(off + sizeof(int32_t) * M);
  l.slot_e = off;    off = align_up(off + sizeof(int32_t) * M);
  l.cs_in = off;     off = align_up(off + sizeof(float2) * N * L * (d / 2));
  l.cs_out = off;    off = align_up(off + sizeof(float2) * N * L * (d / 2));
  l.z = off;         off = align_up(off + zel * M * d);
  l.h = off;         off = align_up(off + zel * M * d);  // H, then dZ
  l.dh = off;        off = align_up(off + zel * M * d);
  l.dx = off;        off = align_up(off + zel * M * d);  // per routed row
  l.wt = off;        if (l.wt_block) off = align_up(off + sizeof(uint32_t) * wwords);
  l.wpt = off;       off = align_up(off + sizeof(uint32_t) * wwords);
  l.wtt = off;       if (l.wt_block) off = align_up(off + sizeof(uint32_t) * wwords);
  l.tiles = off;     off = align_up(off + sizeof(int4) * l.max_tiles);
  l.tile_base = off; off = align_up(off + sizeof(int32_t) * (N + 1));
  l.part_in = off;   off = align_up(off + sizeof(float) * l.max_tiles * L * (d / 2));
  l.part_out = off;  off = align_up(off + sizeof(float) * l.max_tiles * L * (d / 2));
  l.dw_part = off;   off = align_up(off + sizeof(float) * dw_slots(dt, (int)M, d) * d * d);
  l.total = off;
  return l;
}

constexpr int kRouterMaxK = 64;
bool router_shape_ok(bmoe_dtype dt, int T, int d, int N, int k) {
  return shape_ok(dt, T, d, N, k) && valid_d16(d) && k <= kRouterMaxK;
}

bool bwd_shape_ok(bmoe_dtype dt, int T, int d, int N, int k) {
  return shape_ok(dt, T, d, N, k) && valid_d16(d) && d <= 4096;
}

// dW = alpha * dH^T Z (row-major [d][d], fp32), see dw_own_kernel.
// *slices: the number of fp32 partial products left in part for the
// backward's closing kernel to sum (0: dw written directly).
bmoe_status substrate_grad(bmoe_dtype dt, int M, int d, const void* dh, const void* z,
                           float alpha, float* dw, float* part, int* slices, hipStream_t s,
                           const KernelTiming& t) {
  *slices = dw_slots(dt, M, d);
  const hipError_t e =
      dw_own_kernel(dt, d)
          ? launch_dw(M, d, static_cast<const uint16_t*>(dh), static_cast<const uint16_t*>(z),
                      alpha, dw, part, s, t)
          : launch_dw_f32(dt, M, d, dh, z, alpha, dw, part, s, t);
  return e == hipSuccess ? BMOE_OK : BMOE_E_HIP;
}

}  // namespace
}  // namespace bmoe

using namespace bmoe;

extern "C" {

size_t bmoe_packed_words(int d) {
  if (!valid_d(d)) return 0;
  return (size_t)d * ((d + 15) / 16);
}

size_t bmoe_param_count(int d, int n_experts) {
  if (!valid_d(d) || n_experts < 1) return 0;
  return (size_t)d * d + 2 * (size_t)n_experts * log2i(d) * (d / 2);
}

size_t bmoe_workspace_bytes(bmoe_dtype dt, int T, int d, int n_experts, int k) {
  if (!shape_ok(dt, T, d, n_experts, k)) return 0;
  return fwd_layout(dt, T, d, n_experts, k).total;
}

size_t bmoe_pack_workspace_bytes(void) { return kAlign; }

bmoe_status bmoe_pack_ternary(const int8_t* w, int d, uint32_t* packed, void* ws,
                              size_t ws_bytes, void* stream) {
  if (!w || !packed) return BMOE_E_NULL;
  if (!valid_d(d)) return BMOE_E_SHAPE;
  if (!ws || ws_bytes < bmoe_pack_workspace_bytes()) return BMOE_E_WORKSPACE;
  if (!aligned16(w) || !aligned16(packed) || !aligned16(ws)) return BMOE_E_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_pack(w, d, packed, static_cast<int32_t*>(ws), s) != hipSuccess) return BMOE_E_HIP;
  return BMOE_OK;
}

bmoe_status bmoe_product(int M, int d, const void* z, const void* w, bmoe_wformat fmt,
                         float alpha, void* h, void* stream, void* const* events) {
  if (fmt != BMOE_W_2BIT && fmt != BMOE_W_BASE3) return BMOE_E_DTYPE;
  if (M < 0 || !valid_d(d) || d < 128) return BMOE_E_SHAPE;
  if (M == 0) return BMOE_OK;
  if (!z || !w || !h) return BMOE_E_NULL;
  if (!aligned16(z) || !aligned16(w) || !aligned16(h)) return BMOE_E_ALIGN;
  KernelTiming t;
  if (events) {
    t.start = static_cast<hipEvent_t>(events[0]);
    t.stop = static_cast<hipEvent_t>(events[1]);
  }
  if (launch_product(M, d, static_cast<const uint16_t*>(z), w, fmt, alpha,
                     static_cast<uint16_t*>(h), static_cast<hipStream_t>(stream), t) != hipSuccess)
    return BMOE_E_HIP;
  return BMOE_OK;
}

size_t bmoe_packed3_bytes(int d) {
  if (!valid_d16(d)) return 0;
  return ((size_t)d * d + 4) / 5;
}

bmoe_status bmoe_pack_ternary_b3(const int8_t* w, int d, uint8_t* packed3, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (!w || !packed3) return BMOE_E_NULL;
  if (!valid_d16(d)) return BMOE_E_SHAPE;
  if (!ws || ws_bytes < bmoe_pack_workspace_bytes()) return BMOE_E_WORKSPACE;
  if (!aligned16(w) || !aligned16(packed3) || !aligned16(ws)) return BMOE_E_ALIGN;
  if (launch_pack_b3(w, d, packed3, static_cast<int32_t*>(ws), static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return BMOE_E_HIP;
  return BMOE_OK;
}

bmoe_status bmoe_unpack_ternary_b3_timed(const uint8_t* packed3, int d, uint32_t* packed,
                                         void* ws, size_t ws_bytes, void* stream,
                                         void* const* events) {
  if (!packed3 || !packed) return BMOE_E_NULL;
  if (!valid_d16(d)) return BMOE_E_SHAPE;
  if (!ws || ws_bytes < bmoe_pack_workspace_bytes()) return BMOE_E_WORKSPACE;
  if (!aligned16(packed3) || !aligned16(packed) || !aligned16(ws)) return BMOE_E_ALIGN;
  KernelTiming t;
  if (events) {
    t.start = static_cast<hipEvent_t>(events[0]);
    t.stop = static_cast<hipEvent_t>(events[1]);
  }
  if (launch_unpack_b3(packed3, d, packed, static_cast<int32_t*>(ws),
                       static_cast<hipStream_t>(stream), t) != hipSuccess)
    return BMOE_E_HIP;
  return BMOE_OK;
}

bmoe_status bmoe_unpack_ternary_b3(const uint8_t* packed3, int d, uint32_t* packed, void* ws,
                                   size_t ws_bytes, void* stream) {
  return bmoe_unpack_ternary_b3_timed(packed3, d, packed, ws, ws_bytes, stream, nullptr);
}

namespace {
// status_at: where the kernels write the status word (NULL: the workspace's
// own word).
bmoe_status forward_impl(bmoe_dtype dt, int T, int d, int n_experts, int k, const void* x,
                         const int32_t* ids, const float* gates, const float* theta,
                         const float* phi, const uint32_t* w_packed, float alpha, void* y,
                         void* ws, size_t ws_bytes, int32_t* route_out, void* stream,
                         void* const* events, bool keep, int32_t* status_at = nullptr) {
  if (dt != BMOE_F32 && dt != BMOE_BF16) return BMOE_E_DTYPE;
  if (!shape_ok(dt, T, d, n_experts, k) || (keep && small_d(d))) return BMOE_E_SHAPE;
  if (T == 0) return BMOE_OK;
  if (!x || !ids || !gates || !theta || !phi || !w_packed || !y) return BMOE_E_NULL;
  const FwdLayout l = fwd_layout(dt, T, d, n_experts, k, keep);
  if (!ws || ws_bytes < l.total) return BMOE_E_WORKSPACE;
  const void* ptrs[] = {x, ids, gates, theta, phi, w_packed, y, ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return BMOE_E_ALIGN;
  if (route_out && (reinterpret_cast<uintptr_t>(route_out) & 3u)) return BMOE_E_ALIGN;

  char* base = static_cast<char*>(ws);
  const int M = T * k;
  RouteTables rt;
  if (route_out) {
    rt.offsets = route_out;
    rt.perm = route_out + n_experts + 1;
    rt.inv = rt.perm + M;
  } else {
    rt.offsets = reinterpret_cast<int32_t*>(base + l.offsets);
    rt.perm = reinterpret_cast<int32_t*>(base + l.perm);
    rt.inv = reinterpret_cast<int32_t*>(base + l.inv);
  }
  rt.slot_e = reinterpret_cast<int32_t*>(base + l.slot_e);
  int32_t* status = status_at ? status_at : reinterpret_cast<int32_t*>(base + l.status);
  float2* cs_in = reinterpret_cast<float2*>(base + l.cs_in);
  float2* cs_out = reinterpret_cast<float2*>(base + l.cs_out);
  void* z = base + l.z;
  void* h = base + l.h;
  void* u = base + l.u;
  hipStream_t s = static_cast<hipStream_t>(stream);

  int ki = 0;
  // Timing events of the next kernel (none when events is NULL).
  auto timing = [&]() -> KernelTiming {
    KernelTiming t;
    if (events) {
      t.start = static_cast<hipEvent_t>(events[2 * ki]);
      t.stop = static_cast<hipEvent_t>(events[2 * ki + 1]);
      ++ki;
    }
    return t;
  };
  // keep: the fused kernel also writes Z and H (d = 256, 512), or the
  // unfused path leaves them in the workspace.
  const bool fused = fused_supported(dt, d);
  const bool routed = !keep && fused && fused_wave_routes(dt, M, d, n_experts);
  const int wt_block = gemm_tiled_w_block(dt, M, d);
  uint32_t* wt = wt_block ? reinterpret_cast<uint32_t*>(base + l.wt) : nullptr;
  BwdSetup bs;  // keep: the backward's tiles and W_base^T, for bmoe_backward_kept
  if (keep) {
    bs.tiles = reinterpret_cast<int4*>(base + l.tiles);
    bs.tile_base = reinterpret_cast<int32_t*>(base + l.tile_base);
    bs.max_tiles = l.max_tiles;
    bs.tile_rows = bwd_tile_rows_for(d);
    bs.wpt = reinterpret_cast<uint32_t*>(base + l.wpt);
    bs.wtt = wt_block ? reinterpret_cast<uint32_t*>(base + l.wtt) : nullptr;
    bs.wtt_block = wt_block;
  }
  if (routed) {
    // Routing and coefficient tables inside the fused kernel: no prep launch.
    if (launch_fused_wave(M, d, k, n_experts, x, ids, gates, theta, phi, w_packed, alpha, u, rt,
                          status, s, timing()) != hipSuccess)
      return BMOE_E_HIP;
    if (launch_combine(dt, T, d, k, u, y, s, timing()) != hipSuccess) return BMOE_E_HIP;
    return BMOE_OK;
  }
  // The fused kernel after prep evaluates its own tiles' tables from the
  // angles: prep only routes, or with keep also writes the tables the
  // backward reads.
  const bool tables = !fused || keep;
  if (launch_prep(ids, M, n_experts, tables ? theta : nullptr, tables ? phi : nullptr, d, rt,
                  cs_in, cs_out, status, w_packed, wt, wt_block, s, timing(), bs) !=
      hipSuccess)
    return BMOE_E_HIP;
  if (small_d(d)) {
    // Rotations, product, gates and the sum over j in one launch.
    return launch_small(dt, T, d, k, n_experts, x, ids, gates, cs_in, cs_out, w_packed, alpha, y,
                        s, timing()) == hipSuccess
               ? BMOE_OK
               : BMOE_E_HIP;
  }
  if (fused) {
    if (launch_fused_wave_prepped(M, d, k, x, gates, theta, phi, w_packed, alpha, u,
                                  keep ? z : nullptr, keep ? h : nullptr, rt, s,
                                  timing()) != hipSuccess)
      return BMOE_E_HIP;
  } else {
    if (launch_bfly_in(dt, M, d, k, x, rt, cs_in, z, s, timing()) != hipSuccess)
      return BMOE_E_HIP;
    if (launch_gemm(dt, M, d, z, w_packed, wt, alpha, h, s, timing()) != hipSuccess)
      return BMOE_E_HIP;
    if (launch_bfly_out(dt, M, d, h, gates, rt, cs_out, u, s, timing()) != hipSuccess)
      return BMOE_E_HIP;
  }
  if (launch_combine(dt, T, d, k, u, y, s, timing()) != hipSuccess) return BMOE_E_HIP;
  return BMOE_OK;
}
}  // namespace

bmoe_status bmoe_forward_timed(bmoe_dtype dt, int T, int d, int n_experts, int k, const void* x,
                               const int32_t* ids, const float* gates, const float* theta,
                               const float* phi, const uint32_t* w_packed, float alpha, void* y,
                               void* ws, size_t ws_bytes, int32_t* route_out, void* stream,
                               void* const* events) {
  return forward_impl(dt, T, d, n_experts, k, x, ids, gates, theta, phi, w_packed, alpha, y, ws,
                      ws_bytes, route_out, stream, events, false);
}

}  // extern "C"

// ---- allocation-free forward -------------------------------------------
// The workspace of bmoe_forward_noalloc: one array per GPU, in the code
// object's device memory, held until the process ends. In host code `scratch`
// names a host-side stand-in, not device memory: kernels get the address
// hipGetSymbolAddress returns for the device, never the name itself.
static __device__ __align__(256) uint8_t scratch[BMOE_NOALLOC_MAX_WORKSPACE];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_addr[kMaxDevices] = {};

// The device address of `scratch` on the device `stream` belongs to (the
// current device for the NULL stream), looked up once per device with that
// device current.
bmoe_status scratch_for(hipStream_t stream, void** out) {
  int cur = 0, dev = 0;
  if (hipGetDevice(&cur) != hipSuccess) return BMOE_E_HIP;
  dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return BMOE_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return BMOE_E_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_addr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return BMOE_E_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return BMOE_E_HIP;
    if (e != hipSuccess || !p) return BMOE_E_HIP;
    scratch_addr[dev] = p;
  }
  *out = scratch_addr[dev];
  return BMOE_OK;
}
}  // namespace

extern "C" {

bmoe_status bmoe_forward_noalloc(bmoe_dtype dt, int T, int d, int n_experts, int k,
                                 const void* x, const int32_t* ids, const float* gates,
                                 const float* theta, const float* phi, const uint32_t* w_packed,
                                 float alpha, void* y, int32_t* route_out, int32_t* status,
                                 void* stream) {
  if (dt != BMOE_F32 && dt != BMOE_BF16) return BMOE_E_DTYPE;
  if (!shape_ok(dt, T, d, n_experts, k)) return BMOE_E_SHAPE;
  if (T == 0) return BMOE_OK;
  if (fwd_layout(dt, T, d, n_experts, k).total > BMOE_NOALLOC_MAX_WORKSPACE)
    return BMOE_E_WORKSPACE;
  if (status && (reinterpret_cast<uintptr_t>(status) & 3u)) return BMOE_E_ALIGN;
  void* ws = nullptr;
  const bmoe_status st = scratch_for(static_cast<hipStream_t>(stream), &ws);
  if (st != BMOE_OK) return st;
  return forward_impl(dt, T, d, n_experts, k, x, ids, gates, theta, phi, w_packed, alpha, y, ws,
                      BMOE_NOALLOC_MAX_WORKSPACE, route_out, stream, nullptr, false,
                      status ? status : nullptr);
}

size_t bmoe_forward_keep_workspace_bytes(bmoe_dtype dt, int T, int d, int n_experts, int k) {
  if (!shape_ok(dt, T, d, n_experts, k) || !valid_d16(d)) return 0;
  return fwd_layout(dt, T, d, n_experts, k, true).total;
}

bmoe_status bmoe_forward_keep(bmoe_dtype dt, int T, int d, int n_experts, int k, const void* x,
                              const int32_t* ids, const float* gates, const float* theta,
                              const float* phi, const uint32_t* w_packed, float alpha, void* y,
                              void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(dt, T, d, n_experts, k, x, ids, gates, theta, phi, w_packed, alpha, y, ws,
                      ws_bytes, nullptr, stream, nullptr, true);
}

bmoe_status bmoe_forward(bmoe_dtype dt, int T, int d, int n_experts, int k, const void* x,
                         const int32_t* ids, const float* gates, const float* theta,
                         const float* phi, const uint32_t* w_packed, float alpha, void* y,
                         void* ws, size_t ws_bytes, int32_t* route_out, void* stream) {
  return bmoe_forward_timed(dt, T, d, n_experts, k, x, ids, gates, theta, phi, w_packed, alpha, y,
                            ws, ws_bytes, route_out, stream, nullptr);
}

int bmoe_forward_kernel_count(bmoe_dtype dt, int T, int d, int n_experts, int k) {
  if (!shape_ok(dt, T, d, n_experts, k) || T == 0) return 0;
  if (small_d(d)) return 2;
  if (fused_wave_routes(dt, T * k, d, n_experts)) return 2;
  return fused_supported(dt, d) ? 3 : 5;
}

const char* bmoe_forward_kernel_name(bmoe_dtype dt, int T, int d, int n_experts, int k, int i) {
  static const char* routed_names[] = {"fused_wave_kernel", "combine_kernel"};
  static const char* small_names[] = {"prep_kernel", "small_kernel"};
  static const char* fused_names[] = {"prep_kernel", "fused_wave_kernel", "combine_kernel"};
  static const char* split_names[] = {"prep_kernel", "bfly_in_kernel", "gemm_kernel",
                                      "bfly_out_kernel", "combine_kernel"};
  if (i < 0 || i >= bmoe_forward_kernel_count(dt, T, d, n_experts, k)) return "";
  if (small_d(d)) return small_names[i];
  if (fused_wave_routes(dt, T * k, d, n_experts)) return routed_names[i];
  return fused_supported(dt, d) ? fused_names[i] : split_names[i];
}

bmoe_status bmoe_sync_status(const void* ws, void* stream) {
  if (!ws) return BMOE_E_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t v = 0;
  if (hipMemcpyAsync(&v, ws, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess) return BMOE_E_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return BMOE_E_HIP;
  if (v == BMOE_E_EXPERT) return BMOE_E_EXPERT;
  if (v == BMOE_E_TERNARY) return BMOE_E_TERNARY;
  return v == BMOE_OK ? BMOE_OK : BMOE_E_HIP;
}

size_t bmoe_backward_workspace_bytes(bmoe_dtype dt, int T, int d, int n_experts, int k) {
  if (!bwd_shape_ok(dt, T, d, n_experts, k)) return 0;
  return bwd_layout(dt, T, d, n_experts, k).total;
}

namespace {
// kept: the workspace of a bmoe_forward_keep call (routing and cos/sin
// tables, Z and H are read from it and not recomputed), or NULL.
bmoe_status backward_impl(bmoe_dtype dt, int T, int d, int n_experts, int k, const void* x,
                          const int32_t* ids, const float* gates, const float* theta,
                          const float* phi, const uint32_t* w_packed, float alpha,
                          const void* dy, void* dx, float* dgates, float* dtheta, float* dphi,
                          float* dw, const void* kept, size_t kept_bytes, void* ws,
                          size_t ws_bytes, void* stream, void* const* events) {
  if (dt != BMOE_F32 && dt != BMOE_BF16) return BMOE_E_DTYPE;
  if (!bwd_shape_ok(dt, T, d, n_experts, k)) return BMOE_E_SHAPE;
  if (T == 0) return BMOE_OK;
  if (!x || !gates || !w_packed || !dy || !dx || !dgates || !dtheta || !dphi) return BMOE_E_NULL;
  if (!kept && (!ids || !theta || !phi)) return BMOE_E_NULL;
  const BwdLayout l = bwd_layout(dt, T, d, n_experts, k);
  if (!ws || ws_bytes < l.total) return BMOE_E_WORKSPACE;
  const FwdLayout fl = fwd_layout(dt, T, d, n_experts, k, true);
  if (kept && kept_bytes < fl.total) return BMOE_E_WORKSPACE;
  const void* ptrs[] = {x, gates, w_packed, dy, dx, dgates, dtheta, dphi, ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return BMOE_E_ALIGN;
  if (!kept) {
    const void* rec[] = {ids, theta, phi};
    for (const void* p : rec)
      if (!aligned16(p)) return BMOE_E_ALIGN;
  }
  if ((dw && !aligned16(dw)) || (kept && !aligned16(kept))) return BMOE_E_ALIGN;

  char* base = static_cast<char*>(ws);
  // Tables, Z and H: this workspace (recomputed below) or the kept forward's.
  char* src = kept ? const_cast<char*>(static_cast<const char*>(kept)) : base;
  const size_t o_off = kept ? fl.offsets : l.offsets, o_perm = kept ? fl.perm : l.perm;
  const size_t o_inv = kept ? fl.inv : l.inv, o_slot = kept ? fl.slot_e : l.slot_e;
  const size_t o_csi = kept ? fl.cs_in : l.cs_in, o_cso = kept ? fl.cs_out : l.cs_out;
  const size_t o_z = kept ? fl.z : l.z, o_h = kept ? fl.h : l.h;
  const int M = T * k;
  RouteTables rt;
  rt.offsets = reinterpret_cast<int32_t*>(src + o_off);
  rt.perm = reinterpret_cast<int32_t*>(src + o_perm);
  rt.inv = reinterpret_cast<int32_t*>(src + o_inv);
  rt.slot_e = reinterpret_cast<int32_t*>(src + o_slot);
  int32_t* status = reinterpret_cast<int32_t*>(base + l.status);
  float2* cs_in = reinterpret_cast<float2*>(src + o_csi);
  float2* cs_out = reinterpret_cast<float2*>(src + o_cso);
  void* z = src + o_z;
  void* h = src + o_h;
  void* dz = base + l.h;  // dZ: this workspace's H region (the kept H stays intact)
  void* dh = base + l.dh;
  void* dxr = base + l.dx;
  uint32_t* wt = l.wt_block ? reinterpret_cast<uint32_t*>(base + l.wt) : nullptr;
  // Row tiles and W_base^T: written by this call's prep, or the kept forward's.
  uint32_t* wpt = reinterpret_cast<uint32_t*>(src + (kept ? fl.wpt : l.wpt));
  uint32_t* wtt =
      l.wt_block ? reinterpret_cast<uint32_t*>(src + (kept ? fl.wtt : l.wtt)) : nullptr;
  int4* tiles = reinterpret_cast<int4*>(src + (kept ? fl.tiles : l.tiles));
  int32_t* tile_base = reinterpret_cast<int32_t*>(src + (kept ? fl.tile_base : l.tile_base));
  float* part_in = reinterpret_cast<float*>(base + l.part_in);
  float* part_out = reinterpret_cast<float*>(base + l.part_out);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int ki = 0;
  // Timing events of the next launch (none when events is NULL).
  auto timing = [&]() -> KernelTiming {
    KernelTiming t;
    if (events) {
      t.start = static_cast<hipEvent_t>(events[2 * ki]);
      t.stop = static_cast<hipEvent_t>(events[2 * ki + 1]);
      ++ki;
    }
    return t;
  };

  // An empty timing slot for a launch the kept forward already did.
  auto skip = [&]() -> bool {
    const KernelTiming t = timing();
    return (!t.start || hipEventRecord(t.start, s) == hipSuccess) &&
           (!t.stop || hipEventRecord(t.stop, s) == hipSuccess);
  };
  // Forward recompute: routing, cos/sin (with the row tiles and W_base^T),
  // Z = B^T x, H = alpha Z W^T.
  if (kept) {
    // Bad ids were the forward's to report; the closing kernel clears this
    // workspace's status word.
    if (!skip()) return BMOE_E_HIP;
  } else {
    BwdSetup bs;
    bs.tiles = tiles;
    bs.tile_base = tile_base;
    bs.max_tiles = l.max_tiles;
    bs.tile_rows = bwd_tile_rows_for(d);
    bs.wpt = wpt;
    bs.wtt = wtt;
    bs.wtt_block = l.wt_block;
    if (launch_prep(ids, M, n_experts, theta, phi, d, rt, cs_in, cs_out, status, w_packed, wt,
                    l.wt_block, s, timing(), bs) != hipSuccess)
      return BMOE_E_HIP;
  }
  // d = 256, 512 (bf16): Z and H from the fused kernel, as bmoe_forward_keep
  // writes them; otherwise the input-side butterfly and the product.
  const bool fused_zh = fused_supported(dt, d);
  if (kept) {
    if (!skip() || (!fused_zh && !skip())) return BMOE_E_HIP;
  } else if (fused_zh) {
    if (launch_fused_wave_prepped(M, d, k, x, gates, theta, phi, w_packed, alpha, nullptr, z, h,
                                  rt, s, timing()) != hipSuccess)
      return BMOE_E_HIP;
  } else {
    if (launch_bfly_in(dt, M, d, k, x, rt, cs_in, z, s, timing()) != hipSuccess) return BMOE_E_HIP;
    if (launch_gemm(dt, M, d, z, w_packed, wt, alpha, h, s, timing()) != hipSuccess)
      return BMOE_E_HIP;
  }
  // Output side: dH, dgates, dphi partials.
  if (launch_bfly_bwd(false, dt, M, d, k, tiles, l.max_tiles, rt.perm, cs_out, gates, h, dy, dh,
                      dgates, part_out, s, timing()) != hipSuccess)
    return BMOE_E_HIP;
  float* dw_part = reinterpret_cast<float*>(base + l.dw_part);
  int dw_slices = 0;
  {
    const KernelTiming t = timing();
    if (dw) {
      if (substrate_grad(dt, M, d, dh, z, alpha, dw, dw_part, &dw_slices, s, t) != BMOE_OK)
        return BMOE_E_HIP;
    } else if ((t.start && hipEventRecord(t.start, s) != hipSuccess) ||
               (t.stop && hipEventRecord(t.stop, s) != hipSuccess)) {
      return BMOE_E_HIP;  // no dw: the slot's events bracket nothing
    }
  }
  // dZ = alpha dH W (the product with the transposed substrate).
  if (launch_gemm(dt, M, d, dh, wpt, wtt, alpha, dz, s, timing()) != hipSuccess) return BMOE_E_HIP;
  // Input side: dX per routed row, dtheta partials.
  if (launch_bfly_bwd(true, dt, M, d, k, tiles, l.max_tiles, rt.perm, cs_in, gates, x, dz, dxr,
                      nullptr, part_in, s, timing()) != hipSuccess)
    return BMOE_E_HIP;
  // dx_t = sum_j dX[t k + j], dphi / dtheta from the tile partials, and dW
  // from its row-range slices, in one launch.
  if (launch_bwd_finish(dt, T, d, k, dxr, dx, part_out, part_in, tile_base, n_experts, dphi,
                        dtheta, dw_part, dw_slices, dw, kept ? status : nullptr, s,
                        timing()) != hipSuccess)
    return BMOE_E_HIP;
  return BMOE_OK;
}
}  // namespace

bmoe_status bmoe_backward_timed(bmoe_dtype dt, int T, int d, int n_experts, int k,
                                const void* x, const int32_t* ids, const float* gates,
                                const float* theta, const float* phi, const uint32_t* w_packed,
                                float alpha, const void* dy, void* dx, float* dgates,
                                float* dtheta, float* dphi, float* dw, void* ws, size_t ws_bytes,
                                void* stream, void* const* events) {
  return backward_impl(dt, T, d, n_experts, k, x, ids, gates, theta, phi, w_packed, alpha, dy, dx,
                       dgates, dtheta, dphi, dw, nullptr, 0, ws, ws_bytes, stream, events);
}

bmoe_status bmoe_backward_kept_timed(bmoe_dtype dt, int T, int d, int n_experts, int k,
                                     const void* x, const float* gates,
                                     const uint32_t* w_packed, float alpha, const void* dy,
                                     void* dx, float* dgates, float* dtheta, float* dphi,
                                     float* dw, const void* fwd_ws, size_t fwd_ws_bytes, void* ws,
                                     size_t ws_bytes, void* stream, void* const* events) {
  if (!fwd_ws) return BMOE_E_NULL;
  return backward_impl(dt, T, d, n_experts, k, x, nullptr, gates, nullptr, nullptr, w_packed,
                       alpha, dy, dx, dgates, dtheta, dphi, dw, fwd_ws, fwd_ws_bytes, ws, ws_bytes,
                       stream, events);
}

bmoe_status bmoe_backward_kept(bmoe_dtype dt, int T, int d, int n_experts, int k, const void* x,
                               const float* gates, const uint32_t* w_packed, float alpha,
                               const void* dy, void* dx, float* dgates, float* dtheta,
                               float* dphi, float* dw, const void* fwd_ws, size_t fwd_ws_bytes,
                               void* ws, size_t ws_bytes, void* stream) {
  return bmoe_backward_kept_timed(dt, T, d, n_experts, k, x, gates, w_packed, alpha, dy, dx,
                                  dgates, dtheta, dphi, dw, fwd_ws, fwd_ws_bytes, ws, ws_bytes,
                                  stream, nullptr);
}

bmoe_status bmoe_backward(bmoe_dtype dt, int T, int d, int n_experts, int k, const void* x,
                          const int32_t* ids, const float* gates, const float* theta,
                          const float* phi, const uint32_t* w_packed, float alpha,
                          const void* dy, void* dx, float* dgates, float* dtheta, float* dphi,
                          float* dw, void* ws, size_t ws_bytes, void* stream) {
  return bmoe_backward_timed(dt, T, d, n_experts, k, x, ids, gates, theta, phi, w_packed, alpha,
                             dy, dx, dgates, dtheta, dphi, dw, ws, ws_bytes, stream, nullptr);
}

namespace {
const char* const kBackwardNames[] = {
    "prep_kernel",         "bfly_in_kernel",      "gemm_kernel",        "bfly_bwd_out_kernel",
    "dw_kernel",           "gemm_t_kernel",       "bfly_bwd_in_kernel", "finish_kernel"};
// d = 256, 512 (bf16): Z and H recomputed by the fused kernel in one launch.
const char* const kBackwardNamesFused[] = {
    "prep_kernel",         "fused_wave_kernel",   "bfly_bwd_out_kernel", "dw_kernel",
    "gemm_t_kernel",       "bfly_bwd_in_kernel",  "finish_kernel"};
}  // namespace

size_t bmoe_rotate_in_workspace_bytes(bmoe_dtype dt, int T, int d, int n_experts, int k) {
  if (!shape_ok(dt, T, d, n_experts, k) || !valid_d16(d)) return 0;
  return rot_layout(T, d, n_experts, k).total;
}

bmoe_status bmoe_rotate_in(bmoe_dtype dt, int T, int d, int n_experts, int k, const void* x,
                           const int32_t* ids, const float* theta, void* z, void* ws,
                           size_t ws_bytes, void* stream) {
  if (dt != BMOE_F32 && dt != BMOE_BF16) return BMOE_E_DTYPE;
  if (!shape_ok(dt, T, d, n_experts, k) || !valid_d16(d)) return BMOE_E_SHAPE;
  if (T == 0) return BMOE_OK;
  if (!x || !ids || !theta || !z) return BMOE_E_NULL;
  const RotLayout l = rot_layout(T, d, n_experts, k);
  if (!ws || ws_bytes < l.total) return BMOE_E_WORKSPACE;
  const void* ptrs[] = {x, ids, theta, z, ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return BMOE_E_ALIGN;
  char* base = static_cast<char*>(ws);
  RouteTables rt;
  rt.offsets = reinterpret_cast<int32_t*>(base + l.offsets);
  rt.perm = reinterpret_cast<int32_t*>(base + l.perm);
  rt.inv = reinterpret_cast<int32_t*>(base + l.inv);
  rt.slot_e = reinterpret_cast<int32_t*>(base + l.slot_e);
  float2* cs_in = reinterpret_cast<float2*>(base + l.cs_in);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int M = T * k;
  if (launch_prep(ids, M, n_experts, theta, nullptr, d, rt, cs_in, nullptr,
                  reinterpret_cast<int32_t*>(base + l.status), nullptr, nullptr, 0, s) !=
      hipSuccess)
    return BMOE_E_HIP;
  if (launch_bfly_in(dt, M, d, k, x, rt, cs_in, z, s, KernelTiming{}, true) != hipSuccess)
    return BMOE_E_HIP;
  return BMOE_OK;
}

bmoe_status bmoe_quant_error(bmoe_dtype dt, int rows, int d, const void* src, int m, int mode,
                             float* err, float* crest, void* stream) {
  if (dt != BMOE_F32 && dt != BMOE_BF16) return BMOE_E_DTYPE;
  if (rows < 0 || !valid_d16(d) || m < 1 || (mode != 0 && mode != 1)) return BMOE_E_SHAPE;
  if (rows == 0) return BMOE_OK;
  if (!src || !err) return BMOE_E_NULL;
  if (!aligned16(src) || !aligned16(err) || (crest && !aligned16(crest))) return BMOE_E_ALIGN;
  if (launch_quant_error(dt, rows, d, src, m, mode, err, crest,
                         static_cast<hipStream_t>(stream)) != hipSuccess)
    return BMOE_E_HIP;
  return BMOE_OK;
}

size_t bmoe_router_workspace_bytes(bmoe_dtype dt, int T, int d, int n_experts, int k) {
  if (!router_shape_ok(dt, T, d, n_experts, k)) return 0;
  return align_up(sizeof(float) * (size_t)T * n_experts + 1);
}

bmoe_status bmoe_router_timed(bmoe_dtype dt, int T, int d, int n_experts, int k, const void* x,
                              const void* w_router, int32_t* ids, float* gates, float* logits,
                              void* ws, size_t ws_bytes, void* stream, void* const* events) {
  if (dt != BMOE_F32 && dt != BMOE_BF16) return BMOE_E_DTYPE;
  if (!router_shape_ok(dt, T, d, n_experts, k)) return BMOE_E_SHAPE;
  if (T == 0) return BMOE_OK;
  if (!x || !w_router || !ids || !gates) return BMOE_E_NULL;
  float* lg = logits;
  if (!lg) {
    if (!ws || ws_bytes < bmoe_router_workspace_bytes(dt, T, d, n_experts, k))
      return BMOE_E_WORKSPACE;
    lg = static_cast<float*>(ws);
  }
  const void* ptrs[] = {x, w_router, ids, gates, lg};
  for (const void* p : ptrs)
    if (!aligned16(p)) return BMOE_E_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  KernelTiming t0, t1;
  if (events) {
    t0.start = static_cast<hipEvent_t>(events[0]);
    t0.stop = static_cast<hipEvent_t>(events[1]);
    t1.start = static_cast<hipEvent_t>(events[2]);
    t1.stop = static_cast<hipEvent_t>(events[3]);
  }
  if (launch_router_logits(dt, T, d, n_experts, x, w_router, lg, s, t0) != hipSuccess)
    return BMOE_E_HIP;
  if (launch_topk(lg, T, n_experts, k, ids, gates, s, t1) != hipSuccess) return BMOE_E_HIP;
  return BMOE_OK;
}

bmoe_status bmoe_router(bmoe_dtype dt, int T, int d, int n_experts, int k, const void* x,
                        const void* w_router, int32_t* ids, float* gates, float* logits, void* ws,
                        size_t ws_bytes, void* stream) {
  return bmoe_router_timed(dt, T, d, n_experts, k, x, w_router, ids, gates, logits, ws, ws_bytes,
                           stream, nullptr);
}

int bmoe_backward_kernel_count(bmoe_dtype dt, int T, int d, int n_experts, int k) {
  if (!bwd_shape_ok(dt, T, d, n_experts, k) || T == 0) return 0;
  return fused_supported(dt, d) ? 7 : 8;
}

const char* bmoe_backward_kernel_name(bmoe_dtype dt, int T, int d, int n_experts, int k, int i) {
  if (i < 0 || i >= bmoe_backward_kernel_count(dt, T, d, n_experts, k)) return "";
  return fused_supported(dt, d) ? kBackwardNamesFused[i] : kBackwardNames[i];
}

const char* bmoe_status_str(bmoe_status s) {
  switch (s) {
    case BMOE_OK: return "ok";
    case BMOE_E_NULL: return "required pointer is NULL";
    case BMOE_E_SHAPE:
      return "unsupported shape (d power of two in [2,8192] for the forward and pack, [16,8192] "
             "otherwise (backward: [16,4096]); 1<=N<=4096, 1<=k<=N, T>=0)";
    case BMOE_E_DTYPE: return "unknown dtype";
    case BMOE_E_TERNARY: return "W_base entry outside {-1,0,+1}";
    case BMOE_E_EXPERT: return "expert id outside [0,N)";
    case BMOE_E_WORKSPACE: return "workspace missing or too small";
    case BMOE_E_HIP: return "HIP runtime error";
    case BMOE_E_ALIGN: return "pointer not 16-byte aligned";
  }
  return "unknown status";
}

}  // extern "C"
