// C ABI of libbmoe.so: host-side validation, workspace carving and the
// launch sequence of the forward. Every step of the forward runs in the HIP
// kernels of this library; nothing here touches element data.
#include <climits>

#include "common.h"
#include "kernels.h"

namespace bmoe {
namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool valid_d(int d) { return d >= 16 && d <= 8192 && (d & (d - 1)) == 0; }

int log2i(int d) {
  int L = 0;
  while ((1 << L) < d) ++L;
  return L;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct FwdLayout {
  size_t status, offsets, perm, inv, slot_e, cs_in, cs_out, z, h, u, w16, wt, total;
};

bool shape_ok(bmoe_dtype dt, int T, int d, int N, int k) {
  if (dt != BMOE_F32 && dt != BMOE_BF16) return false;
  if (!valid_d(d) || N < 1 || N > kMaxExperts || k < 1 || k > N || T < 0) return false;
  if ((long long)T * k > INT_MAX) return false;
  return true;
}

FwdLayout fwd_layout(bmoe_dtype dt, int T, int d, int N, int k) {
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
  l.cs_in = off;   off = align_up(off + sizeof(float2) * N * L * (d / 2));
  l.cs_out = off;  off = align_up(off + sizeof(float2) * N * L * (d / 2));
  const bool fused = fused_supported(dt, d);
  // The fused path keeps Z and H on chip; only U (and the bf16 substrate)
  // live in the workspace.
  l.z = off;       if (!fused) off = align_up(off + zel * M * d);
  l.h = off;       if (!fused) off = align_up(off + zel * M * d);
  l.u = off;       off = align_up(off + zel * M * d);
  l.w16 = off;
  if (fused) off = align_up(off + sizeof(uint16_t) * (size_t)d * d);
  // Tile-major copy of the packed substrate for the large-tile product.
  l.wt = off;
  if (gemm_tiled_w_block(dt, (int)M, d)) off = align_up(off + sizeof(uint32_t) * (size_t)d * (d / 16));
  l.total = off;
  return l;
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

bmoe_status bmoe_forward_timed(bmoe_dtype dt, int T, int d, int n_experts, int k, const void* x,
                               const int32_t* ids, const float* gates, const float* theta,
                               const float* phi, const uint32_t* w_packed, float alpha, void* y,
                               void* ws, size_t ws_bytes, int32_t* route_out, void* stream,
                               void* const* events) {
  if (dt != BMOE_F32 && dt != BMOE_BF16) return BMOE_E_DTYPE;
  if (!shape_ok(dt, T, d, n_experts, k)) return BMOE_E_SHAPE;
  if (T == 0) return BMOE_OK;
  if (!x || !ids || !gates || !theta || !phi || !w_packed || !y) return BMOE_E_NULL;
  const FwdLayout l = fwd_layout(dt, T, d, n_experts, k);
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
  int32_t* status = reinterpret_cast<int32_t*>(base + l.status);
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
  const bool fused = fused_supported(dt, d);
  uint16_t* w16 = fused ? reinterpret_cast<uint16_t*>(base + l.w16) : nullptr;
  const int wt_block = gemm_tiled_w_block(dt, M, d);
  uint32_t* wt = wt_block ? reinterpret_cast<uint32_t*>(base + l.wt) : nullptr;
  if (launch_prep(ids, M, n_experts, theta, phi, d, rt, cs_in, cs_out, status, w_packed, w16, wt,
                  wt_block, s, timing()) != hipSuccess)
    return BMOE_E_HIP;
  if (fused) {
    if (launch_fused(M, d, k, x, gates, rt, cs_in, cs_out, w16, w_packed, alpha, u, s,
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

bmoe_status bmoe_forward(bmoe_dtype dt, int T, int d, int n_experts, int k, const void* x,
                         const int32_t* ids, const float* gates, const float* theta,
                         const float* phi, const uint32_t* w_packed, float alpha, void* y,
                         void* ws, size_t ws_bytes, int32_t* route_out, void* stream) {
  return bmoe_forward_timed(dt, T, d, n_experts, k, x, ids, gates, theta, phi, w_packed, alpha, y,
                            ws, ws_bytes, route_out, stream, nullptr);
}

int bmoe_forward_kernel_count(bmoe_dtype dt, int T, int d, int n_experts, int k) {
  if (!shape_ok(dt, T, d, n_experts, k) || T == 0) return 0;
  return fused_supported(dt, d) ? 3 : 5;
}

const char* bmoe_forward_kernel_name(bmoe_dtype dt, int T, int d, int n_experts, int k, int i) {
  static const char* fused_names[] = {"prep_kernel", "fused_kernel", "combine_kernel"};
  static const char* split_names[] = {"prep_kernel", "bfly_in_kernel", "gemm_kernel",
                                      "bfly_out_kernel", "combine_kernel"};
  if (i < 0 || i >= bmoe_forward_kernel_count(dt, T, d, n_experts, k)) return "";
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

const char* bmoe_status_str(bmoe_status s) {
  switch (s) {
    case BMOE_OK: return "ok";
    case BMOE_E_NULL: return "required pointer is NULL";
    case BMOE_E_SHAPE: return "unsupported shape (d power of two in [16,8192], 1<=N<=4096, 1<=k<=N, T>=0)";
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
