"""Thin ctypes binding of libbmoe.so (declared in include/bmoe.h).

Argument marshalling only: every step of the forward runs in the library's
HIP kernels. torch supplies device memory and the current stream. There is
no CPU fallback: if the library is missing, loading it raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbmoe.so")
_lib = None

BMOE_F32 = 0
BMOE_BF16 = 1
BMOE_E_TERNARY = 4
BMOE_E_EXPERT = 5

STATUS = {
    0: "BMOE_OK", 1: "BMOE_E_NULL", 2: "BMOE_E_SHAPE", 3: "BMOE_E_DTYPE",
    4: "BMOE_E_TERNARY", 5: "BMOE_E_EXPERT", 6: "BMOE_E_WORKSPACE", 7: "BMOE_E_HIP",
    8: "BMOE_E_ALIGN",
}


class BmoeError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {STATUS.get(code, code)} ({lib().bmoe_status_str(code).decode()})")
        self.code = code


def lib():
    """Load libbmoe.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m butterfly_rotated_ternary_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        c_int, c_sz, vp, c_f = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
        L.bmoe_packed_words.argtypes = [c_int]
        L.bmoe_packed_words.restype = c_sz
        L.bmoe_param_count.argtypes = [c_int, c_int]
        L.bmoe_param_count.restype = c_sz
        L.bmoe_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int]
        L.bmoe_workspace_bytes.restype = c_sz
        L.bmoe_pack_workspace_bytes.argtypes = []
        L.bmoe_pack_workspace_bytes.restype = c_sz
        L.bmoe_pack_ternary.argtypes = [vp, c_int, vp, vp, c_sz, vp]
        L.bmoe_pack_ternary.restype = c_int
        L.bmoe_packed3_bytes.argtypes = [c_int]
        L.bmoe_packed3_bytes.restype = c_sz
        L.bmoe_pack_ternary_b3.argtypes = [vp, c_int, vp, vp, c_sz, vp]
        L.bmoe_pack_ternary_b3.restype = c_int
        L.bmoe_unpack_ternary_b3.argtypes = [vp, c_int, vp, vp, c_sz, vp]
        L.bmoe_unpack_ternary_b3.restype = c_int
        L.bmoe_unpack_ternary_b3_timed.argtypes = [vp, c_int, vp, vp, c_sz, vp, vp]
        L.bmoe_unpack_ternary_b3_timed.restype = c_int
        L.bmoe_forward.argtypes = [c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp, vp, c_f,
                                   vp, vp, c_sz, vp, vp]
        L.bmoe_forward.restype = c_int
        L.bmoe_forward_noalloc.argtypes = [c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp,
                                           vp, c_f, vp, vp, vp, vp]
        L.bmoe_forward_noalloc.restype = c_int
        c_dp = ctypes.POINTER(ctypes.c_double)
        for name in ("bmoe_ceiling_mfma_bf16", "bmoe_ceiling_valu_f32"):
            getattr(L, name).argtypes = [c_int, vp, vp, vp, c_dp]
            getattr(L, name).restype = c_int
        L.bmoe_ceiling_copy.argtypes = [vp, vp, c_sz, vp, vp]
        L.bmoe_ceiling_copy.restype = c_int
        L.bmoe_product.argtypes = [c_int, c_int, vp, vp, c_int, c_f, vp, vp, vp]
        L.bmoe_product.restype = c_int
        L.bmoe_forward_timed.argtypes = L.bmoe_forward.argtypes + [vp]
        L.bmoe_forward_timed.restype = c_int
        L.bmoe_forward_kernel_count.argtypes = [c_int, c_int, c_int, c_int, c_int]
        L.bmoe_forward_kernel_count.restype = c_int
        L.bmoe_forward_kernel_name.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int]
        L.bmoe_forward_kernel_name.restype = ctypes.c_char_p
        L.bmoe_sync_status.argtypes = [vp, vp]
        L.bmoe_sync_status.restype = c_int
        L.bmoe_status_str.argtypes = [c_int]
        L.bmoe_status_str.restype = ctypes.c_char_p
        L.bmoe_backward_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int]
        L.bmoe_backward_workspace_bytes.restype = c_sz
        L.bmoe_backward.argtypes = [c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp, vp,
                                    c_f, vp, vp, vp, vp, vp, vp, vp, c_sz, vp]
        L.bmoe_backward.restype = c_int
        L.bmoe_forward_keep_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int]
        L.bmoe_forward_keep_workspace_bytes.restype = c_sz
        L.bmoe_forward_keep.argtypes = [c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp,
                                        vp, c_f, vp, vp, c_sz, vp]
        L.bmoe_forward_keep.restype = c_int
        L.bmoe_backward_kept.argtypes = [c_int, c_int, c_int, c_int, c_int, vp, vp, vp, c_f, vp,
                                         vp, vp, vp, vp, vp, vp, c_sz, vp, c_sz, vp]
        L.bmoe_backward_kept.restype = c_int
        L.bmoe_backward_kept_timed.argtypes = L.bmoe_backward_kept.argtypes + [vp]
        L.bmoe_backward_kept_timed.restype = c_int
        L.bmoe_rotate_in_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int]
        L.bmoe_rotate_in_workspace_bytes.restype = c_sz
        L.bmoe_rotate_in.argtypes = [c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp, c_sz,
                                     vp]
        L.bmoe_rotate_in.restype = c_int
        L.bmoe_quant_error.argtypes = [c_int, c_int, c_int, vp, c_int, c_int, vp, vp, vp]
        L.bmoe_quant_error.restype = c_int
        L.bmoe_router_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int]
        L.bmoe_router_workspace_bytes.restype = c_sz
        L.bmoe_router.argtypes = [c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp, vp, c_sz,
                                  vp]
        L.bmoe_router.restype = c_int
        L.bmoe_router_timed.argtypes = L.bmoe_router.argtypes + [vp]
        L.bmoe_router_timed.restype = c_int
        L.bmoe_backward_timed.argtypes = L.bmoe_backward.argtypes + [vp]
        L.bmoe_backward_timed.restype = c_int
        L.bmoe_backward_kernel_count.argtypes = [c_int, c_int, c_int, c_int, c_int]
        L.bmoe_backward_kernel_count.restype = c_int
        L.bmoe_backward_kernel_name.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int]
        L.bmoe_backward_kernel_name.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream=None):
    """Make `stream` torch's current stream while a wrapper allocates and
    launches: the caching allocator then ties the temporary workspace and the
    outputs to the stream the kernels run on, so memory freed when the wrapper
    returns is not handed to other work before those kernels finish."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _check(code: int, what: str):
    if code != 0:
        raise BmoeError(code, what)


# ---- the C entry points, same names -------------------------------------

def bmoe_packed_words(d: int) -> int:
    return lib().bmoe_packed_words(d)


def bmoe_param_count(d: int, n_experts: int) -> int:
    return lib().bmoe_param_count(d, n_experts)


def bmoe_workspace_bytes(dt: int, T: int, d: int, n_experts: int, k: int) -> int:
    return lib().bmoe_workspace_bytes(dt, T, d, n_experts, k)


def bmoe_pack_workspace_bytes() -> int:
    return lib().bmoe_pack_workspace_bytes()


def bmoe_pack_ternary(w: torch.Tensor, d: int, packed: torch.Tensor, ws: torch.Tensor,
                      stream=None) -> int:
    return lib().bmoe_pack_ternary(_ptr(w), d, _ptr(packed), _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream))


def bmoe_packed3_bytes(d: int) -> int:
    return lib().bmoe_packed3_bytes(d)


def bmoe_pack_ternary_b3(w: torch.Tensor, d: int, packed3: torch.Tensor, ws: torch.Tensor,
                         stream=None) -> int:
    return lib().bmoe_pack_ternary_b3(_ptr(w), d, _ptr(packed3), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(stream))


def bmoe_unpack_ternary_b3(packed3: torch.Tensor, d: int, packed: torch.Tensor,
                           ws: torch.Tensor, stream=None) -> int:
    return lib().bmoe_unpack_ternary_b3(_ptr(packed3), d, _ptr(packed), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream))


def bmoe_unpack_ternary_b3_timed(packed3: torch.Tensor, d: int, packed: torch.Tensor,
                                 ws: torch.Tensor, stream=None, events=None) -> int:
    ev = None
    if events is not None:
        ev = (ctypes.c_void_p * len(events))(*events)
    return lib().bmoe_unpack_ternary_b3_timed(_ptr(packed3), d, _ptr(packed), _ptr(ws),
                                              ws.numel() * ws.element_size(), _stream(stream), ev)


def bmoe_forward(dt: int, T: int, d: int, n_experts: int, k: int, x, ids, gates, theta, phi,
                 w_packed, alpha: float, y, ws, route_out=None, stream=None) -> int:
    return lib().bmoe_forward(dt, T, d, n_experts, k, _ptr(x), _ptr(ids), _ptr(gates), _ptr(theta),
                              _ptr(phi), _ptr(w_packed), float(alpha), _ptr(y), _ptr(ws),
                              ws.numel() * ws.element_size(), _ptr(route_out), _stream(stream))


def bmoe_forward_timed(dt: int, T: int, d: int, n_experts: int, k: int, x, ids, gates, theta, phi,
                       w_packed, alpha: float, y, ws, route_out=None, stream=None,
                       events=None) -> int:
    """``events``: raw hipEvent_t handles (ints), two per kernel: the start and
    stop events of kernel i are events[2i] and events[2i+1]."""
    ev = None
    if events is not None:
        ev = (ctypes.c_void_p * len(events))(*events)
    return lib().bmoe_forward_timed(dt, T, d, n_experts, k, _ptr(x), _ptr(ids), _ptr(gates),
                                    _ptr(theta), _ptr(phi), _ptr(w_packed), float(alpha), _ptr(y),
                                    _ptr(ws), ws.numel() * ws.element_size(), _ptr(route_out),
                                    _stream(stream), ev)


def bmoe_forward_noalloc(dt: int, T: int, d: int, n_experts: int, k: int, x, ids, gates, theta,
                         phi, w_packed, alpha: float, y, route_out=None, status=None,
                         stream=None) -> int:
    return lib().bmoe_forward_noalloc(dt, T, d, n_experts, k, _ptr(x), _ptr(ids), _ptr(gates),
                                      _ptr(theta), _ptr(phi), _ptr(w_packed), alpha, _ptr(y),
                                      _ptr(route_out), _ptr(status), _stream(stream))


BMOE_NOALLOC_MAX_WORKSPACE = 64 << 20


BMOE_W_2BIT = 0
BMOE_W_BASE3 = 1


def bmoe_product(M: int, d: int, z, w, fmt: int, alpha: float, h, stream=None,
                 events=None) -> int:
    return lib().bmoe_product(M, d, _ptr(z), _ptr(w), fmt, alpha, _ptr(h), _stream(stream),
                              _events_arg(events))


BMOE_CEILING_SINK_FLOATS = 256 * 8 * 256


def _events_arg(events):
    return None if events is None else (ctypes.c_void_p * len(events))(*events)


def bmoe_ceiling_mfma_bf16(iters: int, sink, stream=None, events=None):
    """(status, flops executed)."""
    f = ctypes.c_double()
    rc = lib().bmoe_ceiling_mfma_bf16(iters, _ptr(sink), _stream(stream), _events_arg(events),
                                      ctypes.byref(f))
    return rc, f.value


def bmoe_ceiling_valu_f32(iters: int, sink, stream=None, events=None):
    """(status, flops executed)."""
    f = ctypes.c_double()
    rc = lib().bmoe_ceiling_valu_f32(iters, _ptr(sink), _stream(stream), _events_arg(events),
                                     ctypes.byref(f))
    return rc, f.value


def bmoe_ceiling_copy(src, dst, nbytes: int, stream=None, events=None) -> int:
    return lib().bmoe_ceiling_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream),
                                   _events_arg(events))


def bmoe_forward_kernel_count(dt: int, T: int, d: int, n_experts: int, k: int) -> int:
    return lib().bmoe_forward_kernel_count(dt, T, d, n_experts, k)


def bmoe_forward_kernel_name(dt: int, T: int, d: int, n_experts: int, k: int, i: int) -> str:
    return lib().bmoe_forward_kernel_name(dt, T, d, n_experts, k, i).decode()


def bmoe_sync_status(ws: torch.Tensor, stream=None) -> int:
    return lib().bmoe_sync_status(_ptr(ws), _stream(stream))


def bmoe_status_str(code: int) -> str:
    return lib().bmoe_status_str(code).decode()


def bmoe_backward_workspace_bytes(dt: int, T: int, d: int, n_experts: int, k: int) -> int:
    return lib().bmoe_backward_workspace_bytes(dt, T, d, n_experts, k)


def bmoe_backward(dt: int, T: int, d: int, n_experts: int, k: int, x, ids, gates, theta, phi,
                  w_packed, alpha: float, dy, dx, dgates, dtheta, dphi, dw, ws,
                  stream=None) -> int:
    return lib().bmoe_backward(dt, T, d, n_experts, k, _ptr(x), _ptr(ids), _ptr(gates),
                               _ptr(theta), _ptr(phi), _ptr(w_packed), float(alpha), _ptr(dy),
                               _ptr(dx), _ptr(dgates), _ptr(dtheta), _ptr(dphi), _ptr(dw),
                               _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))


def bmoe_backward_timed(dt: int, T: int, d: int, n_experts: int, k: int, x, ids, gates, theta,
                        phi, w_packed, alpha: float, dy, dx, dgates, dtheta, dphi, dw, ws,
                        stream=None, events=None) -> int:
    """``events``: raw hipEvent_t handles (ints), two per launch (start, stop)."""
    ev = None
    if events is not None:
        ev = (ctypes.c_void_p * len(events))(*events)
    return lib().bmoe_backward_timed(dt, T, d, n_experts, k, _ptr(x), _ptr(ids), _ptr(gates),
                                     _ptr(theta), _ptr(phi), _ptr(w_packed), float(alpha),
                                     _ptr(dy), _ptr(dx), _ptr(dgates), _ptr(dtheta), _ptr(dphi),
                                     _ptr(dw), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream), ev)


def bmoe_backward_kernel_count(dt: int, T: int, d: int, n_experts: int, k: int) -> int:
    return lib().bmoe_backward_kernel_count(dt, T, d, n_experts, k)


def bmoe_backward_kernel_name(dt: int, T: int, d: int, n_experts: int, k: int, i: int) -> str:
    return lib().bmoe_backward_kernel_name(dt, T, d, n_experts, k, i).decode()


def bmoe_forward_keep_workspace_bytes(dt: int, T: int, d: int, n_experts: int, k: int) -> int:
    return lib().bmoe_forward_keep_workspace_bytes(dt, T, d, n_experts, k)


def bmoe_forward_keep(dt: int, T: int, d: int, n_experts: int, k: int, x, ids, gates, theta, phi,
                      w_packed, alpha: float, y, ws, stream=None) -> int:
    return lib().bmoe_forward_keep(dt, T, d, n_experts, k, _ptr(x), _ptr(ids), _ptr(gates),
                                   _ptr(theta), _ptr(phi), _ptr(w_packed), float(alpha), _ptr(y),
                                   _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))


def bmoe_backward_kept(dt: int, T: int, d: int, n_experts: int, k: int, x, gates, w_packed,
                       alpha: float, dy, dx, dgates, dtheta, dphi, dw, fwd_ws, ws,
                       stream=None) -> int:
    return lib().bmoe_backward_kept(dt, T, d, n_experts, k, _ptr(x), _ptr(gates),
                                    _ptr(w_packed), float(alpha), _ptr(dy), _ptr(dx),
                                    _ptr(dgates), _ptr(dtheta), _ptr(dphi), _ptr(dw),
                                    _ptr(fwd_ws), fwd_ws.numel() * fwd_ws.element_size(),
                                    _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))


def bmoe_backward_kept_timed(dt: int, T: int, d: int, n_experts: int, k: int, x, gates,
                             w_packed, alpha: float, dy, dx, dgates, dtheta, dphi, dw, fwd_ws,
                             ws, stream=None, events=None) -> int:
    ev = None
    if events is not None:
        ev = (ctypes.c_void_p * len(events))(*events)
    return lib().bmoe_backward_kept_timed(dt, T, d, n_experts, k, _ptr(x), _ptr(gates),
                                          _ptr(w_packed), float(alpha), _ptr(dy), _ptr(dx),
                                          _ptr(dgates), _ptr(dtheta), _ptr(dphi), _ptr(dw),
                                          _ptr(fwd_ws), fwd_ws.numel() * fwd_ws.element_size(),
                                          _ptr(ws), ws.numel() * ws.element_size(),
                                          _stream(stream), ev)


def bmoe_rotate_in_workspace_bytes(dt: int, T: int, d: int, n_experts: int, k: int) -> int:
    return lib().bmoe_rotate_in_workspace_bytes(dt, T, d, n_experts, k)


def bmoe_rotate_in(dt: int, T: int, d: int, n_experts: int, k: int, x, ids, theta, z, ws,
                   stream=None) -> int:
    return lib().bmoe_rotate_in(dt, T, d, n_experts, k, _ptr(x), _ptr(ids), _ptr(theta), _ptr(z),
                                _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))


def bmoe_quant_error(dt: int, rows: int, d: int, src, m: int, mode: int, err, crest=None,
                     stream=None) -> int:
    return lib().bmoe_quant_error(dt, rows, d, _ptr(src), m, mode, _ptr(err), _ptr(crest),
                                  _stream(stream))


def bmoe_router_workspace_bytes(dt: int, T: int, d: int, n_experts: int, k: int) -> int:
    return lib().bmoe_router_workspace_bytes(dt, T, d, n_experts, k)


def bmoe_router(dt: int, T: int, d: int, n_experts: int, k: int, x, w_router, ids, gates,
                logits=None, ws=None, stream=None) -> int:
    nb = 0 if ws is None else ws.numel() * ws.element_size()
    return lib().bmoe_router(dt, T, d, n_experts, k, _ptr(x), _ptr(w_router), _ptr(ids),
                             _ptr(gates), _ptr(logits), _ptr(ws), nb, _stream(stream))


def bmoe_router_timed(dt: int, T: int, d: int, n_experts: int, k: int, x, w_router, ids, gates,
                      logits=None, ws=None, stream=None, events=None) -> int:
    """``events``: 4 raw hipEvent_t handles (start/stop of the logits and
    top-k launches)."""
    ev = None
    if events is not None:
        ev = (ctypes.c_void_p * len(events))(*events)
    nb = 0 if ws is None else ws.numel() * ws.element_size()
    return lib().bmoe_router_timed(dt, T, d, n_experts, k, _ptr(x), _ptr(w_router), _ptr(ids),
                                   _ptr(gates), _ptr(logits), _ptr(ws), nb, _stream(stream), ev)


# ---- conveniences over the entry points (allocation + error checks) -------

def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BMOE_BF16
    if t.dtype == torch.float32:
        return BMOE_F32
    raise TypeError(f"x must be float32 or bfloat16, got {t.dtype}")


def pack_ternary(w: torch.Tensor) -> torch.Tensor:
    """int8 [d][d] device tensor -> packed uint32 words (as int32 storage)."""
    d = w.shape[0]
    n = bmoe_packed_words(d)
    if n == 0:
        raise BmoeError(2, "bmoe_pack_ternary")
    packed = torch.empty(n, dtype=torch.int32, device=w.device)
    ws = torch.empty(bmoe_pack_workspace_bytes(), dtype=torch.uint8, device=w.device)
    _check(bmoe_pack_ternary(w.contiguous(), d, packed, ws), "bmoe_pack_ternary")
    _check(bmoe_sync_status(ws), "bmoe_pack_ternary")
    return packed


class Workspace:
    """Caller-owned workspace sized for one shape (reused across calls)."""

    def __init__(self, dt: int, T: int, d: int, n_experts: int, k: int, device="cuda"):
        n = bmoe_workspace_bytes(dt, T, d, n_experts, k)
        if n == 0:
            raise BmoeError(2, "bmoe_workspace_bytes")
        self.buf = torch.empty(n, dtype=torch.uint8, device=device)
        self.key = (dt, T, d, n_experts, k)


def forward(x: torch.Tensor, ids: torch.Tensor, gates: torch.Tensor, theta: torch.Tensor,
            phi: torch.Tensor, w_packed: torch.Tensor, alpha: float, *, y=None, ws=None,
            route_out=None, stream=None) -> torch.Tensor:
    with _on(stream):
        T, d = x.shape
        k = ids.shape[1]
        N = theta.shape[0]
        dt = dtype_code(x)
        if y is None:
            y = torch.empty_like(x)
        if ws is None:
            ws = Workspace(dt, T, d, N, k, device=x.device)
        _check(bmoe_forward(dt, T, d, N, k, x, ids, gates, theta, phi, w_packed, alpha, y, ws.buf,
                            route_out, stream), "bmoe_forward")
        return y


def backward(x: torch.Tensor, ids: torch.Tensor, gates: torch.Tensor, theta: torch.Tensor,
             phi: torch.Tensor, w_packed: torch.Tensor, alpha: float, dy: torch.Tensor, *,
             want_dw: bool = True, stream=None) -> dict:
    """Gradients of sum(dy * y) for the layer bmoe_forward computes: dict of
    dx (dtype of x), dgates, dtheta, dphi and (want_dw) dw, all fp32 but dx."""
    with _on(stream):
        T, d = x.shape
        k = ids.shape[1]
        N = theta.shape[0]
        dt = dtype_code(x)
        n = bmoe_backward_workspace_bytes(dt, T, d, N, k)
        if n == 0:
            raise BmoeError(2, "bmoe_backward_workspace_bytes")
        ws = torch.empty(n, dtype=torch.uint8, device=x.device)
        out = {
            "dx": torch.empty_like(x),
            "dgates": torch.empty(T, k, dtype=torch.float32, device=x.device),
            "dtheta": torch.empty_like(theta),
            "dphi": torch.empty_like(phi),
            "dw": torch.empty(d, d, dtype=torch.float32, device=x.device) if want_dw else None,
        }
        _check(bmoe_backward(dt, T, d, N, k, x, ids, gates, theta, phi, w_packed, alpha, dy,
                             out["dx"], out["dgates"], out["dtheta"], out["dphi"], out["dw"], ws,
                             stream), "bmoe_backward")
        return out


def route(x: torch.Tensor, w_router: torch.Tensor, k: int, *, want_logits: bool = False,
          stream=None):
    """Router: (ids int32 [T][k], gates fp32 [T][k]) for bmoe_forward, plus
    the fp32 [T][N] logits when want_logits."""
    with _on(stream):
        T, d = x.shape
        N = w_router.shape[0]
        dt = dtype_code(x)
        if w_router.dtype != x.dtype or w_router.shape[1] != d:
            raise ValueError("w_router must be [N][d] in x's dtype")
        ids = torch.empty(T, k, dtype=torch.int32, device=x.device)
        gates = torch.empty(T, k, dtype=torch.float32, device=x.device)
        logits = torch.empty(T, N, dtype=torch.float32, device=x.device) if want_logits else None
        ws = None
        if logits is None:
            n = bmoe_router_workspace_bytes(dt, T, d, N, k)
            if n == 0:
                raise BmoeError(2, "bmoe_router_workspace_bytes")
            ws = torch.empty(n, dtype=torch.uint8, device=x.device)
        _check(bmoe_router(dt, T, d, N, k, x, w_router, ids, gates, logits, ws, stream),
               "bmoe_router")
        return (ids, gates, logits) if want_logits else (ids, gates)


def pack_ternary_b3(w: torch.Tensor) -> torch.Tensor:
    """int8 [d][d] in {-1,0,+1} on the GPU -> uint8 base-3 stream (raises on
    a bad entry)."""
    d = w.shape[0]
    n = bmoe_packed3_bytes(d)
    if n == 0 or w.shape != (d, d) or w.dtype != torch.int8:
        raise ValueError("w must be int8 [d][d] with a supported d")
    # 8 bytes of slack past the stream, as bmoe_product reads whole dwords
    out = torch.zeros((n + 8 + 15) // 16 * 16, dtype=torch.uint8, device=w.device)
    ws = torch.empty(bmoe_pack_workspace_bytes(), dtype=torch.uint8, device=w.device)
    _check(bmoe_pack_ternary_b3(w, d, out, ws), "bmoe_pack_ternary_b3")
    _check(bmoe_sync_status(ws), "bmoe_pack_ternary_b3 (device)")
    return out[:n]


def unpack_ternary_b3(packed3: torch.Tensor, d: int) -> torch.Tensor:
    """Base-3 stream -> the 2-bit words bmoe_forward takes (raises on a byte
    above 242)."""
    out = torch.empty(d, d // 16, dtype=torch.int32, device=packed3.device)
    ws = torch.empty(bmoe_pack_workspace_bytes(), dtype=torch.uint8, device=packed3.device)
    _check(bmoe_unpack_ternary_b3(packed3, d, out, ws), "bmoe_unpack_ternary_b3")
    _check(bmoe_sync_status(ws), "bmoe_unpack_ternary_b3 (device)")
    return out


def rotate_in(x: torch.Tensor, ids: torch.Tensor, theta: torch.Tensor) -> torch.Tensor:
    """z [T*k][d] (x's dtype), row t*k + j = B(theta_{ids[t][j]})^T x[t]."""
    T, d = x.shape
    k = ids.shape[1]
    N = theta.shape[0]
    dt = dtype_code(x)
    n = bmoe_rotate_in_workspace_bytes(dt, T, d, N, k)
    if n == 0:
        raise BmoeError(2, "bmoe_rotate_in_workspace_bytes")
    ws = torch.empty(n, dtype=torch.uint8, device=x.device)
    z = torch.empty(T * k, d, dtype=x.dtype, device=x.device)
    _check(bmoe_rotate_in(dt, T, d, N, k, x, ids, theta, z, ws), "bmoe_rotate_in")
    _check(bmoe_sync_status(ws), "bmoe_rotate_in (device)")
    return z


def quant_error(v: torch.Tensor, m: int, mode: int = 0):
    """(err, crest) fp32 [rows] for the rows of v (bf16 or fp32)."""
    rows, d = v.shape
    err = torch.empty(rows, dtype=torch.float32, device=v.device)
    crest = torch.empty(rows, dtype=torch.float32, device=v.device)
    _check(bmoe_quant_error(dtype_code(v), rows, d, v, m, mode, err, crest), "bmoe_quant_error")
    return err, crest


def forward_keep(x: torch.Tensor, ids: torch.Tensor, gates: torch.Tensor, theta: torch.Tensor,
                 phi: torch.Tensor, w_packed: torch.Tensor, alpha: float, stream=None):
    """(y, kept workspace): the forward on the unfused path, with its routing
    tables, cos/sin tables, Z and H left in the returned workspace for
    backward_kept."""
    with _on(stream):
        T, d = x.shape
        k = ids.shape[1]
        N = theta.shape[0]
        dt = dtype_code(x)
        n = bmoe_forward_keep_workspace_bytes(dt, T, d, N, k)
        if n == 0:
            raise BmoeError(2, "bmoe_forward_keep_workspace_bytes")
        ws = torch.empty(n, dtype=torch.uint8, device=x.device)
        y = torch.empty_like(x)
        _check(bmoe_forward_keep(dt, T, d, N, k, x, ids, gates, theta, phi, w_packed, alpha, y, ws,
                                 stream), "bmoe_forward_keep")
        return y, ws


def backward_kept(x: torch.Tensor, gates: torch.Tensor, n_experts: int, w_packed: torch.Tensor,
                  alpha: float, dy: torch.Tensor, kept: torch.Tensor, *, want_dw: bool = True,
                  stream=None) -> dict:
    """As backward(), reading the forward's intermediates from forward_keep's
    workspace instead of recomputing them."""
    with _on(stream):
        T, d = x.shape
        k = gates.shape[1]
        N = n_experts
        dt = dtype_code(x)
        L = int(d).bit_length() - 1
        n = bmoe_backward_workspace_bytes(dt, T, d, N, k)
        if n == 0:
            raise BmoeError(2, "bmoe_backward_workspace_bytes")
        ws = torch.empty(n, dtype=torch.uint8, device=x.device)
        out = {
            "dx": torch.empty_like(x),
            "dgates": torch.empty(T, k, dtype=torch.float32, device=x.device),
            "dtheta": torch.empty(N, L, d // 2, dtype=torch.float32, device=x.device),
            "dphi": torch.empty(N, L, d // 2, dtype=torch.float32, device=x.device),
            "dw": torch.empty(d, d, dtype=torch.float32, device=x.device) if want_dw else None,
        }
        _check(bmoe_backward_kept(dt, T, d, N, k, x, gates, w_packed, alpha, dy, out["dx"],
                                  out["dgates"], out["dtheta"], out["dphi"], out["dw"], kept, ws,
                                  stream), "bmoe_backward_kept")
        return out
