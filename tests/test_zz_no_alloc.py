"""bmoe_forward_noalloc (the forward with its workspace in the library's own
fixed device array) against bmoe_forward with a caller workspace, through the
C ABI: same kernels, so the outputs and routing tables must be identical bit
for bit, call after call, as the shapes shrink and change path."""
import numpy as np
import pytest
import torch

from butterfly_rotated_ternary_amd import bmoe
from butterfly_rotated_ternary_amd import workloads as W
from devinputs import to_device

pytestmark = pytest.mark.gpu


def _dt(inp):
    return bmoe.BMOE_BF16 if inp.dtype == "bf16" else bmoe.BMOE_F32


def _both(inp):
    """(y, route) of bmoe_forward and of bmoe_forward_noalloc on the same
    device inputs."""
    dev = to_device(inp)
    T, d, N, k = inp.T, inp.d, inp.N, inp.k
    dt = _dt(inp)
    M = T * k
    print(f"[noalloc] d={d} N={N} k={k} T={T} {inp.dtype} "
          f"ws={bmoe.bmoe_workspace_bytes(dt, T, d, N, k)}", flush=True)
    args = (dt, T, d, N, k, dev["x"], dev["ids"], dev["gates"], dev["theta"], dev["phi"],
            dev["w_packed"], dev["alpha"])
    y_ref = torch.empty_like(dev["x"])
    r_ref = torch.empty(N + 1 + 2 * M, dtype=torch.int32, device="cuda")
    ws = torch.empty(bmoe.bmoe_workspace_bytes(dt, T, d, N, k), dtype=torch.uint8, device="cuda")
    assert bmoe.bmoe_forward(*args, y_ref, ws, r_ref) == 0
    y = torch.full_like(dev["x"], float("nan"))
    r = torch.full((N + 1 + 2 * M,), -7, dtype=torch.int32, device="cuda")
    status = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    assert bmoe.bmoe_forward_noalloc(*args, y, r, status) == 0
    assert bmoe.bmoe_sync_status(status) == 0
    torch.cuda.synchronize()
    return (y_ref, r_ref), (y, r), dev


# Each pair runs back to back on the shared array: a full-size call, then a
# smaller one of the same path; then the prep-routed fused path, the split
# path, the fp32 path and the small-d path.
SEQUENCE = [
    dict(name=W.HEADLINE),                                   # routed fused, T = 4096
    dict(name=W.HEADLINE, T=1000, seed=5),                   # same path, smaller
    dict(name="d512_e256_top2_zipf_bf16", T=9000),           # prep + fused (M > 8192)
    dict(name="d512_e256_top2_zipf_bf16", T=4500, seed=9),   # same path, smaller
    dict(name="d2048_e64_top2_outliers_bf16", T=1500),       # split path
    dict(name="d2048_e64_top2_outliers_bf16", T=300, seed=3),
    dict(name="tiny_d64_e8_top2_f32"),                       # fp32
    dict(name="custom", d=8, N=5, k=2, T=700, seed=8, dtype="bf16"),  # d < 16
]


def test_noalloc_matches_forward_call_after_call():
    for case in SEQUENCE:
        case = dict(case)
        inp = W.make_inputs(case.pop("name"), **case)
        (y_ref, r_ref), (y, r), _ = _both(inp)
        assert torch.equal(r, r_ref)
        assert torch.equal(y, y_ref)


def test_noalloc_reports_bad_ids_and_oversized_shapes():
    inp = W.make_inputs(W.HEADLINE, T=300, seed=12)
    dev = to_device(inp)
    T, d, N, k = inp.T, inp.d, inp.N, inp.k
    y = torch.empty_like(dev["x"])
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dev["ids"][7, 1] = N + 3
    args = (bmoe.BMOE_BF16, T, d, N, k, dev["x"], dev["ids"], dev["gates"], dev["theta"],
            dev["phi"], dev["w_packed"], dev["alpha"], y)
    assert bmoe.bmoe_forward_noalloc(*args, None, status) == 0
    assert bmoe.bmoe_sync_status(status) == 5
    dev["ids"][7, 1] = 0
    assert bmoe.bmoe_forward_noalloc(*args, None, status) == 0
    assert bmoe.bmoe_sync_status(status) == 0
    # d = 2048, T = 16384 needs Z, H and U of 64 MiB each: refused up front
    big = (bmoe.BMOE_BF16, 16384, 2048, 64, 2)
    assert bmoe.bmoe_workspace_bytes(*big) > bmoe.BMOE_NOALLOC_MAX_WORKSPACE
    assert bmoe.bmoe_forward_noalloc(*big, dev["x"], dev["ids"], dev["gates"], dev["theta"],
                                     dev["phi"], dev["w_packed"], 1.0, y) == 6
