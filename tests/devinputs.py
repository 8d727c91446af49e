"""Move a seeded workload onto the GPU for the library (test helper)."""
import numpy as np
import torch

from butterfly_rotated_ternary_amd import bmoe


def to_device(inp, device="cuda"):
    if inp.dtype == "bf16":
        x = torch.from_numpy(inp.x_bits.view(np.int16)).view(torch.bfloat16).to(device)
    else:
        x = torch.from_numpy(inp.x).to(device)
    w8 = torch.from_numpy(inp.w).to(device)
    return dict(
        x=x,
        ids=torch.from_numpy(inp.ids).to(device),
        gates=torch.from_numpy(inp.gates).to(device),
        theta=torch.from_numpy(inp.theta).to(device),
        phi=torch.from_numpy(inp.phi).to(device),
        w8=w8,
        w_packed=bmoe.pack_ternary(w8),
        alpha=float(inp.alpha),
    )


def run_forward(dev, inp, with_route=True):
    T, d, N, k = inp.T, inp.d, inp.N, inp.k
    route = None
    if with_route:
        route = torch.empty(N + 1 + 2 * T * k, dtype=torch.int32, device=dev["x"].device)
    y = bmoe.forward(dev["x"], dev["ids"], dev["gates"], dev["theta"], dev["phi"], dev["w_packed"],
                     dev["alpha"], route_out=route)
    torch.cuda.synchronize()
    yh = y.float().cpu().numpy().astype(np.float64)
    if not with_route:
        return yh, None
    r = route.cpu().numpy()
    M = T * k
    return yh, (r[:N + 1], r[N + 1:N + 1 + M], r[N + 1 + M:])
