#!/usr/bin/env python3
"""Throughput of the ButterflyMoE expert-layer forward on one MI355X.

One step = one bmoe_forward over the whole batch (routing, butterfly-in,
shared ternary product, butterfly-out, gate-weighted combine) with the inputs
already resident in HBM. Prints one JSON line on stdout.

    python bench.py [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed tokens/sec of ButterflyMoE layer fwd (d=512,N=64,top-2); % MFMA/HBM peak"

# MI355X published peaks
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles (the library records them on its own stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def kernel_work(name, dt_bytes, T, d, N, k):
    """Algorithmic work of one launch of each forward kernel:
    (bound, amount, unit) with bytes for HBM-bound kernels and flops for the
    contraction. Counts only what the kernel must read and write once."""
    M = T * k
    L = d.bit_length() - 1
    A = N * L * (d // 2)             # angles per side
    xb = dt_bytes
    zb = dt_bytes                    # Z stored in the activation type
    if name.startswith("prep"):
        return "hbm", M * 4 + 2 * A * 4 + 2 * A * 8 + 3 * M * 4 + (N + 1) * 4, "B"
    if name.startswith("bfly_in"):
        return "hbm", M * d * xb + M * d * zb + A * 8 + 2 * M * 4, "B"
    if name.startswith("gemm"):
        return "mfma", 2 * M * d * d, "flop"
    if name.startswith("bfly_out"):
        return "hbm", M * d * 4 + M * d * 4 + A * 8 + 3 * M * 4, "B"
    if name.startswith("combine"):
        return "hbm", M * d * 4 + T * d * xb, "B"
    raise KeyError(name)


def min_hbm_bytes(dt_bytes, T, d, N, k):
    """Bytes any forward must move: x, y, the packed substrate, both angle
    sets, ids and gates."""
    L = d.bit_length() - 1
    return 2 * T * d * dt_bytes + d * d // 4 + 2 * N * L * (d // 2) * 4 + 2 * T * k * 4


def cpu_baseline(inp, seconds):
    """The fp64 oracle, as it stands, on a bounded sample of the workload."""
    import numpy as np
    from threadpoolctl import threadpool_info
    import oracle as O

    def run(nt):
        t0 = time.perf_counter()
        O.forward(inp.x[:nt], inp.ids[:nt], inp.gates[:nt], inp.theta, inp.phi, inp.w, inp.alpha)
        return time.perf_counter() - t0

    probe_t = min(inp.T, 256)
    dt = run(probe_t)
    per_tok = dt / probe_t
    nt = int(min(inp.T, max(probe_t, seconds / max(per_tok, 1e-9))))
    reps, total = 0, 0.0
    while total < seconds and reps < 100:
        total += run(nt)
        reps += 1
        if nt < inp.T:
            break
    threads = [i.get("num_threads", 1) for i in threadpool_info()]
    cores = max(threads) if threads else 1
    return {
        "value": nt * reps / total,
        "unit": "tokens/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"first {nt} of {inp.T} tokens x {reps} run(s), {total:.1f} s; numpy fp64 "
                  f"(BLAS threads {cores}; rotations single-threaded)",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()
    if args.gpus != 1:
        log("bench.py measures one GPU only: the forward shards by tokens with no exchange, "
            "so a multi-GPU figure is not produced. Run with --gpus 1.")
        sys.exit(2)

    import numpy as np
    import torch
    from butterfly_rotated_ternary_amd import bmoe
    from butterfly_rotated_ternary_amd import workloads as W

    name = args.workload or W.HEADLINE
    inp = W.make_inputs(name)
    T, d, N, k = inp.T, inp.d, inp.N, inp.k
    dev = torch.device("cuda:0")
    if inp.dtype == "bf16":
        x = torch.from_numpy(inp.x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        dt, dt_bytes = bmoe.BMOE_BF16, 2
    else:
        x = torch.from_numpy(inp.x).to(dev)
        dt, dt_bytes = bmoe.BMOE_F32, 4
    ids = torch.from_numpy(inp.ids).to(dev)
    gates = torch.from_numpy(inp.gates).to(dev)
    theta = torch.from_numpy(inp.theta).to(dev)
    phi = torch.from_numpy(inp.phi).to(dev)
    wp = bmoe.pack_ternary(torch.from_numpy(inp.w).to(dev))
    alpha = float(inp.alpha)
    ws = bmoe.Workspace(dt, T, d, N, k, device=dev)
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()

    def step():
        rc = bmoe.bmoe_forward(dt, T, d, N, k, x, ids, gates, theta, phi, wp, alpha, y, ws.buf,
                               None, stream)
        if rc != 0:
            raise bmoe.BmoeError(rc, "bmoe_forward")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if bmoe.bmoe_sync_status(ws.buf) != 0:
        raise RuntimeError("device status not OK")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    value = T / (ms * 1e-3)
    log(f"[bench] {name}: {ms * 1e3:.2f} us/step, {value:.4g} tokens/s")

    # Per-kernel durations, HIP events on the library's stream, same workload.
    nk = bmoe.bmoe_forward_kernel_count(dt, T, d, N, k)
    names = [bmoe.bmoe_forward_kernel_name(dt, T, d, N, k, i) for i in range(nk)]
    hip = HipEvents()
    n_ev_steps = min(args.steps, 200)
    evsets = [hip.create(nk + 1) for _ in range(n_ev_steps)]
    torch.cuda.synchronize()
    for evs in evsets:
        rc = bmoe.bmoe_forward_timed(dt, T, d, N, k, x, ids, gates, theta, phi, wp, alpha, y,
                                     ws.buf, None, stream, evs)
        if rc != 0:
            raise bmoe.BmoeError(rc, "bmoe_forward_timed")
    torch.cuda.synchronize()
    per_kernel = {n: 0.0 for n in names}
    for evs in evsets:
        for i, n in enumerate(names):
            per_kernel[n] += hip.elapsed_ms(evs[i], evs[i + 1]) / n_ev_steps
    for evs in evsets:
        hip.destroy(evs)
    log("[bench] per-kernel ms (events): " + ", ".join(f"{n}={v * 1e3:.2f}us"
                                                        for n, v in per_kernel.items()))

    dom = max(per_kernel, key=per_kernel.get)
    bound, amount, unit = kernel_work(dom, dt_bytes, T, d, N, k)
    dur_s = per_kernel[dom] * 1e-3
    if bound == "mfma":
        peak = PEAK_BF16_TFLOPS if dt == bmoe.BMOE_BF16 else PEAK_FP32_TFLOPS
        achieved = amount / dur_s / 1e12
        runit = "TFLOP/s"
    else:
        peak = PEAK_HBM_GBS
        achieved = amount / dur_s / 1e9
        runit = "GB/s"
    roofline = {"bound": bound, "achieved": achieved, "peak": peak, "unit": runit,
                "frac": achieved / peak, "traffic": None, "kernel": dom,
                "work_per_launch": amount, "work_unit": unit}

    M = T * k
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dt == bmoe.BMOE_BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": name, "d": d, "n_experts": N, "top_k": k, "tokens": T,
                   "routed_rows": M},
        "roofline": roofline,
        "routed_rows_per_s": M / (ms * 1e-3),
        "e2e_frac": {"mfma_bf16": 2 * M * d * d / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
                     "hbm": min_hbm_bytes(dt_bytes, T, d, N, k) / (ms * 1e-3) / (PEAK_HBM_GBS * 1e9)},
        "kernels_us": {n: v * 1e3 for n, v in per_kernel.items()},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
        log(f"[bench] cpu baseline {out['cpu_baseline']['value']:.4g} tokens/s "
            f"({out['cpu_baseline']['sample']})")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
