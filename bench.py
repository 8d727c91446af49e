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
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed tokens/sec of ButterflyMoE layer fwd (d=512,N=64,top-2); % MFMA/HBM peak"

# MI355X published peaks
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0        # dense bf16 MFMA
PEAK_FP32_MFMA_TFLOPS = 157.3    # dense fp32 MFMA
# fp32 vector: 256 CU x 4 SIMD x 32 lanes x 2 flop (FMA) x 2.4 GHz. A plain
# stream of non-packed v_fma_f32 (bench.py ceilings) reaches about 119
# TFLOP/s on the box, above the 78.6 a 16-lane SIMD would allow, so the
# published figure is the ceiling for the non-packed code built here too.
PEAK_VALU_F32_TFLOPS = 256 * 4 * 32 * 2 * 2.4e9 / 1e12

GEMM_WORKLOAD = "d4096_e256_top4_bf16"
SHARD_TOKENS = 4096


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


def kernel_work(name, act_bytes, T, d, N, k, routed=False, trig=None):
    """Algorithmic work of one launch of a forward kernel: the bytes it must
    move to or from HBM (each input read once, each output written once), the
    flops of its dense contraction (MFMA) and the flops of its rotations
    (fp32 VALU: 2 multiplies and 2 fused multiply-adds, 6 flops, per pair and
    stage). act_bytes is the size of one activation element (x, Z, H, U, y).
    routed: the fused kernel routes itself (no prep launch): it reads the ids,
    both angle sets and the packed substrate, and writes the routing tables.
    trig: prep writes the cos/sin tables (default: unless the fused kernel
    runs after it, which evaluates its own tiles' tables from the angles)."""
    M = T * k
    L = d.bit_length() - 1
    A = N * L * (d // 2)                     # angles (pairs) per side
    rot = M * L * (d // 2) * 6               # flops of one rotation side
    routing = M * 4                          # one int32 per routed row
    if name.startswith("prep"):
        fused = act_bytes == 2 and d in (256, 512)
        b = M * 4 + 3 * routing + (N + 1) * 4          # ids in; perm, inv, slot_e out
        if trig if trig is not None else not fused:
            b += 2 * A * 4 + 2 * A * 8               # angles in, cos/sin tables out
        if act_bytes == 2 and d % 512 == 0 and -(-M // 128) * (d // 512) >= 512:
            b += 2 * (d * d // 4)                    # tile-major copy of the packed substrate
        return {"bytes": b, "mfma_flops": 0, "valu_flops": 0}
    if name.startswith("fused") and routed:
        b = (T * d * act_bytes + M * d * act_bytes + d * d // 4 + 2 * A * 4
             + 5 * routing + (N + 1) * 4)     # ids and gates in; perm, inv, slot_e out
        return {"bytes": b, "mfma_flops": 2 * M * d * d, "valu_flops": 2 * rot}
    if name.startswith("fused"):             # after prep: perm and slot_e in
        b = (T * d * act_bytes + M * d * act_bytes + d * d // 4 + 2 * A * 4
             + 3 * routing)                  # perm, slot_e, gates
        return {"bytes": b, "mfma_flops": 2 * M * d * d, "valu_flops": 2 * rot}
    if name.startswith("bfly_in"):
        b = T * d * act_bytes + M * d * act_bytes + A * 8 + 2 * routing
        return {"bytes": b, "mfma_flops": 0, "valu_flops": rot}
    if name.startswith("gemm"):
        b = 2 * M * d * act_bytes + d * d // 4
        return {"bytes": b, "mfma_flops": 2 * M * d * d, "valu_flops": 0}
    if name.startswith("bfly_out"):
        b = 2 * M * d * act_bytes + A * 8 + 2 * routing + M * 4
        return {"bytes": b, "mfma_flops": 0, "valu_flops": rot}
    if name.startswith("combine"):
        return {"bytes": M * d * act_bytes + T * d * act_bytes, "mfma_flops": 0, "valu_flops": 0}
    raise KeyError(name)


def backward_work(name, act_bytes, T, d, N, k):
    """Algorithmic work of one launch of the backward (same conventions as
    kernel_work). A butterfly-backward stage costs 22 flops per pair and row:
    6 to recompute the forward rotation, 6 each to invert it on the values and
    on the gradients, 4 for the angle gradient and its sum."""
    M = T * k
    L = d.bit_length() - 1
    A = N * L * (d // 2)
    tile_rows = 64 if d >= 1024 else 16 if d in (256, 512) else 32
    tiles = -(-M // tile_rows) + N           # upper bound on expert-aligned row tiles
    partial = tiles * L * (d // 2) * 4
    routing = M * 4
    if name == "prep_kernel":               # the forward's prep + tile list and packed W_base^T
        w = kernel_work(name, act_bytes, T, d, N, k, trig=True)
        w["bytes"] += d * d // 4 * (3 if d % 512 == 0 else 2) + (N + 1) * 4 * 2 + tiles * 16
        return w
    if name in ("bfly_in_kernel", "gemm_kernel", "combine_kernel"):
        return kernel_work(name, act_bytes, T, d, N, k)
    if name == "fused_wave_kernel":         # d = 256, 512: Z and H recomputed in one launch
        b = T * d * act_bytes + 2 * M * d * act_bytes + d * d // 4 + A * 4 + 2 * routing
        return {"bytes": b, "mfma_flops": 2 * M * d * d, "valu_flops": M * L * (d // 2) * 6}
    if name == "gemm_t_kernel":
        return kernel_work("gemm_kernel", act_bytes, T, d, N, k)
    if name == "dw_kernel":
        return {"bytes": 2 * M * d * act_bytes + d * d * 4, "mfma_flops": 2 * M * d * d,
                "valu_flops": 0}
    if name in ("bfly_bwd_out_kernel", "bfly_bwd_in_kernel"):
        b = (2 * M * d + T * d) * act_bytes + A * 8 + routing + partial
        if name == "bfly_bwd_out_kernel":
            b += 2 * M * 4                   # gates in, dgates out
        return {"bytes": b, "mfma_flops": 0, "valu_flops": M * L * (d // 2) * 22}
    if name == "finish_kernel":             # dx combine, both angle sums, dW slices
        slices = dw_slices(M, d)
        b = (M + T) * d * act_bytes + 2 * (partial + A * 4)
        if slices > 1:
            b += (slices + 1) * d * d * 4
        return {"bytes": b, "mfma_flops": 0, "valu_flops": 0}
    raise KeyError(name)


def dw_slices(M, d):
    """Row-range slices of the bf16 substrate gradient the closing kernel sums
    (the library's split rule for d = 128 .. 1024; 0 or 1: no sum)."""
    if d < 128 or d > 1024:
        return 0
    tiles = (d // 128) ** 2
    S = min(-(-256 // tiles), M // 512)
    return max(S, 1)


def router_work(name, act_bytes, T, d, N, k):
    """Algorithmic work of one router launch: the logits product reads x and
    the router weights once and writes fp32 logits (2 T d N flops, MFMA on
    bf16, VALU on fp32); the top-k reads the logits and writes ids and gates."""
    if name == "router_logits_kernel":
        b = T * d * act_bytes + N * d * act_bytes + T * N * 4
        f = 2 * T * d * N
        if act_bytes == 2:
            return {"bytes": b, "mfma_flops": f, "valu_flops": 0}
        return {"bytes": b, "mfma_flops": 0, "valu_flops": f}
    if name == "topk_kernel":
        return {"bytes": T * N * 4 + T * k * 8, "mfma_flops": 0, "valu_flops": 0}
    raise KeyError(name)


def roofline(work, dur_s, mfma_peak_tflops):
    """The roofline of one kernel: the resource whose ideal time (work over
    published peak) is largest bounds it; achieved = that work / measured
    duration. frac_by_resource gives each resource's ideal time over the
    measured duration."""
    t_hbm = work["bytes"] / (PEAK_HBM_GBS * 1e9)
    t_mfma = work["mfma_flops"] / (mfma_peak_tflops * 1e12)
    t_alu = work["valu_flops"] / (PEAK_VALU_F32_TFLOPS * 1e12)
    bound = max((t_hbm, "hbm"), (t_mfma, "mfma"), (t_alu, "alu"))[1]
    if bound == "hbm":
        ach, peak, unit, amount = work["bytes"] / dur_s / 1e9, PEAK_HBM_GBS, "GB/s", work["bytes"]
    elif bound == "mfma":
        ach, peak, unit = work["mfma_flops"] / dur_s / 1e12, mfma_peak_tflops, "TFLOP/s"
        amount = work["mfma_flops"]
    else:
        ach, peak, unit = work["valu_flops"] / dur_s / 1e12, PEAK_VALU_F32_TFLOPS, "TFLOP/s"
        amount = work["valu_flops"]
    return {"bound": bound, "achieved": ach, "peak": peak, "unit": unit, "frac": ach / peak,
            "work_per_launch": amount, "duration_us": dur_s * 1e6,
            "ideal_us": {"hbm": t_hbm * 1e6, "mfma": t_mfma * 1e6, "alu": t_alu * 1e6},
            "frac_by_resource": {"hbm": t_hbm / dur_s, "mfma": t_mfma / dur_s,
                                 "alu": t_alu / dur_s}}


def min_hbm_bytes(act_bytes, T, d, N, k):
    """Bytes any forward must move: x, y, the packed substrate, both angle
    sets, ids and gates."""
    L = d.bit_length() - 1
    return 2 * T * d * act_bytes + d * d // 4 + 2 * N * L * (d // 2) * 4 + 2 * T * k * 4


def source_digest():
    """sha256 over the kernel sources and the C header: a stored counter
    figure is only valid for the sources it was taken from."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "butterfly_rotated_ternary_amd", "csrc", "*")))
    files += sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(kernel, workload):
    """HBM bytes per launch from the counter summary of this kernel and
    workload under profiles/ (FETCH_SIZE + WRITE_SIZE, scaled by a copy-kernel
    calibration), or None if absent or taken from other sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}.traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith((" ", "#", "$")):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("source_sha256") != source_digest():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


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


class Problem:
    """Device-resident inputs of one workload, ready for bmoe_forward."""

    def __init__(self, name, T=None):
        import numpy as np
        import torch
        from butterfly_rotated_ternary_amd import bmoe
        from butterfly_rotated_ternary_amd import workloads as W

        self.name = name
        self.inp = inp = W.make_inputs(name, T=T)
        self.T, self.d, self.N, self.k = inp.T, inp.d, inp.N, inp.k
        dev = torch.device("cuda:0")
        if inp.dtype == "bf16":
            self.x = torch.from_numpy(inp.x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
            self.dt, self.act_bytes = bmoe.BMOE_BF16, 2
        else:
            self.x = torch.from_numpy(inp.x).to(dev)
            self.dt, self.act_bytes = bmoe.BMOE_F32, 4
        self.ids = torch.from_numpy(inp.ids).to(dev)
        self.gates = torch.from_numpy(inp.gates).to(dev)
        self.theta = torch.from_numpy(inp.theta).to(dev)
        self.phi = torch.from_numpy(inp.phi).to(dev)
        self.wp = bmoe.pack_ternary(torch.from_numpy(inp.w).to(dev))
        self.alpha = float(inp.alpha)
        self.ws = bmoe.Workspace(self.dt, self.T, self.d, self.N, self.k, device=dev)
        self.y = torch.empty_like(self.x)
        self.stream = torch.cuda.current_stream()
        self.bmoe = bmoe

    def args(self):
        return (self.dt, self.T, self.d, self.N, self.k, self.x, self.ids, self.gates, self.theta,
                self.phi, self.wp, self.alpha, self.y, self.ws.buf, None, self.stream)

    def step(self):
        rc = self.bmoe.bmoe_forward(*self.args())
        if rc != 0:
            raise self.bmoe.BmoeError(rc, "bmoe_forward")

    def kernel_names(self):
        b = self.bmoe
        nk = b.bmoe_forward_kernel_count(self.dt, self.T, self.d, self.N, self.k)
        return [b.bmoe_forward_kernel_name(self.dt, self.T, self.d, self.N, self.k, i)
                for i in range(nk)]

    def time_steps(self, steps, warmup):
        """Wall time per step over `steps` back-to-back forwards (ms)."""
        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        if self.bmoe.bmoe_sync_status(self.ws.buf) != 0:
            raise RuntimeError("device status not OK")
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    def time_kernels(self, steps):
        """Average execution time of each kernel (ms), from the start/stop
        events its own dispatch records, over `steps` forwards."""
        import torch
        names = self.kernel_names()
        hip = HipEvents()
        evsets = [hip.create(2 * len(names)) for _ in range(steps)]
        torch.cuda.synchronize()
        for evs in evsets:
            rc = self.bmoe.bmoe_forward_timed(*self.args(), evs)
            if rc != 0:
                raise self.bmoe.BmoeError(rc, "bmoe_forward_timed")
        torch.cuda.synchronize()
        per = {n: 0.0 for n in names}
        for evs in evsets:
            for i, n in enumerate(names):
                per[n] += hip.elapsed_ms(evs[2 * i], evs[2 * i + 1]) / steps
        for evs in evsets:
            hip.destroy(evs)
        return per

    def backward_setup(self):
        import numpy as np
        import torch
        rng = np.random.default_rng(5)
        dy = torch.from_numpy(rng.standard_normal((self.T, self.d)).astype(np.float32))
        self.dy = dy.to(self.x.device).to(self.x.dtype)
        b = self.bmoe
        n = b.bmoe_backward_workspace_bytes(self.dt, self.T, self.d, self.N, self.k)
        if n == 0:
            raise ValueError(f"backward does not support {self.name}")
        self.bws = torch.empty(n, dtype=torch.uint8, device=self.x.device)
        self.g = {"dx": torch.empty_like(self.x),
                  "dgates": torch.empty_like(self.gates),
                  "dtheta": torch.empty_like(self.theta),
                  "dphi": torch.empty_like(self.phi),
                  "dw": torch.empty(self.d, self.d, dtype=torch.float32, device=self.x.device)}

    def backward_args(self):
        g = self.g
        return (self.dt, self.T, self.d, self.N, self.k, self.x, self.ids, self.gates, self.theta,
                self.phi, self.wp, self.alpha, self.dy, g["dx"], g["dgates"], g["dtheta"],
                g["dphi"], g["dw"], self.bws, self.stream)

    def time_backward(self, steps, warmup):
        """Wall time per backward over `steps` back-to-back calls (ms), then
        each launch's average time from its own events (ms)."""
        import torch
        b = self.bmoe
        for _ in range(warmup):
            rc = b.bmoe_backward(*self.backward_args())
            if rc != 0:
                raise b.BmoeError(rc, "bmoe_backward")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            b.bmoe_backward(*self.backward_args())
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        nk = b.bmoe_backward_kernel_count(self.dt, self.T, self.d, self.N, self.k)
        names = [b.bmoe_backward_kernel_name(self.dt, self.T, self.d, self.N, self.k, i)
                 for i in range(nk)]
        hip = HipEvents()
        evsets = [hip.create(2 * nk) for _ in range(steps)]
        for evs in evsets:
            rc = b.bmoe_backward_timed(*self.backward_args(), events=evs)
            if rc != 0:
                raise b.BmoeError(rc, "bmoe_backward_timed")
        torch.cuda.synchronize()
        per = {n: 0.0 for n in names}
        for evs in evsets:
            for i, n in enumerate(names):
                per[n] += hip.elapsed_ms(evs[2 * i], evs[2 * i + 1]) / steps
        for evs in evsets:
            hip.destroy(evs)
        return ms, per

    def router_setup(self):
        import numpy as np
        import torch
        from butterfly_rotated_ternary_amd import workloads as W
        rw = W.make_router_weights(self.inp)
        if self.act_bytes == 2:
            self.wr = torch.from_numpy(rw.w_bits.view(np.int16)).view(torch.bfloat16).to(
                self.x.device)
        else:
            self.wr = torch.from_numpy(rw.w).to(self.x.device)
        b = self.bmoe
        self.r_ids = torch.empty_like(self.ids)
        self.r_gates = torch.empty_like(self.gates)
        n = b.bmoe_router_workspace_bytes(self.dt, self.T, self.d, self.N, self.k)
        self.rws = torch.empty(n, dtype=torch.uint8, device=self.x.device)

    def router_args(self):
        return (self.dt, self.T, self.d, self.N, self.k, self.x, self.wr, self.r_ids,
                self.r_gates, None, self.rws, self.stream)

    def time_router(self, steps, warmup):
        """(router ms, router + forward ms per step, per-launch router ms)."""
        import torch
        b = self.bmoe
        fwd = (self.dt, self.T, self.d, self.N, self.k, self.x, self.r_ids, self.r_gates,
               self.theta, self.phi, self.wp, self.alpha, self.y, self.ws.buf, None, self.stream)
        for _ in range(warmup):
            rc = b.bmoe_router(*self.router_args())
            if rc != 0:
                raise b.BmoeError(rc, "bmoe_router")
            rc = b.bmoe_forward(*fwd)
            if rc != 0:
                raise b.BmoeError(rc, "bmoe_forward")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            b.bmoe_router(*self.router_args())
        torch.cuda.synchronize()
        r_ms = (time.perf_counter() - t0) * 1e3 / steps
        t0 = time.perf_counter()
        for _ in range(steps):
            b.bmoe_router(*self.router_args())
            b.bmoe_forward(*fwd)
        torch.cuda.synchronize()
        rf_ms = (time.perf_counter() - t0) * 1e3 / steps
        if b.bmoe_sync_status(self.ws.buf) != 0:
            raise RuntimeError("device status not OK after routed forwards")
        names = ["router_logits_kernel", "topk_kernel"]
        hip = HipEvents()
        evsets = [hip.create(4) for _ in range(steps)]
        for evs in evsets:
            rc = b.bmoe_router_timed(*self.router_args(), events=evs)
            if rc != 0:
                raise b.BmoeError(rc, "bmoe_router_timed")
        torch.cuda.synchronize()
        per = {n: 0.0 for n in names}
        for evs in evsets:
            for i, n in enumerate(names):
                per[n] += hip.elapsed_ms(evs[2 * i], evs[2 * i + 1]) / steps
        for evs in evsets:
            hip.destroy(evs)
        return r_ms, rf_ms, per

    def time_training_step(self, steps, warmup):
        """Per-step ms of forward + backward (the backward recomputes the
        forward) and of keep-forward + kept backward, and of the kept
        backward alone."""
        import torch
        b = self.bmoe
        kept = torch.empty(b.bmoe_forward_keep_workspace_bytes(self.dt, self.T, self.d, self.N,
                                                               self.k),
                           dtype=torch.uint8, device=self.x.device)
        g = self.g
        fwd_keep = (self.dt, self.T, self.d, self.N, self.k, self.x, self.ids, self.gates,
                    self.theta, self.phi, self.wp, self.alpha, self.y, kept, self.stream)
        bwd_kept = (self.dt, self.T, self.d, self.N, self.k, self.x, self.gates, self.wp,
                    self.alpha, self.dy, g["dx"], g["dgates"], g["dtheta"], g["dphi"], g["dw"],
                    kept, self.bws, self.stream)

        def run(fn, n):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(n):
                fn()
            torch.cuda.synchronize()
            return (time.perf_counter() - t0) * 1e3 / n

        def recompute():
            if b.bmoe_forward(*self.args()) != 0 or b.bmoe_backward(*self.backward_args()) != 0:
                raise RuntimeError("forward/backward failed")

        def kept_step():
            if b.bmoe_forward_keep(*fwd_keep) != 0 or b.bmoe_backward_kept(*bwd_kept) != 0:
                raise RuntimeError("kept forward/backward failed")

        def kept_bwd():
            if b.bmoe_backward_kept(*bwd_kept) != 0:
                raise RuntimeError("kept backward failed")

        out = {"recompute_ms": run(recompute, steps), "kept_ms": run(kept_step, steps)}
        out["kept_backward_ms"] = run(kept_bwd, steps)
        del kept
        return out

    def mfma_peak(self):
        return PEAK_BF16_TFLOPS if self.dt == self.bmoe.BMOE_BF16 else PEAK_FP32_MFMA_TFLOPS


def backward_section(P, steps):
    """The backward (all gradients, forward recomputed inside) on the same
    workload: tokens/s and the roofline of its longest launch."""
    P.backward_setup()
    ms, per = P.time_backward(steps, max(3, steps // 10))
    T, d, N, k = P.T, P.d, P.N, P.k
    dom = max(per, key=per.get)
    roof = roofline(backward_work(dom, P.act_bytes, T, d, N, k), per[dom] * 1e-3, P.mfma_peak())
    roof["traffic"] = stored_traffic(dom, P.name)
    roof["kernel"] = dom
    kern = {}
    for n, v in per.items():
        r = roofline(backward_work(n, P.act_bytes, T, d, N, k), v * 1e-3, P.mfma_peak())
        kern[n] = {"us": v * 1e3, "bound": r["bound"], "frac": r["frac"]}
    log(f"[bench] backward {P.name}: {ms * 1e3:.1f} us/step; "
        + ", ".join(f"{n}={v * 1e3:.1f}" for n, v in per.items()))
    train = P.time_training_step(steps, max(3, steps // 10))
    log(f"[bench] training step {P.name}: forward + backward {train['recompute_ms'] * 1e3:.1f} us; "
        f"keep-forward + kept backward {train['kept_ms'] * 1e3:.1f} us "
        f"(kept backward alone {train['kept_backward_ms'] * 1e3:.1f} us)")
    return {"workload": P.name, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
            "steps": steps, "roofline": roof, "kernels": kern, "training_step": train}


def router_section(P, steps):
    """The router on the same workload (synthetic router weights), alone and
    followed by the forward on its ids and gates."""
    P.router_setup()
    r_ms, rf_ms, per = P.time_router(steps, max(3, steps // 10))
    T, d, N, k = P.T, P.d, P.N, P.k
    kern = {}
    for n, v in per.items():
        r = roofline(router_work(n, P.act_bytes, T, d, N, k), v * 1e-3, P.mfma_peak())
        kern[n] = {"us": v * 1e3, "bound": r["bound"], "frac": r["frac"],
                   "achieved": r["achieved"], "unit": r["unit"]}
    log(f"[bench] router {P.name}: {r_ms * 1e3:.1f} us; router + forward {rf_ms * 1e3:.1f} us; "
        + ", ".join(f"{n}={v * 1e3:.1f}" for n, v in per.items()))
    return {"workload": P.name, "ms_per_step": r_ms, "routed_forward_ms_per_step": rf_ms,
            "routed_forward_tokens_per_s": T / (rf_ms * 1e-3), "steps": steps, "kernels": kern}


def base3_section(P, steps, fwd_ms):
    """Base-3 storage of the substrate (five ternary digits per byte): bytes at
    rest, and the kernel that decodes it into the 2-bit words the forward
    reads (HBM-bound: d*d/5 bytes read, d*d/4 written)."""
    import torch
    b, d = P.bmoe, P.d
    w8 = torch.from_numpy(P.inp.w).to(P.x.device)
    p3 = b.pack_ternary_b3(w8)
    out = torch.empty(d, d // 16, dtype=torch.int32, device=P.x.device)
    ws = torch.empty(b.bmoe_pack_workspace_bytes(), dtype=torch.uint8, device=P.x.device)
    hip = HipEvents()
    evsets = [hip.create(2) for _ in range(steps)]
    for evs in [hip.create(2) for _ in range(3)] + evsets:
        rc = b.bmoe_unpack_ternary_b3_timed(p3, d, out, ws, events=evs)
        if rc != 0:
            raise b.BmoeError(rc, "bmoe_unpack_ternary_b3")
    torch.cuda.synchronize()
    if b.bmoe_sync_status(ws) != 0 or not torch.equal(out.reshape(-1), P.wp.reshape(-1)):
        raise RuntimeError("base-3 decoding differs from the 2-bit pack")
    us = sum(hip.elapsed_ms(e[0], e[1]) for e in evsets) / steps * 1e3
    nbytes = p3.numel() + d * d // 4
    log(f"[bench] base-3 d={d}: {p3.numel()} B at rest vs {d * d // 4} B (2-bit); "
        f"decode {us:.2f} us ({nbytes / us / 1e3:.0f} GB/s)")
    return {"d": d, "bytes_base3": p3.numel(), "bytes_2bit": d * d // 4,
            "bits_per_weight": 8 * p3.numel() / (d * d), "decode_us": us,
            "decode_gbs": nbytes / us / 1e3, "decode_frac_of_forward": us * 1e-3 / fwd_ms}


def product_formats_section(steps=20):
    """The shared-substrate product alone (bmoe_product) with the substrate
    as 2-bit words and as the base-3 stream decoded inside the product's
    substrate staging, same kernel otherwise: median kernel time of `steps`
    launches from its own dispatch events, on random bf16 Z of the d = 512
    (M = 8192) and d = 4096 (M = 131072) workloads' routed-row counts."""
    import torch
    from butterfly_rotated_ternary_amd import bmoe
    from butterfly_rotated_ternary_amd import workloads as W
    hip = HipEvents()
    dev = torch.device("cuda:0")
    out = []
    for wname in (W.HEADLINE, GEMM_WORKLOAD):
        inp = W.make_inputs(wname, T=1)
        full = W.WORKLOADS[wname]
        M, d = full["T"] * full["k"], inp.d
        w8 = torch.from_numpy(inp.w).to(dev)
        fmts = {"2bit": bmoe.pack_ternary(w8), "base3": bmoe.pack_ternary_b3(w8)}
        gen = torch.Generator(device=dev)
        gen.manual_seed(11)
        z = torch.randn(M, d, device=dev, generator=gen).to(torch.bfloat16)
        h = torch.empty_like(z)
        res = {"d": d, "M": M}
        for name, w in fmts.items():
            code = bmoe.BMOE_W_2BIT if name == "2bit" else bmoe.BMOE_W_BASE3
            evsets = [hip.create(2) for _ in range(steps + 2)]
            for evs in evsets:
                rc = bmoe.bmoe_product(M, d, z, w, code, float(inp.alpha), h, events=evs)
                if rc != 0:
                    raise bmoe.BmoeError(rc, "bmoe_product")
            torch.cuda.synchronize()
            ms = sorted(hip.elapsed_ms(e[0], e[1]) for e in evsets[2:])
            for evs in evsets:
                hip.destroy(evs)
            us = ms[len(ms) // 2] * 1e3
            res[name] = {"us": us, "tflops": 2.0 * M * d * d / (us * 1e-6) / 1e12,
                         "substrate_bytes": int(w.numel() * w.element_size())}
        res["base3_over_2bit"] = res["base3"]["us"] / res["2bit"]["us"]
        log(f"[bench] product d={d} M={M}: 2-bit {res['2bit']['us']:.1f} us "
            f"({res['2bit']['tflops']:.0f} TFLOP/s), base-3 {res['base3']['us']:.1f} us "
            f"({res['base3']['tflops']:.0f} TFLOP/s)")
        out.append(res)
        del z, h, fmts, w8
        torch.cuda.empty_cache()
    return out


OUTLIER_WORKLOAD = "d2048_e64_top2_outliers_bf16"
QUANTISERS = [("int8_absmax", 127, 0), ("int4_absmax", 7, 0), ("ternary_absmax", 1, 0),
              ("ternary_absmean", 1, 1)]


def workloads_section(steps, skip):
    """Forward step time and per-kernel times of the other workloads (the
    headline and the d = 4096 workload have sections of their own)."""
    import torch
    from butterfly_rotated_ternary_amd import workloads as W
    res = {}
    for wname in W.WORKLOADS:
        if wname in skip:
            continue
        P = Problem(wname)
        ms = P.time_steps(steps, 5)
        per = P.time_kernels(min(steps, 50))
        res[wname] = {"tokens": P.T, "ms_per_step": ms, "tokens_per_s": P.T / (ms * 1e-3),
                      "kernels_us": {n: v * 1e3 for n, v in per.items()}}
        log(f"[bench] {wname}: {ms * 1e3:.1f} us/step, {P.T / (ms * 1e-3):.4g} tokens/s; "
            + ", ".join(f"{n}={v * 1e3:.1f}" for n, v in per.items()))
        del P
        torch.cuda.empty_cache()
    return res


def outliers_section():
    """Outlier spreading on the workload with outlier channels: per-token
    quantisation error and crest factor of x and of z = B(theta_e)^T x (the
    workload's random angles), each averaged over rows."""
    import numpy as np
    import torch
    from butterfly_rotated_ternary_amd import bmoe
    from butterfly_rotated_ternary_amd import workloads as W
    inp = W.make_inputs(OUTLIER_WORKLOAD)
    dev = torch.device("cuda:0")
    x = torch.from_numpy(inp.x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    ids = torch.from_numpy(inp.ids).to(dev)
    theta = torch.from_numpy(inp.theta).to(dev)
    z = bmoe.rotate_in(x, ids, theta)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        z = bmoe.rotate_in(x, ids, theta)
    torch.cuda.synchronize()
    rot_ms = (time.perf_counter() - t0) * 1e3 / 5
    out = {"workload": OUTLIER_WORKLOAD, "rows_x": inp.T, "rows_z": inp.T * inp.k,
           "rotate_in_ms": rot_ms, "angles": "random U(-pi, pi), not learned"}
    # the fully spread limit: iid N(0, 1) rows of the same shape
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    gauss = torch.randn(inp.T, inp.d, device=dev, generator=gen).to(torch.bfloat16)
    for tag, v in (("x", x), ("z", z), ("gaussian_reference", gauss)):
        res = {}
        for name, m, mode in QUANTISERS:
            err, crest = bmoe.quant_error(v, m, mode)
            res[name] = float(err.double().mean())
        res["crest"] = float(crest.double().mean())
        out[tag] = res
    log(f"[bench] outliers {OUTLIER_WORKLOAD}: "
        + "; ".join(f"{q}: x {out['x'][q]:.4f} -> z {out['z'][q]:.4f} "
                    f"(iid normal {out['gaussian_reference'][q]:.4f})"
                    for q in [n for n, _, _ in QUANTISERS] + ["crest"]))
    del x, z, ids, theta, gauss
    torch.cuda.empty_cache()
    return out


def ceilings_section(reps=10):
    """Measured ceilings of the three resources, beside the published peaks:
    dense bf16 MFMA, fp32 vector FMA without packed ops, and a plain device
    copy (bytes read + written over time). Median of `reps` timed launches
    after two untimed ones, from each launch's own dispatch events."""
    import torch
    from butterfly_rotated_ternary_amd import bmoe
    hip = HipEvents()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sink = torch.empty(bmoe.BMOE_CEILING_SINK_FLOATS, device=dev)

    def median_ms(launch):
        evsets = [hip.create(2) for _ in range(reps + 2)]
        for evs in evsets:
            rc = launch(evs)
            if rc != 0:
                raise bmoe.BmoeError(rc, "ceiling launch")
        torch.cuda.synchronize()
        ms = sorted(hip.elapsed_ms(e[0], e[1]) for e in evsets[2:])
        for evs in evsets:
            hip.destroy(evs)
        return ms[len(ms) // 2]

    out = {}
    flops = {}

    def mfma(evs):
        rc, flops["mfma"] = bmoe.bmoe_ceiling_mfma_bf16(8000, sink, stream, evs)
        return rc

    def valu(evs):
        rc, flops["valu"] = bmoe.bmoe_ceiling_valu_f32(2000, sink, stream, evs)
        return rc

    t = median_ms(mfma)
    out["mfma_bf16"] = {"measured": flops["mfma"] / (t * 1e-3) / 1e12, "unit": "TFLOP/s",
                        "published": PEAK_BF16_TFLOPS}
    t = median_ms(valu)
    out["valu_f32"] = {"measured": flops["valu"] / (t * 1e-3) / 1e12, "unit": "TFLOP/s",
                       "published": PEAK_VALU_F32_TFLOPS}
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    t = median_ms(lambda evs: bmoe.bmoe_ceiling_copy(src, dst, nbytes, stream, evs))
    out["hbm_copy"] = {"measured": 2 * nbytes / (t * 1e-3) / 1e9, "unit": "GB/s",
                       "published": PEAK_HBM_GBS, "bytes_each_way": nbytes}
    for v in out.values():
        v["frac_of_published"] = v["measured"] / v["published"]
    del src, dst, sink
    torch.cuda.empty_cache()
    log("[bench] ceilings: " + "; ".join(f"{k} {v['measured']:.0f} {v['unit']} "
                                         f"({100 * v['frac_of_published']:.0f}% of published)"
                                         for k, v in out.items()))
    return out


def measured_ceiling(ceilings, roof):
    """The measured ceiling of a roofline's bound resource, or None."""
    key = {"hbm": "hbm_copy", "mfma": "mfma_bf16", "alu": "valu_f32"}[roof["bound"]]
    if roof["bound"] == "mfma" and roof["peak"] != PEAK_BF16_TFLOPS:
        return None
    return ceilings[key]["measured"] if ceilings and key in ceilings else None


def profile_run(names, steps, backward):
    """Only `steps` forwards (and backwards) of each workload, for counter
    collection under rocprofv3 --pmc: no timing, no JSON."""
    import torch
    for name in names:
        P = Problem(name)
        for _ in range(steps):
            P.step()
        if backward:
            P.backward_setup()
            for _ in range(steps):
                rc = P.bmoe.bmoe_backward(*P.backward_args())
                if rc != 0:
                    raise P.bmoe.BmoeError(rc, "bmoe_backward")
        torch.cuda.synchronize()
        log(f"[bench] profiled {name}: {steps} forward(s)" + (" and backward(s)" if backward else ""))
        del P
        torch.cuda.empty_cache()


def copy_calibration(mib, reps):
    """Plain device-to-device copies of a known size, for scaling the HBM
    byte counters (run under rocprofv3 --pmc)."""
    import torch
    n = mib << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--gemm-steps", type=int, default=20,
                    help="forwards of the d=4096 workload timed for its GEMM figure (0: skip)")
    ap.add_argument("--bwd-steps", type=int, default=100,
                    help="backward passes timed on the same workload (0: skip)")
    ap.add_argument("--router-steps", type=int, default=200,
                    help="router passes timed on the same workload (0: skip)")
    ap.add_argument("--workload-steps", type=int, default=50,
                    help="forward steps timed for each other workload (0: skip)")
    ap.add_argument("--no-outliers", action="store_true",
                    help="skip the outlier-spreading measurement")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run plain copies of MIB MiB (counter calibration) and exit")
    ap.add_argument("--print-source-digest", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured MFMA / VALU / copy ceilings")
    ap.add_argument("--profile", default=None, metavar="WORKLOADS",
                    help="only run --profile-steps forwards of these comma-separated workloads "
                         "(counter collection) and exit")
    ap.add_argument("--profile-steps", type=int, default=20)
    ap.add_argument("--profile-backward", action="store_true",
                    help="with --profile: also run that many backwards")
    args = ap.parse_args()
    if args.print_source_digest:
        print(source_digest())
        return
    if args.gpus != 1:
        log("bench.py measures one GPU only: the forward shards by tokens with no exchange, "
            "so a multi-GPU figure is not produced. Run with --gpus 1.")
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 10)
        return
    if args.profile:
        profile_run(args.profile.split(","), args.profile_steps, args.profile_backward)
        return

    from butterfly_rotated_ternary_amd import workloads as W

    name = args.workload or W.HEADLINE
    ceilings = None if args.no_ceilings else ceilings_section()
    P = Problem(name)
    T, d, N, k = P.T, P.d, P.N, P.k
    ms = P.time_steps(args.steps, args.warmup)
    value = T / (ms * 1e-3)
    log(f"[bench] {name}: {ms * 1e3:.2f} us/step, {value:.4g} tokens/s")

    per_kernel = P.time_kernels(min(args.steps, 200))
    log("[bench] per-kernel us (dispatch events): "
        + ", ".join(f"{n}={v * 1e3:.2f}" for n, v in per_kernel.items()))
    dom = max(per_kernel, key=per_kernel.get)
    routed = "prep_kernel" not in per_kernel
    work = kernel_work(dom, P.act_bytes, T, d, N, k, routed)
    roof = roofline(work, per_kernel[dom] * 1e-3, P.mfma_peak())
    roof["traffic"] = stored_traffic(dom, name)
    roof["kernel"] = dom
    mc = measured_ceiling(ceilings, roof)
    roof["frac_of_measured_ceiling"] = roof["achieved"] / mc if mc else None
    others = {}
    for n, v in per_kernel.items():
        r = roofline(kernel_work(n, P.act_bytes, T, d, N, k, routed), v * 1e-3, P.mfma_peak())
        others[n] = {"us": v * 1e3, "bound": r["bound"], "frac": r["frac"]}

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
        "dtype": "bf16" if P.act_bytes == 2 else "f32",
        "data": "synthetic",
        "config": {"workload": name, "d": d, "n_experts": N, "top_k": k, "tokens": T,
                   "routed_rows": M},
        "roofline": roof,
        "routed_rows_per_s": M / (ms * 1e-3),
        "e2e_frac": {"mfma_bf16": 2 * M * d * d / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
                     "hbm": min_hbm_bytes(P.act_bytes, T, d, N, k) / (ms * 1e-3)
                     / (PEAK_HBM_GBS * 1e9)},
        "kernels": others,
        "ceilings": ceilings,
    }
    if args.router_steps > 0:
        out["router"] = router_section(P, args.router_steps)
        out["base3"] = base3_section(P, 50, ms)
        out["base3"]["product"] = product_formats_section()
    if args.bwd_steps > 0:
        out["backward"] = backward_section(P, args.bwd_steps)
    del P

    if args.gemm_steps > 0 and name != GEMM_WORKLOAD:
        # The shared ternary product at d = 4096 (its own workload, same path).
        import torch
        G = Problem(GEMM_WORKLOAD)
        g_ms = G.time_steps(args.gemm_steps, 3)
        g_per = G.time_kernels(args.gemm_steps)
        g_work = kernel_work("gemm_kernel", G.act_bytes, G.T, G.d, G.N, G.k)
        g_roof = roofline(g_work, g_per["gemm_kernel"] * 1e-3, G.mfma_peak())
        g_roof["traffic"] = stored_traffic("gemm_kernel", GEMM_WORKLOAD)
        mc = measured_ceiling(ceilings, g_roof)
        g_roof["frac_of_measured_ceiling"] = g_roof["achieved"] / mc if mc else None
        out["gemm_d4096"] = {
            "workload": GEMM_WORKLOAD, "kernel": "gemm_kernel", "ms_per_step": g_ms,
            "tokens_per_s": G.T / (g_ms * 1e-3), "roofline": g_roof,
            "kernels_us": {n: v * 1e3 for n, v in g_per.items()},
        }
        log(f"[bench] {GEMM_WORKLOAD}: {g_ms * 1e3:.1f} us/step; gemm_kernel "
            f"{g_roof['achieved']:.0f} TFLOP/s ({100 * g_roof['frac']:.1f}% of bf16 peak); "
            + ", ".join(f"{n}={v * 1e3:.1f}" for n, v in g_per.items()))
        del G
        torch.cuda.empty_cache()
        # One GPU's share when the same workload is split by tokens over 8
        # GPUs (the forward needs no exchange): T = 4096 tokens per GPU.
        S = Problem(GEMM_WORKLOAD, T=SHARD_TOKENS)
        s_ms = S.time_steps(args.gemm_steps, 3)
        s_per = S.time_kernels(args.gemm_steps)
        s_roof = roofline(kernel_work("gemm_kernel", S.act_bytes, S.T, S.d, S.N, S.k),
                          s_per["gemm_kernel"] * 1e-3, S.mfma_peak())
        out["shard_d4096"] = {
            "workload": GEMM_WORKLOAD, "tokens": S.T, "split": "tokens over 8 GPUs",
            "ms_per_step": s_ms, "tokens_per_s": S.T / (s_ms * 1e-3), "gemm_roofline": s_roof,
            "kernels_us": {n: v * 1e3 for n, v in s_per.items()},
        }
        log(f"[bench] {GEMM_WORKLOAD} at T={S.T} (one GPU of 8): {s_ms * 1e3:.1f} us/step, "
            f"{S.T / (s_ms * 1e-3):.4g} tokens/s; gemm_kernel {s_roof['achieved']:.0f} TFLOP/s "
            f"({100 * s_roof['frac']:.1f}%); "
            + ", ".join(f"{n}={v * 1e3:.1f}" for n, v in s_per.items()))
        del S
        torch.cuda.empty_cache()

    if args.workload_steps > 0:
        out["workloads"] = workloads_section(args.workload_steps, skip=(name, GEMM_WORKLOAD))

    if not args.no_outliers:
        out["outliers"] = outliers_section()

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(W.make_inputs(name), args.cpu_seconds)
        log(f"[bench] cpu baseline {out['cpu_baseline']['value']:.4g} tokens/s "
            f"({out['cpu_baseline']['sample']})")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
