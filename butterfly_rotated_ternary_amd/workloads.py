"""Seeded synthetic workloads for the ButterflyMoE expert-layer forward.

This module only draws inputs. It holds none of the method's arithmetic
(no rotation, no contraction, no routing), so both the HIP path and the CPU
oracle can take their inputs from here without sharing any computation.

The pages measure on language-modelling benchmarks with trained weights
(ButterflyMoE arXiv abstract; gist.science summary, section 4). Those are not
available, so seeded random inputs with the shapes below stand in for them.

Recipe (one numpy ``Generator(PCG64(seed))`` per workload; draws happen in
this fixed order):

1. ``W_base`` codes: iid, ``P(+1) = P(-1) = density/2``, ``P(0) = 1 - density``.
2. ``theta`` ~ U(-pi, pi), shape ``[N][L][d/2]``, fp32.
3. ``phi``   ~ U(-pi, pi), same shape.
4. ``x`` ~ N(0, 1), shape ``[T][d]``, fp32.
5. outlier channels (only when ``outlier_frac > 0``): ``round(outlier_frac*d)``
   distinct channels, shared by all tokens, multiplied by ``outlier_scale``
   before any rounding to bf16.
6. routing keys: ``U(0,1)`` of shape ``[T][N]``; each token takes the ``k``
   experts with the largest Gumbel keys ``log w_e - log(-log u)``, listed in
   descending key order (successive sampling without replacement). ``w_e = 1``
   for uniform routing and ``(e+1)^-s`` for Zipf routing, so expert 0 is the
   hottest.
7. gate logits ~ N(0, 1), shape ``[T][k]``; gates are their softmax over the
   ``k`` entries of each token, taken in fp64 and stored as fp32.

Router weights (for the router in front of the layer) come from a separate
generator, ``PCG64(seed + 1_000_000)``, so the draws above do not change:
``w_router`` ~ N(0, 1/d), shape ``[N][d]`` (one row per expert), which gives
logits of unit variance for N(0, 1) inputs; rounded to bf16 like ``x`` for
bf16 workloads.

``alpha = fp32(1/sqrt(d))``. For bf16 workloads ``x`` is rounded to bf16 with
round-to-nearest-even; ``x`` then holds the exact bf16 values as fp32 and
``x_bits`` their raw 16-bit patterns.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

# Named workloads. Each name states its shape; the first is small enough for
# the oracle to finish in seconds, the second is the throughput workload.
WORKLOADS = {
    "tiny_d64_e8_top2_f32": dict(d=64, N=8, k=2, T=256, dtype="f32", density=2.0 / 3.0,
                                 routing="uniform", seed=1001),
    "d512_e64_top2_bf16": dict(d=512, N=64, k=2, T=4096, dtype="bf16", density=2.0 / 3.0,
                               routing="uniform", seed=1002),
    "d512_e256_top2_zipf_bf16": dict(d=512, N=256, k=2, T=16384, dtype="bf16",
                                     density=2.0 / 3.0, routing="zipf", zipf_s=1.1,
                                     seed=1003),
    "d2048_e64_top2_outliers_bf16": dict(d=2048, N=64, k=2, T=16384, dtype="bf16",
                                         density=0.5, routing="uniform",
                                         outlier_frac=0.01, outlier_scale=20.0, seed=1004),
    "d4096_e256_top4_bf16": dict(d=4096, N=256, k=4, T=32768, dtype="bf16",
                                 density=2.0 / 3.0, routing="uniform", seed=1005),
}

SMALL = "tiny_d64_e8_top2_f32"
HEADLINE = "d512_e64_top2_bf16"


def log2_exact(d: int) -> int:
    L = int(d).bit_length() - 1
    if d < 2 or (1 << L) != d:
        raise ValueError(f"d must be a power of two >= 2, got {d}")
    return L


def bf16_round_bits(x32: np.ndarray) -> np.ndarray:
    """Raw bf16 bit patterns of fp32 ``x32`` under round-to-nearest-even.

    Inputs are finite by construction (normal draws), so NaN handling is not
    needed here.
    """
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Inputs:
    name: str
    d: int
    N: int
    k: int
    T: int
    dtype: str             # "f32" or "bf16": storage type of x and y
    x: np.ndarray          # [T][d] fp32: the exact values the kernel receives
    x_bits: Optional[np.ndarray]  # [T][d] uint16 bf16 patterns (bf16 only)
    ids: np.ndarray        # [T][k] int32 expert ids, draw order
    gates: np.ndarray      # [T][k] fp32 gate weights
    theta: np.ndarray      # [N][L][d/2] fp32, input-side angles
    phi: np.ndarray        # [N][L][d/2] fp32, output-side angles
    w: np.ndarray          # [d][d] int8 in {-1,0,+1}; row = output, col = input
    alpha: np.float32      # per-matrix scale of W_base
    outlier_channels: Optional[np.ndarray] = None

    @property
    def L(self) -> int:
        return log2_exact(self.d)

    @property
    def M(self) -> int:
        return self.T * self.k


def _route_ids(rng: np.random.Generator, T: int, N: int, k: int, routing: str,
               zipf_s: float) -> np.ndarray:
    if k > N:
        raise ValueError("k must not exceed N")
    if routing == "uniform":
        logw = np.zeros(N)
    elif routing == "zipf":
        logw = -zipf_s * np.log(np.arange(1, N + 1, dtype=np.float64))
    else:
        raise ValueError(f"unknown routing {routing!r}")
    ids = np.empty((T, k), dtype=np.int32)
    chunk = 4096
    for t0 in range(0, T, chunk):
        u = rng.random((min(chunk, T - t0), N))
        # Gumbel-top-k: u in [0,1); guard the measure-zero u == 0.
        keys = logw[None, :] - np.log(-np.log(np.maximum(u, 1e-300)))
        top = np.argpartition(-keys, k - 1, axis=1)[:, :k] if k < N else \
            np.tile(np.arange(N), (keys.shape[0], 1))
        topkeys = np.take_along_axis(keys, top, axis=1)
        order = np.argsort(-topkeys, axis=1, kind="stable")
        ids[t0:t0 + keys.shape[0]] = np.take_along_axis(top, order, axis=1)
    return ids


def make_inputs(name: str = HEADLINE, *, T: Optional[int] = None, seed: Optional[int] = None,
                **override) -> Inputs:
    """Draw the named workload. ``T``, ``seed`` and any config key may be
    overridden to get a smaller case with the same distributions."""
    if name in WORKLOADS:
        cfg = dict(WORKLOADS[name])
    else:
        cfg = dict(d=64, N=8, k=2, T=16, dtype="f32", density=2.0 / 3.0,
                   routing="uniform", seed=1)
    cfg.update(override)
    if T is not None:
        cfg["T"] = T
    if seed is not None:
        cfg["seed"] = seed
    d, N, k, T = cfg["d"], cfg["N"], cfg["k"], cfg["T"]
    L = log2_exact(d)
    rng = np.random.Generator(np.random.PCG64(cfg["seed"]))

    dens = float(cfg["density"])
    u = rng.random((d, d))
    w = np.zeros((d, d), dtype=np.int8)
    w[u < dens / 2] = 1
    w[(u >= dens / 2) & (u < dens)] = -1
    del u

    theta = rng.uniform(-np.pi, np.pi, size=(N, L, d // 2)).astype(np.float32)
    phi = rng.uniform(-np.pi, np.pi, size=(N, L, d // 2)).astype(np.float32)

    x = rng.standard_normal((T, d), dtype=np.float32)
    outl = None
    frac = float(cfg.get("outlier_frac", 0.0))
    if frac > 0:
        n_out = int(round(frac * d))
        outl = np.sort(rng.choice(d, size=n_out, replace=False))
        x[:, outl] *= np.float32(cfg.get("outlier_scale", 20.0))

    ids = _route_ids(rng, T, N, k, cfg["routing"], float(cfg.get("zipf_s", 1.1)))

    logits = rng.standard_normal((T, k))
    ex = np.exp(logits - logits.max(axis=1, keepdims=True))
    gates = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)

    x_bits = None
    if cfg["dtype"] == "bf16":
        x_bits = bf16_round_bits(x)
        x = bf16_bits_to_f32(x_bits)
    elif cfg["dtype"] != "f32":
        raise ValueError("dtype must be 'f32' or 'bf16'")

    return Inputs(name=name, d=d, N=N, k=k, T=T, dtype=cfg["dtype"], x=x, x_bits=x_bits,
                  ids=ids, gates=gates, theta=theta, phi=phi, w=w,
                  alpha=np.float32(1.0 / math.sqrt(d)), outlier_channels=outl)


@dataclasses.dataclass
class RouterWeights:
    w: np.ndarray                  # [N][d] fp32: the exact values the kernel receives
    w_bits: Optional[np.ndarray]   # [N][d] uint16 bf16 patterns (bf16 only)


def make_router_weights(inp: Inputs, seed: Optional[int] = None) -> RouterWeights:
    """Router weights for a drawn workload (own generator; see the recipe)."""
    base = WORKLOADS[inp.name]["seed"] if seed is None and inp.name in WORKLOADS else (seed or 1)
    rng = np.random.Generator(np.random.PCG64(base + 1_000_000))
    w = (rng.standard_normal((inp.N, inp.d)) / math.sqrt(inp.d)).astype(np.float32)
    if inp.dtype == "bf16":
        bits = bf16_round_bits(w)
        return RouterWeights(w=bf16_bits_to_f32(bits), w_bits=bits)
    return RouterWeights(w=w, w_bits=None)
