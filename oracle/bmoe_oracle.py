"""Plain, slow, fp64 CPU oracle of the ButterflyMoE expert-layer forward.

TEST INFRASTRUCTURE ONLY: used by ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg. The HIP library never calls it, and it
shares no code with the HIP path.

What the pages fix (ButterflyMoE: Sub-Linear Ternary Experts via Structured
Butterfly Orbits, gist.science technical summary):

* §2.1 Basic parameterisation: expert ``i`` is ``W_i = B(phi_i) W_base B(theta_i)^T``
  with one ternary ``W_base`` in {-1, 0, +1} shared by every expert, and
  ``B(.)`` learned butterfly-structured rotations with O(d log d) parameters.
* §2.2 Memory scaling: total storage O(d^2 + N d log d).
* §2.3 Inference: ``W_i`` is never materialised; the input is rotated by
  ``B(theta_i)^T``, multiplied by ``W_base`` (a ternary product), then
  rotated by ``B(phi_i)``.

Readings where the pages are silent (each is also listed in the design notes):

* ``B(a) = S_{L-1}(a_{L-1}) ... S_1(a_1) S_0(a_0)``, ``L = log2 d``. Stage ``s``
  rotates every pair ``(i, i + 2^s)`` with bit ``s`` of ``i`` clear; pair index
  ``p`` enumerates those ``i`` in ascending order. So ``B x`` applies the
  stride-1 stage first, and ``B^T x`` applies ``S_{L-1}^T`` first.
* A Givens rotation acts on ``(x_i, x_j)`` as ``[[c, -s], [s, c]]`` with
  ``c = cos a``, ``s = sin a``; its transpose negates the angle.
* Angles are ``fp32[N][L][d/2]`` (stage-major); the oracle takes cos and sin of
  the fp32 angle in fp64.
* One fp32 scale ``alpha`` multiplies ``W_base`` (applied after the
  contraction; identical in exact arithmetic).
* The top-k expert outputs of a token are summed with the given gates
  (standard top-k MoE): ``y_t = sum_j g_tj W_{e_tj} x_t``.
* Rows are grouped by expert with a stable counting sort keyed by the routed
  index ``r = t*k + j``.

Nothing here rounds: bf16 inputs arrive as their exact values, all arithmetic
is fp64.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "n_stages", "stage_pairs", "apply_butterfly", "stage_matrix", "butterfly_matrix",
    "expert_matrix", "route", "pack_ternary", "unpack_ternary", "param_count",
    "forward", "forward_tokens", "forward_materialized", "forward_bruteforce",
    "max_rel_err",
]


def n_stages(d: int) -> int:
    """Number of butterfly stages, log2 d (d must be a power of two >= 2)."""
    L = int(d).bit_length() - 1
    if d < 2 or (1 << L) != d:
        raise ValueError(f"d must be a power of two >= 2, got {d}")
    return L


def stage_pairs(d: int, s: int):
    """Index pairs ``(i, j = i + 2^s)`` rotated by stage ``s``, for pair index
    ``p = 0 .. d/2-1`` in ascending ``i`` (bit ``s`` of ``i`` clear)."""
    p = np.arange(d // 2, dtype=np.int64)
    low = p & ((1 << s) - 1)
    high = (p >> s) << (s + 1)
    i = high | low
    return i, i + (1 << s)


def apply_butterfly(angles, X, transpose: bool = False) -> np.ndarray:
    """Apply ``B(angles)`` (or ``B(angles)^T``) to every row of ``X``.

    ``angles``: ``[L][d/2]`` for one expert. ``X``: ``[n][d]``. Stage by stage,
    without forming the matrix (gist.science summary, §2.3).
    """
    X = np.array(X, dtype=np.float64, copy=True)
    if X.ndim == 1:
        return apply_butterfly(angles, X[None, :], transpose)[0]
    d = X.shape[1]
    L = n_stages(d)
    ang = np.asarray(angles)
    assert ang.shape == (L, d // 2)
    stages = range(L - 1, -1, -1) if transpose else range(L)
    for s in stages:
        a = ang[s].astype(np.float64)
        c, sn = np.cos(a), np.sin(a)
        if transpose:
            sn = -sn
        i, j = stage_pairs(d, s)
        xi = X[:, i].copy()
        xj = X[:, j].copy()
        X[:, i] = c * xi - sn * xj
        X[:, j] = sn * xi + c * xj
    return X


def stage_matrix(angles_s, d: int, s: int) -> np.ndarray:
    """Dense ``d x d`` matrix of stage ``s``: identity except for one 2x2
    Givens block per pair. Built entry by entry, independently of
    ``apply_butterfly``."""
    S = np.zeros((d, d))
    for p in range(d // 2):
        blk = 1 << s
        i = (p // blk) * (2 * blk) + (p % blk)
        j = i + blk
        a = float(np.float64(np.asarray(angles_s)[p]))
        c, sn = np.cos(a), np.sin(a)
        S[i, i] = c
        S[i, j] = -sn
        S[j, i] = sn
        S[j, j] = c
    return S


def butterfly_matrix(angles) -> np.ndarray:
    """Dense ``B = S_{L-1} ... S_0`` (small d only)."""
    ang = np.asarray(angles)
    L = ang.shape[0]
    d = 2 * ang.shape[1]
    assert n_stages(d) == L
    B = np.eye(d)
    for s in range(L):
        B = stage_matrix(ang[s], d, s) @ B
    return B


def expert_matrix(theta_e, phi_e, w, alpha) -> np.ndarray:
    """Materialised ``alpha * B(phi_e) W_base B(theta_e)^T`` (gist.science
    summary, §2.1). Small d only: this is exactly what inference avoids."""
    return float(alpha) * (butterfly_matrix(phi_e) @ np.asarray(w, dtype=np.float64)
                           @ butterfly_matrix(theta_e).T)


def route(ids, n_experts: int):
    """Group routed rows by expert with a stable counting sort.

    ``ids``: ``[T][k]``; routed index ``r = t*k + j``. Returns int32
    ``offsets[N+1]`` (exclusive prefix of per-expert counts), ``perm[M]``
    (sorted slot -> routed index, ascending ``r`` within an expert, experts
    ascending) and ``inv[M]`` (routed index -> sorted slot).
    """
    flat = np.asarray(ids).reshape(-1).astype(np.int64)
    if flat.size and (flat.min() < 0 or flat.max() >= n_experts):
        raise ValueError("expert id out of range")
    counts = np.zeros(n_experts, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    cursor = offsets[:-1].copy()
    perm = np.empty(flat.size, dtype=np.int64)
    inv = np.empty(flat.size, dtype=np.int64)
    for r, e in enumerate(flat):
        q = cursor[e]
        cursor[e] += 1
        perm[q] = r
        inv[r] = q
    return offsets.astype(np.int32), perm.astype(np.int32), inv.astype(np.int32)


# Packed W_base layout (a storage reading: the pages give 1.58 bit/weight as
# the information content, §2.1; the stored form here uses 2 bits/weight).
# Row o (output), group g of 16 input columns c = 16g .. 16g+15 -> one uint32
# at [o][g]. Each weight is a 2-bit code, nonzero flag in the low bit and
# sign in the high bit: +1 -> 01, -1 -> 11, 0 -> 00 (10 never occurs). For
# v = c - 16g: v = 2j takes bits 2j (flag) and 2j+1 (sign); v = 2j+1 takes
# bits 16+2j and 17+2j, so even columns fill the low half-word and odd columns
# the high one. Rows with d < 16 pad with zeros.

def _bit_positions(v: int):
    j = v >> 1
    if v & 1:
        return 16 + 2 * j, 17 + 2 * j
    return 2 * j, 2 * j + 1


def pack_ternary(w) -> np.ndarray:
    """int8 ``[d][d]`` in {-1,0,+1} -> uint32 ``[d][ceil(d/16)]``."""
    w = np.asarray(w)
    d = w.shape[0]
    assert w.shape == (d, d)
    if not np.isin(w, (-1, 0, 1)).all():
        raise ValueError("W_base entries must be -1, 0 or +1")
    G = (d + 15) // 16
    out = np.zeros((d, G), dtype=np.uint64)
    for c in range(d):
        g, v = divmod(c, 16)
        bnz, bsg = _bit_positions(v)
        col = w[:, c].astype(np.int64)
        out[:, g] |= (col != 0).astype(np.uint64) << np.uint64(bnz)
        out[:, g] |= (col < 0).astype(np.uint64) << np.uint64(bsg)
    return out.astype(np.uint32)


def unpack_ternary(packed, d: int) -> np.ndarray:
    """Inverse of ``pack_ternary``."""
    packed = np.asarray(packed, dtype=np.uint64)
    w = np.zeros((d, d), dtype=np.int8)
    for c in range(d):
        g, v = divmod(c, 16)
        bnz, bsg = _bit_positions(v)
        nz = (packed[:, g] >> np.uint64(bnz)) & np.uint64(1)
        sg = (packed[:, g] >> np.uint64(bsg)) & np.uint64(1)
        if np.any((nz == 0) & (sg == 1)):
            raise ValueError("invalid code (zero with sign set)")
        w[:, c] = np.where(nz == 1, np.where(sg == 1, -1, 1), 0)
    return w


def param_count(w, theta, phi) -> int:
    """Stored parameters: the shared substrate plus both angle sets
    (gist.science summary, §2.2: O(d^2 + N d log d))."""
    return int(np.asarray(w).size + np.asarray(theta).size + np.asarray(phi).size)


def forward(x, ids, gates, theta, phi, w, alpha, chunk: int = 4096) -> np.ndarray:
    """Factored forward for all tokens, in the pages' inference order
    (gist.science summary, §2.3), after grouping rows by expert:

    1. route (stable counting sort);
    2. ``z = B(theta_e)^T x_t`` for every sorted slot;
    3. ``h = alpha * W_base z`` (one fp64 product over all slots);
    4. ``u = B(phi_e) h``;
    5. ``y_t = sum_j g_tj u_{t,j}`` over ascending ``j``.
    """
    x = np.asarray(x)
    T, d = x.shape
    ids = np.asarray(ids)
    k = ids.shape[1]
    N = np.asarray(theta).shape[0]
    offsets, perm, inv = route(ids, N)
    M = T * k
    W64 = np.asarray(w, dtype=np.float64)
    U = np.empty((M, d))
    for e in range(N):
        q0, q1 = int(offsets[e]), int(offsets[e + 1])
        for a in range(q0, q1, chunk):
            b = min(q1, a + chunk)
            rows = perm[a:b]
            Z = apply_butterfly(theta[e], x[rows // k].astype(np.float64), transpose=True)
            H = float(alpha) * (Z @ W64.T)
            U[a:b] = apply_butterfly(phi[e], H, transpose=False)
    y = np.zeros((T, d))
    g = np.asarray(gates, dtype=np.float64)
    for j in range(k):
        y += g[:, j:j + 1] * U[inv.reshape(T, k)[:, j]]
    return y


def forward_tokens(tokens, x, ids, gates, theta, phi, w, alpha) -> np.ndarray:
    """Factored forward of selected tokens only (for sampled checks at sizes
    where the full oracle would take minutes)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    d = np.asarray(x).shape[1]
    W64 = np.asarray(w, dtype=np.float64)
    out = np.zeros((tokens.size, d))
    for n, t in enumerate(tokens):
        for j in range(np.asarray(ids).shape[1]):
            e = int(ids[t, j])
            z = apply_butterfly(theta[e], np.asarray(x[t], dtype=np.float64), transpose=True)
            h = float(alpha) * (W64 @ z)
            out[n] += float(gates[t, j]) * apply_butterfly(phi[e], h)
    return out


def forward_materialized(x, ids, gates, theta, phi, w, alpha) -> np.ndarray:
    """``y_t = sum_j g_tj W_{e_tj} x_t`` with every ``W_e`` formed densely
    (small d only)."""
    x = np.asarray(x, dtype=np.float64)
    N = np.asarray(theta).shape[0]
    We = [expert_matrix(theta[e], phi[e], w, alpha) for e in range(N)]
    y = np.zeros_like(x)
    for t in range(x.shape[0]):
        for j in range(np.asarray(ids).shape[1]):
            y[t] += float(gates[t, j]) * (We[int(ids[t, j])] @ x[t])
    return y


def forward_bruteforce(x, ids, gates, theta, phi, w, alpha) -> np.ndarray:
    """Pure-Python loops over every rotation and product (tiny cases only)."""
    import math
    x = [[float(v) for v in row] for row in np.asarray(x)]
    T = len(x)
    d = len(x[0])
    L = n_stages(d)
    k = np.asarray(ids).shape[1]

    def rotate(vec, ang, transpose):
        v = list(vec)
        order = range(L - 1, -1, -1) if transpose else range(L)
        for s in order:
            h = 1 << s
            p = 0
            for i in range(d):
                if i & h:
                    continue
                a = float(ang[s][p])
                c, sn = math.cos(a), math.sin(a)
                if transpose:
                    sn = -sn
                xi, xj = v[i], v[i + h]
                v[i] = c * xi - sn * xj
                v[i + h] = sn * xi + c * xj
                p += 1
        return v

    y = [[0.0] * d for _ in range(T)]
    for t in range(T):
        for j in range(k):
            e = int(ids[t][j])
            z = rotate(x[t], theta[e], True)
            h = [float(alpha) * sum(float(w[o][c]) * z[c] for c in range(d)) for o in range(d)]
            u = rotate(h, phi[e], False)
            g = float(gates[t][j])
            for o in range(d):
                y[t][o] += g * u[o]
    return np.array(y)


def max_rel_err(y, ref, zero_tol: float = 1e-6) -> float:
    """Largest per-token ``||y_t - ref_t||_inf / ||ref_t||_inf``.

    Elementwise relative error is unbounded at zero crossings, so the error
    of a token is taken relative to its largest reference entry. Tokens whose
    reference is exactly zero contribute ``||y_t||_inf / zero_tol``.
    """
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(y - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    zero = den == 0
    rel = np.where(zero, num / zero_tol, num / np.where(zero, 1.0, den))
    return float(rel.max()) if rel.size else 0.0
