"""Plain, slow, fp64 CPU oracle of the ButterflyMoE expert-layer backward.

TEST INFRASTRUCTURE ONLY: used by ``tests/`` and ``bench.py``'s
``cpu_baseline`` leg. The HIP library never calls it, and it shares no code
with the HIP path.

The layer (ButterflyMoE: Sub-Linear Ternary Experts via Structured Butterfly
Orbits, gist.science technical summary, §2.1 and §2.3) maps token ``t`` to
``y_t = sum_j g_tj * B(phi_e) * alpha * W_base * B(theta_e)^T * x_t`` with
``e = ids[t][j]``. Training the rotations (summary §2.4) needs the gradients
of a scalar loss ``L`` given ``dy = dL/dy``. Written out for one routed row
``r = t*k + j`` with ``z = B(theta_e)^T x_t``, ``h = alpha W_base z`` and
``u = B(phi_e) h``:

* ``dL/dg_r = <dy_t, u>``;
* ``du = g_r dy_t``; ``dh = B(phi_e)^T du``; ``dz = alpha W_base^T dh``;
  ``dx_t = sum_j B(theta_e) dz``;
* ``dL/dW_base = alpha * sum_r dh z^T``: the gradient with respect to the
  substrate taken as a real matrix (the straight-through reading for a
  ternary weight: the update flows to a full-precision latent copy);
* a stage applies ``out_i = c x_i - s x_j``, ``out_j = s x_i + c x_j`` with
  ``c, s = cos a, sin a`` to its pair ``(i, j)``; with ``G = dL/dout`` its
  angle gets ``sum over rows of G_i (-s x_i - c x_j) + G_j (c x_i - s x_j)``
  and its input gets ``S^T G``. On the input side every stage runs
  transposed (angle ``-a``), so its angle gradient changes sign.

Every intermediate is kept from the forward (no inverse stages), all in fp64.
The stage conventions (order, pairs, sign) are the forward oracle's.
"""
from __future__ import annotations

import numpy as np

from .bmoe_oracle import n_stages, route, stage_pairs

__all__ = ["backward", "loss"]


def _stage(X, a, d, s, sign):
    """One stage on every row of X (angle sign * a); returns the output."""
    i, j = stage_pairs(d, s)
    c, sn = np.cos(a), sign * np.sin(a)
    out = X.copy()
    out[:, i] = c * X[:, i] - sn * X[:, j]
    out[:, j] = sn * X[:, i] + c * X[:, j]
    return out


def _stage_grad(X, G, a, d, s, sign):
    """Gradients of one stage (angle sign * a) from its input X and the
    gradient G of its output: returns (dX, dL/da summed over rows)."""
    i, j = stage_pairs(d, s)
    c, sn = np.cos(a), sign * np.sin(a)
    xi, xj, gi, gj = X[:, i], X[:, j], G[:, i], G[:, j]
    dX = np.empty_like(G)
    dX[:, i] = c * gi + sn * gj
    dX[:, j] = -sn * gi + c * gj
    d_eff = (gi * (-sn * xi - c * xj) + gj * (c * xi - sn * xj)).sum(axis=0)
    return dX, sign * d_eff


def backward(x, ids, gates, theta, phi, w, alpha, dy):
    """All gradients of ``L = sum_t <dy_t, y_t>``: returns a dict with
    ``dx [T][d]``, ``dgates [T][k]``, ``dtheta``/``dphi [N][L][d/2]`` and
    ``dw [d][d]``, all fp64."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    T, d = x.shape
    ids = np.asarray(ids)
    k = ids.shape[1]
    theta = np.asarray(theta)
    phi = np.asarray(phi)
    N = theta.shape[0]
    L = n_stages(d)
    W = np.asarray(w, dtype=np.float64)
    g = np.asarray(gates, dtype=np.float64).reshape(-1)
    a64 = float(alpha)
    offsets, perm, _ = route(ids, N)

    dx = np.zeros((T, d))
    dg = np.zeros(T * k)
    dth = np.zeros((N, L, d // 2))
    dph = np.zeros((N, L, d // 2))
    dw = np.zeros((d, d))
    for e in range(N):
        q0, q1 = int(offsets[e]), int(offsets[e + 1])
        if q0 == q1:
            continue
        rows = perm[q0:q1].astype(np.int64)
        tok = rows // k
        th = theta[e].astype(np.float64)
        ph = phi[e].astype(np.float64)
        # forward, keeping every stage input
        V = x[tok]
        in_side = []
        for s in range(L - 1, -1, -1):
            in_side.append((s, V))
            V = _stage(V, th[s], d, s, -1.0)
        Z = V
        H = a64 * (Z @ W.T)
        V = H
        out_side = []
        for s in range(L):
            out_side.append((s, V))
            V = _stage(V, ph[s], d, s, 1.0)
        U = V
        # backward
        Dy = dy[tok]
        dg[rows] = (Dy * U).sum(axis=1)
        G = g[rows][:, None] * Dy
        for s, Vin in reversed(out_side):
            G, da = _stage_grad(Vin, G, ph[s], d, s, 1.0)
            dph[e, s] += da
        dH = G
        dw += a64 * (dH.T @ Z)
        G = a64 * (dH @ W)
        for s, Vin in reversed(in_side):
            G, da = _stage_grad(Vin, G, th[s], d, s, -1.0)
            dth[e, s] += da
        np.add.at(dx, tok, G)
    return {"dx": dx, "dgates": dg.reshape(T, k), "dtheta": dth, "dphi": dph, "dw": dw}


def loss(x, ids, gates, theta, phi, w, alpha, dy) -> float:
    """``sum_t <dy_t, y_t>`` through the forward oracle (for finite-difference
    checks of ``backward``)."""
    from .bmoe_oracle import forward
    y = forward(x, ids, gates, theta, phi, w, alpha)
    return float((np.asarray(dy, dtype=np.float64) * y).sum())
