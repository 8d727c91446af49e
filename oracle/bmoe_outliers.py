"""Plain fp64 CPU oracle of the outlier-spreading measurement.

TEST INFRASTRUCTURE ONLY: used by ``tests/`` and ``bench.py``'s
``cpu_baseline`` leg. The HIP library never calls it, and it shares no code
with the HIP path.

The summary (ButterflyMoE, gist.science technical summary, §2.4 and §4)
credits the learned rotation B(theta_e) with spreading activation outliers
over the dimensions, which lowers the activation quantisation error. The
pages name no quantiser; this measures the plain per-token symmetric ones:

* ``rotate_in``: ``z_r = B(theta_e)^T x_t`` for every routed row
  ``r = t*k + j`` with ``e = ids[t][j]`` (the first step of §2.3);
* ``quant_error``: for one row v and a level count m, with scale
  ``s = max|v| / m`` (``mode = 0``, absmax) or ``s = mean|v|`` (``mode = 1``,
  absmean; used with m = 1 for ternary), ``q = s * clip(rint(v / s), -m, m)``
  and the error ``||v - q|| / ||v||`` (0 for a zero row). ``rint`` rounds
  halves to even; the error does not depend on how a half is rounded, since
  both choices lie s/2 from v.
"""
from __future__ import annotations

import numpy as np

from .bmoe_oracle import apply_butterfly

__all__ = ["rotate_in", "quant_error", "crest_factor"]


def rotate_in(x, ids, theta) -> np.ndarray:
    """fp64 [T*k][d], row r = t*k + j holds B(theta_{ids[t][j]})^T x_t."""
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(ids)
    T, k = ids.shape
    out = np.empty((T * k, x.shape[1]))
    for j in range(k):
        for e in np.unique(ids[:, j]):
            rows = np.nonzero(ids[:, j] == e)[0]
            out[rows * k + j] = apply_butterfly(theta[e], x[rows], transpose=True)
    return out


def quant_error(V, m: int, mode: int = 0) -> np.ndarray:
    """Per-row relative quantisation error of the rows of V (fp64)."""
    V = np.asarray(V, dtype=np.float64)
    a = np.abs(V)
    s = a.max(axis=1) / m if mode == 0 else a.mean(axis=1)
    out = np.zeros(V.shape[0])
    nz = s > 0
    q = np.clip(np.rint(V[nz] / s[nz, None]), -m, m) * s[nz, None]
    out[nz] = np.sqrt(((V[nz] - q) ** 2).sum(axis=1) / (V[nz] ** 2).sum(axis=1))
    return out


def crest_factor(V) -> np.ndarray:
    """Per-row max|v| / rms(v) (0 for a zero row)."""
    V = np.asarray(V, dtype=np.float64)
    rms = np.sqrt((V ** 2).mean(axis=1))
    out = np.zeros(V.shape[0])
    nz = rms > 0
    out[nz] = np.abs(V[nz]).max(axis=1) / rms[nz]
    return out
