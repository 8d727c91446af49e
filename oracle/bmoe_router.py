"""Plain fp64 CPU oracle of the top-k router in front of the expert layer.

TEST INFRASTRUCTURE ONLY: used by ``tests/`` and ``bench.py``'s
``cpu_baseline`` leg. The HIP library never calls it, and it shares no code
with the HIP path.

The pages present the layer as a top-k mixture of experts (ButterflyMoE
abstract; gist.science summary §2.3) but give no router formula. This is the
plain top-k softmax gate, with these readings:

* ``logits[t][e] = <x_t, w_router[e]>``: the router weight is stored one row
  per expert, ``[N][d]`` (``W_r`` transposed);
* the k chosen experts are the k largest logits in descending order, equal
  logits going to the lower expert id;
* the gates are the softmax over the k chosen logits only.
"""
from __future__ import annotations

import numpy as np

__all__ = ["router_logits", "router"]


def router_logits(x, w_router):
    """fp64 logits ``[T][N]``."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w_router, dtype=np.float64).T


def router(x, w_router, k, logits=None):
    """Returns ``(ids int32 [T][k], gates fp64 [T][k], logits fp64 [T][N])``.
    ``logits`` may be given (e.g. another precision's) to choose from them."""
    if logits is None:
        logits = router_logits(x, w_router)
    logits = np.asarray(logits, dtype=np.float64)
    T, N = logits.shape
    if not 1 <= k <= N:
        raise ValueError("need 1 <= k <= N")
    # stable ascending sort of -logit: descending logit, lower id first on ties
    order = np.argsort(-logits, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    chosen = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    ex = np.exp(chosen - chosen[:, :1])
    gates = ex / ex.sum(axis=1, keepdims=True)
    return ids, gates, logits
