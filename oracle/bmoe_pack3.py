"""Plain CPU oracle of the base-3 storage of the ternary substrate.

TEST INFRASTRUCTURE ONLY: used by ``tests/`` and ``bench.py``'s
``cpu_baseline`` leg. The HIP library never calls it, and it shares no code
with the HIP path.

The summary (ButterflyMoE, gist.science technical summary, §2.1) stores the
shared ternary substrate at 1.58 bits per weight, which is log2(3). The
plainest byte-aligned form of that is five ternary digits per byte
(3^5 = 243 <= 256): 8/5 = 1.6 bits per weight. Reading taken here:

* the d*d entries are taken in row-major order, entry n = o*d + c;
* byte j holds entries 5j .. 5j+4 as the base-3 number
  ``sum_i (w[5j+i] + 1) * 3^i`` (digit 0 = -1, 1 = 0, 2 = +1; entry 5j is the
  least significant digit);
* the last byte's digits past d*d are 1 (the value 0); the stream has
  ``ceil(d*d / 5)`` bytes.
"""
from __future__ import annotations

import numpy as np

__all__ = ["packed3_bytes", "pack_ternary_b3", "unpack_ternary_b3"]


def packed3_bytes(d: int) -> int:
    return -(-d * d // 5)


def pack_ternary_b3(w) -> np.ndarray:
    """int8 [d][d] in {-1, 0, +1} -> uint8 [ceil(d*d/5)]."""
    w = np.asarray(w)
    d = w.shape[0]
    if w.shape != (d, d) or not np.isin(w, (-1, 0, 1)).all():
        raise ValueError("w must be a square matrix of -1, 0, +1")
    flat = w.reshape(-1).astype(np.int64) + 1
    n = packed3_bytes(d)
    digits = np.ones(n * 5, dtype=np.int64)
    digits[:flat.size] = flat
    digits = digits.reshape(n, 5)
    out = np.zeros(n, dtype=np.int64)
    for i in range(5):
        out += digits[:, i] * 3 ** i
    return out.astype(np.uint8)


def unpack_ternary_b3(packed, d: int) -> np.ndarray:
    """uint8 [ceil(d*d/5)] -> int8 [d][d]; raises on a byte above 242."""
    b = np.asarray(packed).astype(np.int64)
    if b.shape != (packed3_bytes(d),):
        raise ValueError("wrong stream length")
    if (b > 242).any():
        raise ValueError("byte above 242 is not five ternary digits")
    digits = np.empty((b.size, 5), dtype=np.int64)
    rest = b.copy()
    for i in range(5):
        digits[:, i] = rest % 3
        rest //= 3
    return (digits.reshape(-1)[:d * d] - 1).astype(np.int8).reshape(d, d)
