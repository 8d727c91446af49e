"""Pins of the router oracle (CPU): a hand-worked fixture, pure-Python brute
force, closed forms, and planted mistakes that must each fail a pin."""
import math
import os
import types

import numpy as np
import pytest
from scipy.special import softmax

import oracle as O

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "bmoe_router.py")


def _load_hand(golden_dir):
    rows = {"x": [], "w": [], "ids": [], "gates": []}
    with open(os.path.join(golden_dir, "router_hand.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            key, *vals = line.split()
            rows[key].append([float(v) for v in vals])
    return {k: np.array(v) for k, v in rows.items()}


def pin_hand_fixture(R, golden_dir):
    h = _load_hand(golden_dir)
    ids, gates, _ = R.router(h["x"], h["w"], 2)
    assert np.array_equal(ids, h["ids"].astype(np.int32))
    assert np.allclose(gates, h["gates"], rtol=0, atol=1e-12)


def _brute(x, w, k):
    """Pure-Python loops: dot products, then k rounds of 'largest not yet
    taken, lowest id on ties', then exp / sum."""
    T, d = len(x), len(x[0])
    N = len(w)
    ids, gates = [], []
    for t in range(T):
        lg = [sum(float(x[t][c]) * float(w[e][c]) for c in range(d)) for e in range(N)]
        taken = []
        for _ in range(k):
            best = None
            for e in range(N):
                if e in taken:
                    continue
                if best is None or lg[e] > lg[best]:
                    best = e
            taken.append(best)
        ex = [math.exp(lg[e] - lg[taken[0]]) for e in taken]
        s = sum(ex)
        ids.append(taken)
        gates.append([v / s for v in ex])
    return np.array(ids, dtype=np.int32), np.array(gates)


def pin_bruteforce(R):
    rng = np.random.default_rng(3)
    for d, N in [(4, 5), (8, 3), (2, 7)]:
        x = rng.standard_normal((6, d))
        w = rng.standard_normal((N, d))
        for k in range(1, N + 1):
            ids, gates, _ = R.router(x, w, k)
            bi, bg = _brute(x, w, k)
            assert np.array_equal(ids, bi)
            assert np.allclose(gates, bg, rtol=0, atol=1e-12)


def pin_full_sort(R):
    """k = N: ids are every expert by descending logit and the gates are the
    softmax over all N logits (library routine)."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((9, 6))
    w = rng.standard_normal((5, 6))
    ids, gates, logits = R.router(x, w, 5)
    full = x @ w.T
    for t in range(9):
        assert sorted(ids[t].tolist()) == list(range(5))
        assert np.all(np.diff(full[t][ids[t]]) <= 0)
        ref = softmax(full[t])[ids[t]]
        assert np.allclose(gates[t], ref, rtol=0, atol=1e-12)


def pin_basis_rows(R):
    """Router rows that are unit vectors e_{p(e)} read coordinates: logit
    [t][e] = x[t][p(e)] exactly (a non-symmetric permutation, N = d)."""
    p = np.array([2, 0, 3, 1])
    w = np.eye(4)[p]
    x = np.random.default_rng(5).standard_normal((7, 4))
    _, _, logits = R.router(x, w, 1)
    assert np.array_equal(logits, x[:, p])
    ids, gates, _ = R.router(x, w, 1)
    assert np.array_equal(ids[:, 0], np.argmax(x[:, p], axis=1))
    assert np.array_equal(gates, np.ones((7, 1)))


def pin_ties_lower_id(R):
    """Duplicate router rows give equal logits; the lower id comes first."""
    w = np.array([[1.0, 0.0], [0.5, 0.5], [1.0, 0.0], [0.5, 0.5]])
    x = np.array([[2.0, 1.0], [1.0, 3.0]])
    ids, gates, _ = R.router(x, w, 3)
    assert ids.tolist() == [[0, 2, 1], [1, 3, 0]]
    assert gates[0][0] == gates[0][1] and gates[1][0] == gates[1][1]


PINS = [pin_bruteforce, pin_full_sort, pin_basis_rows, pin_ties_lower_id]


def test_hand_fixture(golden_dir):
    pin_hand_fixture(O, golden_dir)


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_router_pins(pin):
    pin(O)


def test_gates_sum_to_one_and_descend():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((50, 16))
    w = rng.standard_normal((12, 16))
    for k in (1, 3, 12):
        _, gates, _ = O.router(x, w, k)
        assert np.allclose(gates.sum(axis=1), 1.0, atol=1e-14)
        assert np.all(np.diff(gates, axis=1) <= 0) and np.all(gates > 0)


MUTANTS = {
    "ascending": [("np.argsort(-logits", "np.argsort(logits")],
    "ties_to_higher_id": [('order = np.argsort(-logits, axis=1, kind="stable")',
                           'order = N - 1 - np.argsort(-logits[:, ::-1], axis=1, kind="stable")')],
    "softmax_over_all_experts": [
        ("    ex = np.exp(chosen - chosen[:, :1])\n    gates = ex / ex.sum(axis=1, keepdims=True)",
         "    ex = np.exp(logits - logits.max(axis=1, keepdims=True))\n"
         "    gates = np.take_along_axis(ex / ex.sum(axis=1, keepdims=True),"
         " ids.astype(np.int64), axis=1)")],
    "router_not_transposed": [("@ np.asarray(w_router, dtype=np.float64).T",
                               "@ np.asarray(w_router, dtype=np.float64)")],
    "gates_not_normalised": [("    gates = ex / ex.sum(axis=1, keepdims=True)", "    gates = ex")],
}


def _mutant(edits):
    src = open(SRC).read()
    for old, new in edits:
        assert old in src, old
        src = src.replace(old, new)
    mod = types.ModuleType("bmoe_router_mutant")
    exec(compile(src, "bmoe_router_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", list(MUTANTS))
def test_each_planted_router_mistake_is_caught(name, golden_dir):
    mutant = _mutant(MUTANTS[name])  # outside the try: a stale edit must fail loudly
    caught = 0
    for pin in PINS + [lambda R: pin_hand_fixture(R, golden_dir)]:
        try:
            pin(mutant)
        except Exception:
            caught += 1
    assert caught >= 1, f"mutant {name} passed every pin"
