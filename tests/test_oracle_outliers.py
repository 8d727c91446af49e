"""Pins of the outlier-measurement oracle (CPU): a hand-worked quantiser
fixture, closed forms, the input-side rotation through the pinned forward
oracle, and planted mistakes that must each fail a pin."""
import os
import types

import numpy as np
import pytest

import oracle as O
from oracle import bmoe_outliers as Q

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "bmoe_outliers.py")


def _hand(golden_dir):
    errs, v, crest = [], None, None
    with open(os.path.join(golden_dir, "quant_error_hand.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            key, *vals = line.split()
            if key == "v":
                v = np.array([float(a) for a in vals])
            elif key == "err":
                errs.append((int(vals[0]), int(vals[1]), float(vals[2])))
            else:
                crest = float(vals[0])
    return v, errs, crest


def pin_hand(M, golden_dir):
    v, errs, crest = _hand(golden_dir)
    V = np.stack([v, np.zeros_like(v)])
    for mode, m, ref in errs:
        got = M.quant_error(V, m, mode)
        assert abs(got[0] - ref) < 1e-12 and got[1] == 0.0
    c = M.crest_factor(V)
    assert abs(c[0] - crest) < 1e-12 and c[1] == 0.0


def pin_closed_forms(M):
    rng = np.random.default_rng(1)
    # values already on the grid s * {-m..m} quantise exactly
    m = 7
    g = rng.integers(-m, m + 1, size=(5, 32)).astype(np.float64)
    g[:, 0] = m                        # fixes max|v| = m * s with s = 0.37
    assert np.all(M.quant_error(0.37 * g, m, 0) < 1e-15)
    # a constant row is exact for absmax and absmean alike
    c = np.full((3, 16), -2.5)
    assert np.all(M.quant_error(c, 1, 0) < 1e-15) and np.all(M.quant_error(c, 1, 1) < 1e-15)
    # the error never exceeds (s/2) sqrt(d) / ||v|| for absmax, and falls with m
    V = rng.standard_normal((20, 64))
    e8, e4 = M.quant_error(V, 127, 0), M.quant_error(V, 7, 0)
    bound = (np.abs(V).max(axis=1) / 127 / 2) * 8 / np.linalg.norm(V, axis=1)
    assert np.all(e8 <= bound + 1e-15) and np.all(e8 < e4)
    # crest factor of a one-hot row is sqrt(d)
    oh = np.zeros((1, 64)); oh[0, 5] = -3.0
    assert abs(M.crest_factor(oh)[0] - 8.0) < 1e-12


def pin_rotate_in(M):
    """rotate_in equals the pinned forward with W_base = I, phi = 0, alpha = 1
    and k = 1 (gate 1), and keeps every row's norm."""
    rng = np.random.default_rng(2)
    d, N, T = 16, 3, 7
    L = O.n_stages(d)
    theta = rng.uniform(-np.pi, np.pi, (N, L, d // 2))
    x = rng.standard_normal((T, d))
    ids = rng.integers(0, N, size=(T, 1)).astype(np.int32)
    z = M.rotate_in(x, ids, theta)
    y = O.forward(x, ids, np.ones((T, 1)), theta, np.zeros_like(theta),
                  np.eye(d, dtype=np.int8), 1.0)
    assert np.allclose(z, y, atol=1e-12)
    ids2 = rng.integers(0, N, size=(T, 2)).astype(np.int32)
    z2 = M.rotate_in(x, ids2, theta)
    assert np.allclose(np.linalg.norm(z2, axis=1), np.repeat(np.linalg.norm(x, axis=1), 2))
    for t in range(T):
        for j in range(2):
            ref = O.butterfly_matrix(theta[ids2[t, j]]).T @ x[t]
            assert np.allclose(z2[t * 2 + j], ref, atol=1e-12)


PINS = [pin_closed_forms, pin_rotate_in]


def test_hand_fixture(golden_dir):
    pin_hand(Q, golden_dir)


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_outlier_pins(pin):
    pin(Q)


MUTANTS = {
    "scale_uses_rms": [("s = a.max(axis=1) / m if mode == 0", "s = np.sqrt((V ** 2).mean(axis=1)) / m if mode == 0")],
    "no_clip": [("q = np.clip(np.rint(V[nz] / s[nz, None]), -m, m) * s[nz, None]",
                 "q = np.rint(V[nz] / s[nz, None]) * s[nz, None]")],
    "floor_not_round": [("np.rint(V[nz] / s[nz, None])", "np.floor(V[nz] / s[nz, None])")],
    "error_not_relative": [("/ (V[nz] ** 2).sum(axis=1))", "/ V.shape[1])")],
    "rotation_not_transposed": [("transpose=True", "transpose=False")],
    "row_order": [("out[rows * k + j]", "out[j * T + rows]")],
}


def _mutant(edits):
    src = open(SRC).read()
    for old, new in edits:
        assert old in src, old
        src = src.replace(old, new)
    src = src.replace("from .bmoe_oracle import apply_butterfly", "from oracle.bmoe_oracle import apply_butterfly")
    mod = types.ModuleType("bmoe_outliers_mutant")
    exec(compile(src, "bmoe_outliers_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", list(MUTANTS))
def test_each_planted_outlier_mistake_is_caught(name, golden_dir):
    mutant = _mutant(MUTANTS[name])  # outside the try: a stale edit must fail loudly
    caught = 0
    for pin in PINS + [lambda M: pin_hand(M, golden_dir)]:
        try:
            pin(mutant)
        except Exception:
            caught += 1
    assert caught >= 1, f"mutant {name} passed every pin"
