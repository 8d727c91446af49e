"""Pins of the backward oracle (CPU). Each gradient is checked against central
finite differences of the forward oracle, an independent route to the same
numbers, and against closed forms; planted mistakes in a copy of the backward
oracle must fail at least one pin."""
import os
import types

import numpy as np
import pytest

import oracle as O
from oracle import bmoe_oracle as F

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "bmoe_backward.py")


def _case(d, N=3, k=2, T=5, seed=0):
    rng = np.random.default_rng(seed)
    L = F.n_stages(d)
    ids = np.stack([rng.permutation(N)[:k] for _ in range(T)]).astype(np.int32)
    return dict(
        x=rng.standard_normal((T, d)),
        ids=ids,
        gates=rng.uniform(0.1, 1.0, (T, k)),
        theta=rng.uniform(-np.pi, np.pi, (N, L, d // 2)),
        phi=rng.uniform(-np.pi, np.pi, (N, L, d // 2)),
        w=rng.integers(-1, 2, (d, d)).astype(np.float64),
        alpha=0.37,
        dy=rng.standard_normal((T, d)),
    )


def _fd(c, key, h=1e-6):
    """Central differences of sum(dy * y) with respect to every entry of c[key]."""
    base = np.array(c[key], dtype=np.float64)
    out = np.zeros_like(base)
    it = np.nditer(base, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        for sgn in (1.0, -1.0):
            pert = base.copy()
            pert[idx] += sgn * h
            cc = dict(c)
            cc[key] = pert
            out[idx] += sgn * O.backward_loss(**cc) / (2 * h)
    return out


GRADS = [("x", "dx"), ("gates", "dgates"), ("theta", "dtheta"), ("phi", "dphi"), ("w", "dw")]


def _check_fd(B, d, seed=0):
    c = _case(d, seed=seed)
    g = B.backward(**c)
    for key, gk in GRADS:
        ref = _fd(c, key)
        scale = max(1.0, np.abs(ref).max())
        assert np.abs(g[gk] - ref).max() <= 1e-6 * scale, (d, gk)


@pytest.mark.parametrize("d", [2, 4, 8, 16])
def test_gradients_match_finite_differences(d):
    _check_fd(O, d)


def test_zero_angles_closed_form():
    """theta = phi = 0: every stage is the identity, so dx_t = alpha sum_j g_j
    W^T dy_t, dg_tj = <dy_t, alpha W x_t>, dW = alpha sum_r g_r dy_t x_t^T."""
    c = _case(16, seed=3)
    c["theta"] = np.zeros_like(c["theta"])
    c["phi"] = np.zeros_like(c["phi"])
    g = O.backward(**c)
    a, W, x, dy, gt = c["alpha"], c["w"], c["x"], c["dy"], c["gates"]
    dx = a * gt.sum(axis=1)[:, None] * (dy @ W)
    dg = np.repeat(((dy * (a * x @ W.T)).sum(axis=1))[:, None], c["ids"].shape[1], axis=1)
    dw = a * (dy * gt.sum(axis=1)[:, None]).T @ x
    assert np.allclose(g["dx"], dx, atol=1e-12)
    assert np.allclose(g["dgates"], dg, atol=1e-12)
    assert np.allclose(g["dw"], dw, atol=1e-12)


def test_linear_in_dy():
    c = _case(8, seed=5)
    g1 = O.backward(**c)
    c2 = dict(c)
    c2["dy"] = -2.5 * c["dy"]
    g2 = O.backward(**c2)
    for _, gk in GRADS:
        assert np.allclose(g2[gk], -2.5 * g1[gk], atol=1e-12)


MUTANTS = {
    "input_side_angle_sign": [("    return dX, sign * d_eff", "    return dX, d_eff")],
    "stage_input_grad_sign": [("    dX[:, i] = c * gi + sn * gj", "    dX[:, i] = c * gi - sn * gj")],
    "dz_uses_w_transposed": [("        G = a64 * (dH @ W)", "        G = a64 * (dH @ W.T)")],
    "dw_drops_alpha": [("        dw += a64 * (dH.T @ Z)", "        dw += dH.T @ Z")],
    "gate_grad_from_h": [("        dg[rows] = (Dy * U).sum(axis=1)", "        dg[rows] = (Dy * H).sum(axis=1)")],
    "output_side_order": [("        for s, Vin in reversed(out_side):", "        for s, Vin in out_side:")],
}


def _mutant(edits):
    src = open(SRC).read()
    for old, new in edits:
        assert old in src, old
        src = src.replace(old, new)
    src = src.replace("from .bmoe_oracle import n_stages, route, stage_pairs",
                      "from oracle.bmoe_oracle import n_stages, route, stage_pairs")
    src = src.replace("    from .bmoe_oracle import forward", "    from oracle.bmoe_oracle import forward")
    mod = types.ModuleType("bmoe_backward_mutant")
    exec(compile(src, "bmoe_backward_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", list(MUTANTS))
def test_each_planted_backward_mistake_is_caught(name):
    mutant = _mutant(MUTANTS[name])  # outside raises(): a stale edit must fail loudly
    with pytest.raises(AssertionError):
        _check_fd(mutant, 4)
