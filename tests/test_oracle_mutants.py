"""The oracle's pins are strong enough: each plausible mistake, planted in a
copy of the oracle (on the CPU), makes at least one pin fail."""
import os
import types

import pytest

import test_oracle as P

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "bmoe_oracle.py")

MUTANTS = {
    "givens_sign": [("X[:, i] = c * xi - sn * xj", "X[:, i] = c * xi + sn * xj"),
                    ("X[:, j] = sn * xi + c * xj", "X[:, j] = -sn * xi + c * xj")],
    "stage_order": [("stages = range(L - 1, -1, -1) if transpose else range(L)",
                     "stages = range(L) if transpose else range(L - 1, -1, -1)")],
    "transpose_keeps_angle": [("        if transpose:\n            sn = -sn\n", "")],
    "substrate_transposed": [("H = float(alpha) * (Z @ W64.T)", "H = float(alpha) * (Z @ W64)")],
    "alpha_dropped": [("H = float(alpha) * (Z @ W64.T)", "H = (Z @ W64.T)")],
    "pair_index": [("high = (p >> s) << (s + 1)", "high = (p >> (s + 1)) << (s + 1)")],
    "gate_index": [("y += g[:, j:j + 1] * U", "y += g[:, 0:1] * U")],
    "sides_swapped": [("Z = apply_butterfly(theta[e]", "Z = apply_butterfly(phi[e]"),
                      ("U[a:b] = apply_butterfly(phi[e]", "U[a:b] = apply_butterfly(theta[e]")],
    "route_unstable": [("for r, e in enumerate(flat):", "for r, e in reversed(list(enumerate(flat))):")],
    "pack_bits": [("return 16 + 2 * j, 17 + 2 * j", "return 17 + 2 * j, 16 + 2 * j")],
    "token_of_row": [("x[rows // k]", "x[rows % x.shape[0]]")],
}

PINS = [
    lambda: P.test_stage_pairs_enumeration(),
    lambda: P.test_d2_is_a_single_givens_rotation(),
    lambda: P.test_zero_angles_give_identity_exactly(),
    lambda: P.test_stagewise_apply_matches_dense_matrix(8),
    lambda: P.test_uniform_stage_angles_give_kronecker_product(8),
    lambda: P.test_stage_order_fixture(GOLDEN),
    lambda: P.test_factored_equals_materialized(16),
    lambda: P.test_factored_equals_bruteforce(8, 2),
    lambda: P.test_hand_forward_fixture(GOLDEN),
    lambda: P.test_zero_angles_reduce_to_plain_ternary_matmul(),
    lambda: P.test_signed_permutation_substrate_orientation(),
    lambda: P.test_input_side_is_transposed_butterfly(),
    lambda: P.test_output_side_is_plain_butterfly(),
    lambda: P.test_route_is_stable_argsort("zipf"),
    lambda: P.test_pack_golden(GOLDEN),
]


def _mutant(edits):
    src = open(SRC).read()
    for old, new in edits:
        assert old in src, old
        src = src.replace(old, new)
    mod = types.ModuleType("bmoe_oracle_mutant")
    exec(compile(src, "bmoe_oracle_mutant", "exec"), mod.__dict__)
    return mod


def test_pins_pass_on_the_real_oracle():
    for pin in PINS:
        pin()


@pytest.mark.parametrize("name", list(MUTANTS))
def test_each_planted_mistake_is_caught(name, monkeypatch):
    monkeypatch.setattr(P, "O", _mutant(MUTANTS[name]))
    caught = 0
    for pin in PINS:
        try:
            pin()
        except Exception:
            caught += 1
    assert caught >= 1, f"mutant {name} passed every pin"
