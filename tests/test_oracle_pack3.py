"""Pins of the base-3 storage oracle (CPU): a hand-worked fixture, the
bijection between bytes 0..242 and five ternary digits, closed forms, and
planted mistakes that must each fail a pin."""
import itertools
import os
import types

import numpy as np
import pytest

from oracle import bmoe_pack3 as P3

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "bmoe_pack3.py")


def _hand(golden_dir):
    w, b = [], None
    with open(os.path.join(golden_dir, "pack3_d4.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            key, *vals = line.split()
            if key == "w":
                w.append([int(v) for v in vals])
            else:
                b = [int(v) for v in vals]
    return np.array(w, dtype=np.int8), np.array(b, dtype=np.uint8)


def pin_hand(M, golden_dir):
    w, b = _hand(golden_dir)
    assert np.array_equal(M.pack_ternary_b3(w), b)
    assert np.array_equal(M.unpack_ternary_b3(b, 4), w)


def pin_bijection(M):
    """Every 5-digit ternary tuple gets its own byte in 0..242, and decoding
    inverts it: d = 5 is not a power of two, but the stream rule is the same,
    so use d*d = 25 entries (five bytes) per tuple check."""
    seen = set()
    for tup in itertools.product((-1, 0, 1), repeat=5):
        w = np.zeros((5, 5), dtype=np.int8)
        w[0] = tup
        b = M.pack_ternary_b3(w)
        assert b.shape == (5,)
        v = int(b[0])
        assert 0 <= v <= 242
        assert v == sum((t + 1) * 3 ** i for i, t in enumerate(tup))
        seen.add(v)
        assert np.array_equal(M.unpack_ternary_b3(b, 5), w)
    assert seen == set(range(243))


def pin_zero_and_size(M):
    for d in (16, 64, 512):
        w = np.zeros((d, d), dtype=np.int8)
        b = M.pack_ternary_b3(w)
        assert b.size == -(-d * d // 5)
        assert (b == 121).all()          # every digit 1: 1 + 3 + 9 + 27 + 81
        assert 8 * b.size / (d * d) < 1.6 + 8 / (d * d)


def pin_round_trip(M):
    rng = np.random.default_rng(2)
    for d in (16, 32, 128):
        w = rng.integers(-1, 2, size=(d, d)).astype(np.int8)
        assert np.array_equal(M.unpack_ternary_b3(M.pack_ternary_b3(w), d), w)


PINS = [pin_bijection, pin_zero_and_size, pin_round_trip]


def test_hand_fixture(golden_dir):
    pin_hand(P3, golden_dir)


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pack3_pins(pin):
    pin(P3)


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        P3.pack_ternary_b3(np.full((4, 4), 2, dtype=np.int8))
    with pytest.raises(ValueError):
        P3.unpack_ternary_b3(np.full(4, 243, dtype=np.uint8), 4)


MUTANTS = {
    "digit_order_reversed": [("out += digits[:, i] * 3 ** i", "out += digits[:, i] * 3 ** (4 - i)")],
    "no_offset": [("flat = w.reshape(-1).astype(np.int64) + 1", "flat = w.reshape(-1).astype(np.int64) % 3")],
    "pad_digit_zero": [("digits = np.ones(n * 5, dtype=np.int64)", "digits = np.zeros(n * 5, dtype=np.int64)")],
    "base_four": [("out += digits[:, i] * 3 ** i", "out += digits[:, i] * 4 ** i")],
    "decode_order": [("        digits[:, i] = rest % 3\n", "        digits[:, 4 - i] = rest % 3\n")],
}


def _mutant(edits):
    src = open(SRC).read()
    for old, new in edits:
        assert old in src, old
        src = src.replace(old, new)
    mod = types.ModuleType("bmoe_pack3_mutant")
    exec(compile(src, "bmoe_pack3_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", list(MUTANTS))
def test_each_planted_pack3_mistake_is_caught(name, golden_dir):
    mutant = _mutant(MUTANTS[name])  # outside the try: a stale edit must fail loudly
    caught = 0
    for pin in PINS + [lambda M: pin_hand(M, golden_dir)]:
        try:
            pin(mutant)
        except Exception:
            caught += 1
    assert caught >= 1, f"mutant {name} passed every pin"
