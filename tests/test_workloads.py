"""The seeded input generator: shapes and distributions of each workload."""
import numpy as np
import pytest
import torch

from butterfly_rotated_ternary_amd import workloads as W


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_shapes_and_types(name):
    cfg = W.WORKLOADS[name]
    inp = W.make_inputs(name, T=64)
    d, N, k = cfg["d"], cfg["N"], cfg["k"]
    L = W.log2_exact(d)
    assert inp.x.shape == (64, d) and inp.x.dtype == np.float32
    assert inp.ids.shape == (64, k) and inp.ids.dtype == np.int32
    assert inp.gates.shape == (64, k) and inp.gates.dtype == np.float32
    assert inp.theta.shape == (N, L, d // 2) and inp.theta.dtype == np.float32
    assert inp.phi.shape == (N, L, d // 2)
    assert inp.w.shape == (d, d) and inp.w.dtype == np.int8
    assert np.isin(inp.w, (-1, 0, 1)).all()
    assert inp.alpha == np.float32(1 / np.sqrt(d))
    assert (np.abs(inp.theta) <= np.pi).all() and (np.abs(inp.phi) <= np.pi).all()
    # k distinct experts per token, all in range
    assert (inp.ids >= 0).all() and (inp.ids < N).all()
    srt = np.sort(inp.ids, axis=1)
    assert (np.diff(srt, axis=1) > 0).all()
    np.testing.assert_allclose(inp.gates.sum(axis=1), 1.0, rtol=1e-6)
    assert (inp.gates > 0).all()
    if cfg["dtype"] == "bf16":
        assert inp.x_bits.shape == (64, d) and inp.x_bits.dtype == np.uint16


def test_deterministic_per_seed():
    a = W.make_inputs(W.HEADLINE, T=32)
    b = W.make_inputs(W.HEADLINE, T=32)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.ids, b.ids)
    assert np.array_equal(a.theta, b.theta) and np.array_equal(a.w, b.w)
    c = W.make_inputs(W.HEADLINE, T=32, seed=7)
    assert not np.array_equal(a.x, c.x)


@pytest.mark.parametrize("name,dens", [("d512_e64_top2_bf16", 2 / 3),
                                       ("d2048_e64_top2_outliers_bf16", 0.5)])
def test_density(name, dens):
    inp = W.make_inputs(name, T=1)
    nz = np.count_nonzero(inp.w) / inp.w.size
    assert abs(nz - dens) < 0.005
    pos = np.count_nonzero(inp.w == 1) / inp.w.size
    assert abs(pos - dens / 2) < 0.005


def test_zipf_skew():
    inp = W.make_inputs("d512_e256_top2_zipf_bf16")
    first = inp.ids[:, 0]
    w = np.arange(1, 257, dtype=np.float64) ** -1.1
    p0 = w[0] / w.sum()
    assert abs(p0 - 0.2065) < 1e-3
    assert abs(np.mean(first == 0) - p0) < 0.012
    counts = np.bincount(inp.ids.reshape(-1), minlength=256)
    assert counts[0] == counts.max()
    assert counts[-32:].mean() < 40   # thin tail


def test_outlier_channels():
    inp = W.make_inputs("d2048_e64_top2_outliers_bf16", T=256)
    ch = inp.outlier_channels
    assert ch.size == 20 and np.unique(ch).size == 20
    big = np.abs(inp.x[:, ch]).mean()
    rest = np.abs(np.delete(inp.x, ch, axis=1)).mean()
    assert 15 < big / rest < 25


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 37
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 65504.0]   # ties and a large value
    bits = W.bf16_round_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    back = W.bf16_bits_to_f32(bits)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())
