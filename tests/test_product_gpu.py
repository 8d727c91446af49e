"""The shared-substrate product on its own (bmoe_product): H = alpha Z W^T
for the 2-bit words and for the base-3 stream (ButterflyMoE gist.science
summary, §2.1 stores W_base at 1.58 bits per weight; §2.3 the product step).
The two formats must give bit-identical H, and H must match the fp64
definition alpha * Z @ W^T per row within the bf16 bar (the product's
accumulation is fp32 over exact ternary terms; H is rounded to bf16)."""
import numpy as np
import pytest
import torch

import oracle as O
from butterfly_rotated_ternary_amd import bmoe
from butterfly_rotated_ternary_amd import workloads as W

pytestmark = pytest.mark.gpu


def _inputs(M, d, seed, density=2.0 / 3.0):
    rng = np.random.default_rng(seed)
    z32 = rng.standard_normal((M, d)).astype(np.float32)
    zbits = W.bf16_round_bits(z32)
    p = density / 2
    w = rng.choice(np.array([-1, 0, 1], dtype=np.int8), size=(d, d), p=[p, 1 - 2 * p, p])
    return W.bf16_bits_to_f32(zbits).astype(np.float64), zbits, w


@pytest.mark.parametrize("M,d", [(37, 128), (1000, 512), (8192, 512), (8229, 512), (300, 1024),
                                 (700, 4096)])
def test_product_formats_bit_identical_and_exact(M, d):
    z, zbits, w = _inputs(M, d, seed=M + d)
    print(f"[product] M={M} d={d}", flush=True)
    dev = torch.device("cuda")
    zt = torch.from_numpy(zbits.view(np.int16)).view(torch.bfloat16).to(dev)
    wt = torch.from_numpy(w).to(dev)
    w2 = bmoe.pack_ternary(wt)
    w3 = bmoe.pack_ternary_b3(wt)
    alpha = float(np.float32(1 / np.sqrt(d)))
    h2 = torch.empty_like(zt)
    h3 = torch.full_like(zt, float("nan"))
    assert bmoe.bmoe_product(M, d, zt, w2, bmoe.BMOE_W_2BIT, alpha, h2) == 0
    assert bmoe.bmoe_product(M, d, zt, w3, bmoe.BMOE_W_BASE3, alpha, h3) == 0
    torch.cuda.synchronize()
    assert torch.equal(h2, h3)
    ref = alpha * (z @ w.astype(np.float64).T)
    got = h2.float().cpu().numpy().astype(np.float64)
    err = O.max_rel_err(got, ref)
    print(f"  max rel err {err:.3e}", flush=True)
    assert err <= 2e-2


def test_product_rejects_bad_arguments():
    dev = torch.device("cuda")
    z = torch.zeros(4, 256, dtype=torch.bfloat16, device=dev)
    w = torch.zeros(256 * 16, dtype=torch.int32, device=dev)
    h = torch.empty_like(z)
    assert bmoe.bmoe_product(4, 192, z, w, bmoe.BMOE_W_2BIT, 1.0, h) == 2   # d not a power of 2
    assert bmoe.bmoe_product(4, 64, z, w, bmoe.BMOE_W_2BIT, 1.0, h) == 2    # d < 128
    assert bmoe.bmoe_product(4, 256, z, w, 7, 1.0, h) == 3                  # unknown format
    assert bmoe.bmoe_product(0, 256, z, w, bmoe.BMOE_W_2BIT, 1.0, h) == 0   # M = 0: no-op
