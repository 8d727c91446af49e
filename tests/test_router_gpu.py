"""GPU parity of bmoe_router against the fp64 router oracle.

Logits are compared element by element within an fp32-accumulation bound.
The expert choice is an integer decided by floating point, so it is checked
twice: bit-exact against the oracle's selection run on the kernel's own fp32
logits (same precision on both sides), and against the fp64 oracle on every
token whose choice is unique by more than twice that token's largest logit
error."""
import numpy as np
import pytest
import torch

import oracle as O
from butterfly_rotated_ternary_amd import bmoe
from butterfly_rotated_ternary_amd import workloads as W
from devinputs import to_device

pytestmark = pytest.mark.gpu

# |logit error| <= LOGIT_TOL * sum_c |x_c w_c|: the products of bf16 (or fp32)
# values are summed in fp32 over at most 4096 terms.
LOGIT_TOL = 1e-4
GATE_TOL = 1e-5


def _w_dev(inp, rw):
    if inp.dtype == "bf16":
        return torch.from_numpy(rw.w_bits.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(rw.w).cuda()


def _x_dev(inp):
    if inp.dtype == "bf16":
        return torch.from_numpy(inp.x_bits.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(inp.x).cuda()


def _check(x, w, k, ids, gates, logits, rows=None):
    """x, w fp32 exact inputs (x possibly a row sample); ids/gates/logits the
    kernel's outputs for those rows."""
    ref = O.router_logits(x, w)
    scale = np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T
    bound = LOGIT_TOL * scale + 1e-30
    assert (np.abs(logits - ref) <= bound).all(), float((np.abs(logits - ref) / bound).max())
    kid, kg, _ = O.router(None, None, k, logits=logits)
    assert np.array_equal(ids, kid)
    assert np.abs(gates - kg).max() <= GATE_TOL
    oid, og, _ = O.router(x, w, k)
    N = w.shape[0]
    srt = -np.sort(-ref, axis=1)[:, :min(k + 1, N)]
    gaps = -np.diff(srt, axis=1)
    # every kernel logit of token t is within eps_t of the exact one, so where
    # the exact top-(k+1) gaps exceed 2 eps_t the kernel's order is the exact one
    eps = np.abs(logits - ref).max(axis=1, keepdims=True)
    unique = (gaps > 2 * eps).all(axis=1)
    assert np.array_equal(ids[unique], oid[unique])
    assert np.abs(gates[unique] - og[unique]).max(initial=0.0) <= 1e-4
    return unique.mean()


def _run(inp, rw, k=None, want_logits=True):
    k = inp.k if k is None else k
    ids, gates, logits = bmoe.route(_x_dev(inp), _w_dev(inp, rw), k, want_logits=True)
    torch.cuda.synchronize()
    return (ids.cpu().numpy(), gates.cpu().numpy().astype(np.float64),
            logits.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("name,T", [
    ("tiny_d64_e8_top2_f32", 256),
    ("d512_e64_top2_bf16", 1000),
    ("d512_e256_top2_zipf_bf16", 777),
    ("d2048_e64_top2_outliers_bf16", 300),
    ("d4096_e256_top4_bf16", 129),
])
def test_router_matches_oracle(name, T):
    inp = W.make_inputs(name, T=T)
    rw = W.make_router_weights(inp)
    print(f"[router] {name} T={T}", flush=True)
    ids, gates, logits = _run(inp, rw)
    frac = _check(inp.x, rw.w, inp.k, ids, gates, logits)
    assert frac > 0.9


@pytest.mark.parametrize("d,N,k,T,dtype", [
    (16, 8, 3, 5, "bf16"), (32, 70, 5, 65, "bf16"), (64, 1, 1, 3, "f32"), (128, 130, 64, 70, "bf16"),
    (256, 4096, 64, 20, "bf16"), (512, 100, 7, 1, "f32"), (1024, 600, 8, 64, "bf16"),
    # large enough for the LDS-tiled logits (ragged in tokens and experts)
    (512, 130, 4, 32700, "bf16"), (64, 257, 2, 16390, "bf16"), (128, 33, 3, 33000, "bf16"),
])
def test_router_edge_shapes(d, N, k, T, dtype):
    inp = W.make_inputs("tiny_d64_e8_top2_f32", T=T, d=d, N=N, k=min(k, N), dtype=dtype,
                        seed=77 + d + N)
    rw = W.make_router_weights(inp, seed=5 + N)
    print(f"[router] d={d} N={N} k={k} T={T} {dtype}", flush=True)
    ids, gates, logits = _run(inp, rw, k=k)
    _check(inp.x, rw.w, k, ids, gates, logits)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_router_ties_go_to_lower_id(dtype):
    inp = W.make_inputs("tiny_d64_e8_top2_f32", T=37, d=64, N=8, k=2, dtype=dtype, seed=3)
    rw = W.make_router_weights(inp, seed=9)
    # experts 5, 6, 7 repeat experts 1, 3, 0 exactly: equal logits on the GPU too
    for dup, src in ((5, 1), (6, 3), (7, 0)):
        rw.w[dup] = rw.w[src]
        if rw.w_bits is not None:
            rw.w_bits[dup] = rw.w_bits[src]
    ids, gates, logits = _run(inp, rw, k=8)
    for dup, src in ((5, 1), (6, 3), (7, 0)):
        assert np.array_equal(logits[:, dup], logits[:, src])
        pos = {e: np.argmax(ids == e, axis=1) for e in (dup, src)}
        assert (pos[src] < pos[dup]).all()
    _check(inp.x, rw.w, 8, ids, gates, logits)


@pytest.mark.parametrize("name", ["d512_e64_top2_bf16", "d4096_e256_top4_bf16"])
def test_router_full_size_sampled(name):
    inp = W.make_inputs(name)
    rw = W.make_router_weights(inp)
    print(f"[router] full {name}", flush=True)
    ids, gates, logits = _run(inp, rw)
    rows = np.unique(np.concatenate([np.random.default_rng(1).choice(inp.T, 400, replace=False),
                                     np.arange(inp.T - 40, inp.T)]))
    frac = _check(inp.x[rows], rw.w, inp.k, ids[rows], gates[rows], logits[rows])
    assert frac > 0.9


def test_router_feeds_forward():
    """ids and gates from the router drive bmoe_forward directly; the result
    matches the forward oracle run with those ids and gates."""
    inp = W.make_inputs("d512_e64_top2_bf16", T=300)
    rw = W.make_router_weights(inp)
    dev = to_device(inp)
    ids, gates = bmoe.route(dev["x"], _w_dev(inp, rw), inp.k)
    y = bmoe.forward(dev["x"], ids, gates, dev["theta"], dev["phi"], dev["w_packed"],
                     dev["alpha"])
    torch.cuda.synchronize()
    ref = O.forward(inp.x, ids.cpu().numpy(), gates.cpu().numpy(), inp.theta, inp.phi, inp.w,
                    inp.alpha)
    assert O.max_rel_err(y.float().cpu().numpy().astype(np.float64), ref) <= 2e-2


def test_router_timed_matches_untimed_and_rejects_large_k():
    import ctypes
    inp = W.make_inputs("d512_e64_top2_bf16", T=200)
    rw = W.make_router_weights(inp)
    x, w = _x_dev(inp), _w_dev(inp, rw)
    ids0, gates0, lg0 = bmoe.route(x, w, 2, want_logits=True)
    ids1 = torch.empty_like(ids0)
    gates1 = torch.empty_like(gates0)
    lg1 = torch.empty_like(lg0)
    hip = ctypes.CDLL("libamdhip64.so")
    evs = []
    for _ in range(4):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    rc = bmoe.bmoe_router_timed(bmoe.BMOE_BF16, inp.T, inp.d, inp.N, 2, x, w, ids1, gates1,
                                logits=lg1, events=evs)
    assert rc == 0
    torch.cuda.synchronize()
    for e in evs:
        hip.hipEventDestroy(ctypes.c_void_p(e))
    assert torch.equal(ids0, ids1) and torch.equal(gates0, gates1) and torch.equal(lg0, lg1)
    assert bmoe.bmoe_router(bmoe.BMOE_BF16, inp.T, inp.d, inp.N, 65, x, w, ids1, gates1,
                            logits=lg1) == 2
