"""GPU parity of bmoe_backward against the fp64 backward oracle (same seeded
inputs, element by element). Bars: 1e-4 on the fp32 path, 2e-2 on the bf16
path, each applied per block so that a small block cannot hide under a large
one:

* dx per token, like the forward (largest error over the token's largest
  reference entry);
* dtheta and dphi per expert: the largest error over the expert's [L][d/2]
  block over that block's largest reference entry (experts without rows must
  come out exactly zero);
* dW per output row;
* dgates per routed row r = (t, j). A gate gradient is the dot product
  <dy_t, u_r> of d terms, which can cancel to nearly zero, where an error
  relative to the value itself is unbounded; it is taken relative to
  ||dy_t||_2 ||u_r||_2 / sqrt(d), the size of such a dot product (its RMS
  over random directions). ||u_r||_2 = ||alpha W_base z_r||_2 because
  B(phi) is orthogonal; the oracle's rotation gives z_r."""
import numpy as np
import pytest
import torch

import oracle as O
from butterfly_rotated_ternary_amd import bmoe
from butterfly_rotated_ternary_amd import workloads as W
from devinputs import to_device

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _dy(inp, seed):
    rng = np.random.default_rng(seed)
    dy = rng.standard_normal((inp.T, inp.d)).astype(np.float32)
    if inp.dtype == "bf16":
        bits = W.bf16_round_bits(dy)
        return W.bf16_bits_to_f32(bits), bits
    return dy, None


def _global_err(a, ref):
    m = np.abs(ref).max()
    return float(np.abs(a - ref).max() / m) if m > 0 else float(np.abs(a).max())


def _per_block_err(a, ref):
    """Largest over blocks (the leading axis) of max|a - ref| / max|ref| in
    the block; a block whose reference is all zero must be exactly zero."""
    a = a.reshape(a.shape[0], -1)
    ref = ref.reshape(ref.shape[0], -1)
    num = np.abs(a - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    zero = den == 0
    if np.any(zero):
        assert np.all(a[zero] == 0.0), "nonzero gradient where the reference is zero"
    return float((num[~zero] / den[~zero]).max()) if np.any(~zero) else 0.0


def _dgates_err(got, ref, inp, dy, toks=None):
    """Per routed row |got - ref| / (||dy_t|| ||u_r|| / sqrt(d))."""
    toks = np.arange(inp.T) if toks is None else toks
    W64 = inp.w.astype(np.float64)
    unorm = np.empty((toks.size, inp.k))
    for j in range(inp.k):
        e_col = inp.ids[toks, j]
        for e in np.unique(e_col):
            sel = np.nonzero(e_col == e)[0]
            z = O.apply_butterfly(inp.theta[e], inp.x[toks[sel]].astype(np.float64),
                                  transpose=True)
            unorm[sel, j] = np.linalg.norm(float(inp.alpha) * (z @ W64.T), axis=1)
    scale = np.linalg.norm(dy[toks].astype(np.float64), axis=1)[:, None] * unorm / np.sqrt(inp.d)
    num = np.abs(got - ref)
    assert np.all(num[scale == 0] == 0.0)
    return float((num[scale > 0] / scale[scale > 0]).max())


def _run(name, T, seed=11, **override):
    return _check_case(W.make_inputs(name, T=T, **override), seed)


def _check_case(inp, seed):
    name = inp.name
    dy, dy_bits = _dy(inp, seed)
    print(f"[backward] {name} T={inp.T} d={inp.d} N={inp.N} k={inp.k}", flush=True)
    dev = to_device(inp)
    if inp.dtype == "bf16":
        dyt = torch.from_numpy(dy_bits.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        dyt = torch.from_numpy(dy).cuda()
    g = bmoe.backward(dev["x"], dev["ids"], dev["gates"], dev["theta"], dev["phi"],
                      dev["w_packed"], dev["alpha"], dyt)
    torch.cuda.synchronize()
    ref = O.backward(inp.x, inp.ids, inp.gates, inp.theta, inp.phi, inp.w, inp.alpha, dy)
    got = {k: v.float().cpu().numpy().astype(np.float64) for k, v in g.items() if v is not None}
    errs = {
        "dx": O.max_rel_err(got["dx"], ref["dx"]),
        "dgates": _dgates_err(got["dgates"], ref["dgates"], inp, dy),
        "dtheta": _per_block_err(got["dtheta"], ref["dtheta"]),
        "dphi": _per_block_err(got["dphi"], ref["dphi"]),
        "dw": _per_block_err(got["dw"], ref["dw"]),
        "dgates_global": _global_err(got["dgates"], ref["dgates"]),
    }
    print("  " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v <= TOL[inp.dtype], (k, v)
    for v in got.values():
        assert np.isfinite(v).all()
    return got


@pytest.mark.parametrize("name,T", [
    ("tiny_d64_e8_top2_f32", 256),
    ("d512_e64_top2_bf16", 301),
    ("d512_e64_top2_bf16", 401),
    ("d512_e64_top2_bf16", 4103),  # substrate gradient: 16 row ranges, 15 x 544 rows + 46
    ("d512_e256_top2_zipf_bf16", 700),
    ("d2048_e64_top2_outliers_bf16", 97),
    ("d4096_e256_top4_bf16", 23),
])
def test_backward_matches_oracle(name, T):
    _run(name, T)


@pytest.mark.parametrize("d,N,k,T,dtype", [(16, 3, 2, 9, "f32"), (32, 5, 5, 4, "bf16"),
                                           (128, 70, 1, 150, "bf16"), (256, 2, 2, 129, "f32"),
                                           (256, 9, 3, 203, "bf16"), (1024, 3, 2, 40, "bf16")])
def test_backward_edge_shapes(d, N, k, T, dtype):
    # more than 64 rows per expert (several tiles), single-row experts, k = N
    _run("tiny_d64_e8_top2_f32", T, d=d, N=N, k=k, dtype=dtype, seed=900 + d)


def test_backward_dw_row_ranges_at_d2048():
    # 2200 routed rows: the d >= 2048 substrate-gradient kernel splits its
    # reduction over rows into 4 ranges, which the closing kernel sums
    _run("d2048_e64_top2_outliers_bf16", 1100, seed=17)


def test_backward_is_deterministic():
    inp = W.make_inputs(W.HEADLINE, T=200)
    dev = to_device(inp)
    dy = torch.randn(inp.T, inp.d, device="cuda").to(torch.bfloat16)
    a = bmoe.backward(dev["x"], dev["ids"], dev["gates"], dev["theta"], dev["phi"],
                      dev["w_packed"], dev["alpha"], dy)
    b = bmoe.backward(dev["x"], dev["ids"], dev["gates"], dev["theta"], dev["phi"],
                      dev["w_packed"], dev["alpha"], dy)
    torch.cuda.synchronize()
    for k in ("dx", "dgates", "dtheta", "dphi"):
        assert torch.equal(a[k], b[k]), k


def test_backward_rejects_d8192():
    assert bmoe.bmoe_backward_workspace_bytes(bmoe.BMOE_BF16, 4, 8192, 2, 1) == 0


def test_timed_backward_matches_untimed():
    import ctypes
    inp = W.make_inputs(W.HEADLINE, T=300)
    dev = to_device(inp)
    dy = torch.randn(inp.T, inp.d, device="cuda").to(torch.bfloat16)
    a = bmoe.backward(dev["x"], dev["ids"], dev["gates"], dev["theta"], dev["phi"],
                      dev["w_packed"], dev["alpha"], dy)
    b = {k: torch.empty_like(v) for k, v in a.items()}
    dt, T, d, N, k = bmoe.BMOE_BF16, inp.T, inp.d, inp.N, inp.k
    ws = torch.empty(bmoe.bmoe_backward_workspace_bytes(dt, T, d, N, k), dtype=torch.uint8,
                     device="cuda")
    hip = ctypes.CDLL("libamdhip64.so")
    nk = bmoe.bmoe_backward_kernel_count(dt, T, d, N, k)
    evs = []
    for _ in range(2 * nk):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    rc = bmoe.bmoe_backward_timed(dt, T, d, N, k, dev["x"], dev["ids"], dev["gates"],
                                  dev["theta"], dev["phi"], dev["w_packed"], dev["alpha"], dy,
                                  b["dx"], b["dgates"], b["dtheta"], b["dphi"], b["dw"], ws,
                                  events=evs)
    assert rc == 0
    torch.cuda.synchronize()
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    for i in range(nk):
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), evs[2 * i], evs[2 * i + 1]) == 0
        assert ms.value >= 0.0
    for e in evs:
        hip.hipEventDestroy(ctypes.c_void_p(e))
    for key in ("dx", "dgates", "dtheta", "dphi", "dw"):
        assert torch.equal(a[key], b[key]), key


def test_backward_one_expert_takes_every_row():
    inp = W.make_inputs("d512_e64_top2_bf16", T=333)
    inp.ids[:, 0] = 5                       # every token's first pick is expert 5
    inp.ids[:, 1] = np.where(inp.ids[:, 1] == 5, 6, inp.ids[:, 1])
    _check_case(inp, seed=21)


def test_backward_many_empty_experts():
    # 4096 experts, 9 tokens: almost every expert has no rows (zero angle gradients)
    inp = W.make_inputs("tiny_d64_e8_top2_f32", T=9, d=128, N=4096, k=3, dtype="bf16", seed=5)
    got = _check_case(inp, seed=22)
    used = np.unique(inp.ids)
    unused = np.setdiff1d(np.arange(4096), used)
    assert np.all(got["dtheta"][unused] == 0.0) and np.all(got["dphi"][unused] == 0.0)


def test_backward_single_token_all_experts():
    inp = W.make_inputs("tiny_d64_e8_top2_f32", T=1, d=4096, N=3, k=3, dtype="bf16", seed=6)
    _check_case(inp, seed=23)


def test_backward_empty_batch_is_a_noop():
    dev = torch.device("cuda")
    x = torch.empty(0, 256, dtype=torch.bfloat16, device=dev)
    g = bmoe.backward(x, torch.empty(0, 2, dtype=torch.int32, device=dev),
                      torch.empty(0, 2, device=dev), torch.zeros(4, 8, 128, device=dev),
                      torch.zeros(4, 8, 128, device=dev),
                      bmoe.pack_ternary(torch.zeros(256, 256, dtype=torch.int8, device=dev)),
                      1.0, torch.empty(0, 256, dtype=torch.bfloat16, device=dev))
    assert g["dx"].shape == (0, 256)


@pytest.mark.parametrize("name,T", [("tiny_d64_e8_top2_f32", 200), ("d512_e64_top2_bf16", 301),
                                    ("d2048_e64_top2_outliers_bf16", 90),
                                    ("d4096_e256_top4_bf16", 30), ("custom_d256", 157)])
def test_backward_after_kept_forward_is_bit_identical(name, T):
    """bmoe_forward_keep + bmoe_backward_kept gives exactly bmoe_backward's
    gradients (same kernels on the same inputs), and the kept forward's y
    matches the oracle. At d = 256 and 512 (bf16) both take Z and H from the
    fused kernel; the other shapes from the unfused path."""
    if name == "custom_d256":
        inp = W.make_inputs("custom", d=256, N=12, k=3, T=T, seed=256, dtype="bf16")
    else:
        inp = W.make_inputs(name, T=T)
    print(f"[kept] {name} T={T}", flush=True)
    dev = to_device(inp)
    dy = torch.randn(inp.T, inp.d, device="cuda").to(dev["x"].dtype)
    y, kept = bmoe.forward_keep(dev["x"], dev["ids"], dev["gates"], dev["theta"], dev["phi"],
                                dev["w_packed"], dev["alpha"])
    kept_copy = kept.clone()
    a = bmoe.backward_kept(dev["x"], dev["gates"], inp.N, dev["w_packed"], dev["alpha"], dy, kept)
    b = bmoe.backward(dev["x"], dev["ids"], dev["gates"], dev["theta"], dev["phi"],
                      dev["w_packed"], dev["alpha"], dy)
    torch.cuda.synchronize()
    for key in ("dx", "dgates", "dtheta", "dphi", "dw"):
        assert torch.equal(a[key], b[key]), key
    assert torch.equal(kept, kept_copy)      # the kept workspace is only read
    ref = O.forward(inp.x, inp.ids, inp.gates, inp.theta, inp.phi, inp.w, inp.alpha)
    assert O.max_rel_err(y.float().cpu().numpy().astype(np.float64), ref) <= TOL[inp.dtype]


def test_backward_kept_rejects_a_short_forward_workspace():
    inp = W.make_inputs("d512_e64_top2_bf16", T=64)
    dev = to_device(inp)
    dt, T, d, N, k = bmoe.BMOE_BF16, inp.T, inp.d, inp.N, inp.k
    n = bmoe.bmoe_forward_keep_workspace_bytes(dt, T, d, N, k)
    short = torch.empty(n - 256, dtype=torch.uint8, device="cuda")
    ws = torch.empty(bmoe.bmoe_backward_workspace_bytes(dt, T, d, N, k), dtype=torch.uint8,
                     device="cuda")
    o = {key: torch.empty(1024 * 1024, device="cuda") for key in ("dg", "dth", "dph", "dw")}
    dx = torch.empty_like(dev["x"])
    rc = bmoe.bmoe_backward_kept(dt, T, d, N, k, dev["x"], dev["gates"], dev["w_packed"], 1.0,
                                 dev["x"], dx, o["dg"], o["dth"], o["dph"], o["dw"], short, ws)
    assert rc == 6  # BMOE_E_WORKSPACE


@pytest.mark.parametrize("name", ["d512_e64_top2_bf16", "d4096_e256_top4_bf16"])
def test_backward_full_size_sampled_tokens(name):
    """At the full workload size: dx and dgates of a token depend only on that
    token's rows, so the oracle computes them exactly for a sample of tokens
    (the angle and substrate gradients sum over every row and are covered at
    reduced sizes)."""
    inp = W.make_inputs(name)
    print(f"[backward] full {name}", flush=True)
    dy, dy_bits = _dy(inp, 31)
    dev = to_device(inp)
    dyt = torch.from_numpy(dy_bits.view(np.int16)).view(torch.bfloat16).cuda()
    g = bmoe.backward(dev["x"], dev["ids"], dev["gates"], dev["theta"], dev["phi"],
                      dev["w_packed"], dev["alpha"], dyt, want_dw=False)
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([np.random.default_rng(4).choice(inp.T, 160, replace=False),
                                     np.arange(inp.T - 16, inp.T)]))
    ref = O.backward(inp.x[toks], inp.ids[toks], inp.gates[toks], inp.theta, inp.phi, inp.w,
                     inp.alpha, dy[toks])
    t = torch.from_numpy(toks).cuda()
    dx = g["dx"][t].float().cpu().numpy().astype(np.float64)
    dgt = g["dgates"][t].cpu().numpy().astype(np.float64)
    assert O.max_rel_err(dx, ref["dx"]) <= TOL["bf16"]
    assert _dgates_err(dgt, ref["dgates"], inp, dy, toks) <= TOL["bf16"]
    assert _global_err(dgt, ref["dgates"]) <= TOL["bf16"]
