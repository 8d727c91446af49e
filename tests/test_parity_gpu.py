"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Routing tables must match bit for bit. Outputs must be within the
per-token max relative error (||y_t - ref_t||_inf / ||ref_t||_inf, max over t)
of 1e-4 on the fp32 path and 2e-2 on the bf16 path.
"""
import numpy as np
import pytest
import torch

import oracle as O
from butterfly_rotated_ternary_amd import bmoe
from butterfly_rotated_ternary_amd import workloads as W
from devinputs import run_forward, to_device

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}

# Reduced token counts: the full oracle finishes in seconds, the rows still
# span many tiles, and M = T*k is not a multiple of any tile size.
REDUCED_T = {
    "tiny_d64_e8_top2_f32": 256,
    "d512_e64_top2_bf16": 509,
    "d512_e256_top2_zipf_bf16": 2003,
    "d2048_e64_top2_outliers_bf16": 301,
    "d4096_e256_top4_bf16": 61,
}


def check_route(inp, route):
    off, perm, inv = O.route(inp.ids, inp.N)
    g_off, g_perm, g_inv = route
    assert np.array_equal(g_off, off)
    assert np.array_equal(g_perm, perm)
    assert np.array_equal(g_inv, inv)


def _announce(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_forward_matches_oracle_reduced(name):
    inp = W.make_inputs(name, T=REDUCED_T[name])
    _announce(f"[parity reduced] {name} T={inp.T} d={inp.d} N={inp.N} k={inp.k}")
    dev = to_device(inp)
    y, route = run_forward(dev, inp)
    check_route(inp, route)
    ref = O.forward(inp.x, inp.ids, inp.gates, inp.theta, inp.phi, inp.w, inp.alpha)
    err = O.max_rel_err(y, ref)
    _announce(f"  max rel err {err:.3e}")
    assert err <= TOL[inp.dtype]


# Full-size checks. Where the oracle finishes every token in seconds (the
# d = 64 and d = 512 workloads) every token is compared. At d = 2048 and
# d = 4096 the tokens are chosen from the routing so that every block of B
# consecutive sorted slots holds at least one checked routed row: B = 32 is
# the row tile of the routed butterflies and the fused kernel, 128 the row
# tile of the large-tile product. Each block contributes the token of one
# row drawn at random inside it, plus the first and last token.
FULL_ALL_TOKENS = {"tiny_d64_e8_top2_f32", "d512_e64_top2_bf16", "d512_e256_top2_zipf_bf16"}
FULL_SLOT_BLOCK = {"d2048_e64_top2_outliers_bf16": 32, "d4096_e256_top4_bf16": 128}


def tokens_covering_slot_blocks(perm, k, block, T, seed=0):
    """One token per block of `block` sorted slots (a random slot inside the
    block), plus tokens 0 and T-1."""
    rng = np.random.default_rng(seed)
    M = perm.size
    starts = np.arange(0, M, block)
    lens = np.minimum(block, M - starts)
    q = starts + (rng.random(starts.size) * lens).astype(np.int64)
    toks = perm[q].astype(np.int64) // k
    return np.unique(np.concatenate([[0, T - 1], toks]))


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_forward_full_size(name):
    inp = W.make_inputs(name)
    _announce(f"[parity full] {name} T={inp.T} d={inp.d} N={inp.N} k={inp.k}")
    dev = to_device(inp)
    y, route = run_forward(dev, inp)
    check_route(inp, route)
    assert np.isfinite(y).all()
    if name in FULL_ALL_TOKENS:
        toks = np.arange(inp.T)
        ref = O.forward(inp.x, inp.ids, inp.gates, inp.theta, inp.phi, inp.w, inp.alpha)
    else:
        toks = tokens_covering_slot_blocks(route[1], inp.k, FULL_SLOT_BLOCK[name], inp.T)
        # tokens are independent: the forward of a subset of tokens is the
        # subset of the forward
        ref = O.forward(inp.x[toks], inp.ids[toks], inp.gates[toks], inp.theta, inp.phi, inp.w,
                        inp.alpha)
        blocks = np.unique(route[2].reshape(inp.T, inp.k)[toks].ravel() //
                           FULL_SLOT_BLOCK[name])
        assert blocks.size == -(-inp.T * inp.k // FULL_SLOT_BLOCK[name])
    err = O.max_rel_err(y[toks], ref)
    _announce(f"  max rel err {err:.3e} on {toks.size} of {inp.T} tokens")
    assert err <= TOL[inp.dtype]


def test_large_angles_routed_and_prep_paths():
    """Angles are free learned parameters, so they need not stay in
    [-pi, pi]. With theta, phi ~ U(-1000, 1000): T = 4096 (8192 routed rows)
    runs the routed fused kernel, whose coefficients come from the hardware
    sine/cosine after its own range reduction; T = 4200 runs the prep kernel's
    sincosf tables. Both match the oracle, and on their shared first 4096
    tokens they agree to within three bf16 roundings (2^-6 of the token's
    largest entry)."""
    base = W.make_inputs(W.HEADLINE, T=4200, seed=909)
    rng = np.random.default_rng(910)
    base.theta[:] = rng.uniform(-1000, 1000, base.theta.shape).astype(np.float32)
    base.phi[:] = rng.uniform(-1000, 1000, base.phi.shape).astype(np.float32)
    ys = {}
    for T in (4096, 4200):
        inp = W.make_inputs(W.HEADLINE, T=4200, seed=909)
        inp.theta[:], inp.phi[:] = base.theta, base.phi
        for a in ("x", "x_bits", "ids", "gates"):
            setattr(inp, a, getattr(inp, a)[:T].copy())
        inp.T = T
        nk = bmoe.bmoe_forward_kernel_count(bmoe.BMOE_BF16, T, inp.d, inp.N, inp.k)
        assert nk == (2 if T == 4096 else 3)
        _announce(f"[large angles] T={T} kernels={nk}")
        dev = to_device(inp)
        y, route = run_forward(dev, inp)
        check_route(inp, route)
        ref = O.forward(inp.x, inp.ids, inp.gates, inp.theta, inp.phi, inp.w, inp.alpha)
        err = O.max_rel_err(y, ref)
        _announce(f"  max rel err {err:.3e}")
        assert err <= TOL["bf16"]
        ys[T] = y
    diff = O.max_rel_err(ys[4096], ys[4200][:4096])
    _announce(f"  routed vs prep path: {diff:.3e}")
    assert diff <= 2.0 ** -6


def test_small_d_hand_fixture(golden_dir):
    """The hand-worked d = 2 forward (one stage, two experts, top-2) through
    bmoe_forward, on both paths."""
    import os
    vals = [l.split() for l in open(os.path.join(golden_dir, "forward_d2_hand.txt"))
            if l.strip() and not l.startswith("#")]
    want = np.array([[float(v) for v in vals[0][1:]]])
    for dtype in ("f32", "bf16"):
        inp = W.make_inputs("custom", d=2, N=2, k=2, T=1, seed=1, dtype=dtype)
        inp.x[:] = [[1.0, 2.0]]
        if inp.x_bits is not None:
            inp.x_bits[:] = W.bf16_round_bits(inp.x.astype(np.float32))
        inp.w[:] = [[1, -1], [0, 1]]
        inp.theta[:] = np.array([[[np.pi / 2]], [[0.0]]], dtype=np.float32)
        inp.phi[:] = np.array([[[0.0]], [[np.pi / 2]]], dtype=np.float32)
        inp.ids[:] = [[0, 1]]
        inp.gates[:] = [[0.25, 0.75]]
        inp.alpha = np.float32(1 / np.sqrt(2))
        dev = to_device(inp)
        y, route = run_forward(dev, inp)
        check_route(inp, route)
        if dtype == "f32":
            np.testing.assert_allclose(y, want, atol=1e-6)
        else:
            assert O.max_rel_err(y, want) <= TOL["bf16"]


@pytest.mark.parametrize("d,N,k,T,dtype", [(2, 1, 1, 1, "f32"), (2, 5, 2, 300, "f32"),
                                           (4, 7, 3, 257, "bf16"), (4, 3, 3, 1000, "f32"),
                                           (8, 9, 2, 1001, "f32"), (8, 64, 4, 513, "bf16"),
                                           (8, 2, 2, 70000, "bf16")])
def test_small_d_forward(d, N, k, T, dtype):
    inp = W.make_inputs("custom", d=d, N=N, k=k, T=T, seed=40 + d + N, dtype=dtype)
    _announce(f"[small d] d={d} N={N} k={k} T={T} {dtype}")
    dev = to_device(inp)
    y, route = run_forward(dev, inp)
    check_route(inp, route)
    ref = O.forward(inp.x, inp.ids, inp.gates, inp.theta, inp.phi, inp.w, inp.alpha)
    err = O.max_rel_err(y, ref)
    _announce(f"  max rel err {err:.3e}")
    assert err <= TOL[dtype]


def test_stream_argument_without_context_manager():
    """forward()/backward() given stream= (not torch's current stream, and no
    `with torch.cuda.stream(...)` around the call) give the single-stream
    results bit for bit, while the current stream allocates and writes in
    between."""
    inp = W.make_inputs(W.HEADLINE, T=900, seed=71)
    dev = to_device(inp)
    dy = torch.randn(inp.T, inp.d, device="cuda").to(torch.bfloat16)

    def fwd(stream=None):
        return bmoe.forward(dev["x"], dev["ids"], dev["gates"], dev["theta"], dev["phi"],
                            dev["w_packed"], dev["alpha"], stream=stream)

    def bwd(stream=None):
        return bmoe.backward(dev["x"], dev["ids"], dev["gates"], dev["theta"], dev["phi"],
                             dev["w_packed"], dev["alpha"], dy, stream=stream)

    y0, g0 = fwd(), bwd()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    outs = []
    for _ in range(4):
        outs.append((fwd(side), bwd(side)))
        # the current stream reuses freed memory right away
        junk = [torch.full((1 << 20,), 7.0, device="cuda") for _ in range(8)]
        del junk
    torch.cuda.synchronize()
    for y, g in outs:
        assert torch.equal(y, y0)
        for key in ("dx", "dgates", "dtheta", "dphi", "dw"):
            assert torch.equal(g[key], g0[key]), key


# Shapes whose routed-row count is large enough for the large-tile product
# kernel (128 x 512 tiles, at least 512 of them) while M = T*k is ragged
# against its tiles (the last row tile is partly past M). The token sample
# includes the last 40 tokens routed to the last expert, whose rows sit in
# that last tile.
LARGE_TILE_CASES = [
    (1024, 8, 4, 8200),   # M = 32800 = 256 * 128 + 32
    (4096, 16, 2, 4200),  # M = 8400 = 65 * 128 + 80
]


@pytest.mark.parametrize("d,N,k,T", LARGE_TILE_CASES)
def test_large_tile_product_ragged(d, N, k, T):
    inp = W.make_inputs(W.HEADLINE, d=d, N=N, k=k, T=T, seed=77 + d)
    _announce(f"[parity large tiles] T={T} d={d} N={N} k={k} M={T * k}")
    dev = to_device(inp)
    y, route = run_forward(dev, inp)
    check_route(inp, route)
    rng = np.random.default_rng(1)
    last = np.nonzero((inp.ids == N - 1).any(axis=1))[0]
    toks = np.unique(np.concatenate([[0, T - 1], last[-40:], rng.choice(T, 60, replace=False)]))
    ref = O.forward_tokens(toks, inp.x, inp.ids, inp.gates, inp.theta, inp.phi, inp.w, inp.alpha)
    err = O.max_rel_err(y[toks], ref)
    _announce(f"  max rel err {err:.3e} on {toks.size} sampled tokens")
    assert err <= TOL[inp.dtype]
    assert np.isfinite(y).all()


@pytest.mark.parametrize("d", [2, 4, 8, 16, 64, 512, 4096])
def test_pack_bit_exact(d):
    inp = W.make_inputs("custom", d=d, N=1, k=1, T=1, seed=d)
    w8 = torch.from_numpy(inp.w).cuda()
    packed = bmoe.pack_ternary(w8).cpu().numpy().view(np.uint32).reshape(d, -(-d // 16))
    assert np.array_equal(packed, O.pack_ternary(inp.w))


def test_pack_reports_non_ternary():
    w = torch.zeros(16, 16, dtype=torch.int8, device="cuda")
    w[3, 5] = 2
    with pytest.raises(bmoe.BmoeError) as ei:
        bmoe.pack_ternary(w)
    assert ei.value.code == 4


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_angles_are_a_plain_ternary_product(dtype):
    inp = W.make_inputs("custom", d=256, N=5, k=2, T=130, seed=3, dtype=dtype)
    inp.theta[:] = 0
    inp.phi[:] = 0
    dev = to_device(inp)
    y, _ = run_forward(dev, inp, with_route=False)
    want = float(inp.alpha) * inp.gates.astype(np.float64).sum(1, keepdims=True) * \
        (inp.x.astype(np.float64) @ inp.w.astype(np.float64).T)
    assert O.max_rel_err(y, want) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identity_substrate_equal_angles(dtype):
    inp = W.make_inputs("custom", d=128, N=7, k=3, T=77, seed=4, dtype=dtype)
    inp.w[:] = np.eye(128, dtype=np.int8)
    inp.phi[:] = inp.theta
    dev = to_device(inp)
    y, _ = run_forward(dev, inp, with_route=False)
    want = float(inp.alpha) * inp.gates.astype(np.float64).sum(1, keepdims=True) * inp.x
    assert O.max_rel_err(y, want) <= TOL[dtype]


@pytest.mark.parametrize("d,N,k,T", [(16, 1, 1, 1), (32, 3, 3, 5), (64, 300, 1, 1000),
                                     (1024, 2, 2, 33), (8192, 4, 2, 3),
                                     # the routed fused kernel at its limits:
                                     # 8192 routed rows; 512 experts at
                                     # d = 256, 256 at d = 512
                                     (256, 512, 2, 4096), (512, 256, 1, 8192),
                                     # routed: top-3 and top-4, one expert
                                     (256, 8, 3, 111), (512, 16, 4, 300), (512, 1, 1, 100),
                                     # fused after prep, ragged, more tiles than
                                     # workgroups (three or two per workgroup)
                                     (256, 64, 3, 5555), (512, 600, 2, 9000)])
def test_edge_shapes(d, N, k, T):
    inp = W.make_inputs("custom", d=d, N=N, k=k, T=T, seed=d + N, dtype="bf16")
    _announce(f"[edge] d={d} N={N} k={k} T={T}")
    dev = to_device(inp)
    y, route = run_forward(dev, inp)
    check_route(inp, route)
    ref = O.forward(inp.x, inp.ids, inp.gates, inp.theta, inp.phi, inp.w, inp.alpha)
    assert O.max_rel_err(y, ref) <= TOL["bf16"]


@pytest.mark.parametrize("d,tail", [(256, 0), (512, 0), (512, 8072)])
def test_fused_tiles_holding_several_experts(d, tail):
    """Sorted rows are cut into 32-row tiles regardless of expert: one tile
    splits two experts (the first and last expert's coefficients come from
    LDS tables), one holds five (the middle ones: a per-group table written by
    the whole workgroup when the kernel routes, reloads from global memory
    after the prep kernel), one a single expert, and the last ends on an empty
    expert. tail > 0 appends an expert of that many rows, taking M above 8192
    so the prep kernel routes."""
    counts = [13, 19, 3, 1, 2, 70, 0, 20] + ([tail] if tail else [])
    M = sum(counts)
    labels = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    inp = W.make_inputs("custom", d=d, N=len(counts), k=2, T=M // 2, seed=d + 11, dtype="bf16")
    inp.ids[:] = np.random.default_rng(d).permutation(labels).reshape(M // 2, 2)
    nk = bmoe.bmoe_forward_kernel_count(bmoe.BMOE_BF16, inp.T, d, inp.N, 2)
    assert nk == (3 if tail else 2)
    _announce(f"[tiles] d={d} counts={counts} kernels={nk}")
    dev = to_device(inp)
    y, route = run_forward(dev, inp)
    check_route(inp, route)
    assert np.array_equal(np.diff(route[0]), counts)
    ref = O.forward(inp.x, inp.ids, inp.gates, inp.theta, inp.phi, inp.w, inp.alpha)
    assert O.max_rel_err(y, ref) <= TOL["bf16"]


@pytest.mark.parametrize("N", [256, 257, 512])
def test_fused_tiles_of_many_small_experts(N):
    """600 routed rows over N experts: most tiles hold 13 to 27 experts,
    nearly all of them middle experts. N = 256 routes inside the fused
    kernel, N = 257 and 512 in the prep kernel."""
    inp = W.make_inputs("custom", d=512, N=N, k=2, T=300, seed=N, dtype="bf16")
    _announce(f"[many experts] d=512 N={N} T=300")
    dev = to_device(inp)
    y, route = run_forward(dev, inp)
    check_route(inp, route)
    ref = O.forward(inp.x, inp.ids, inp.gates, inp.theta, inp.phi, inp.w, inp.alpha)
    assert O.max_rel_err(y, ref) <= TOL["bf16"]


def test_concurrent_streams_give_the_single_stream_results():
    """Distinct workspaces on distinct streams, enqueued without waiting for
    each other (fused d = 512 and split d = 2048 paths, forward and backward):
    every result equals the same call made alone, bit for bit."""
    cases = [W.make_inputs(W.HEADLINE, T=700, seed=61), W.make_inputs(W.HEADLINE, T=333, seed=62),
             W.make_inputs("d2048_e64_top2_outliers_bf16", T=129, seed=63)]
    devs = [to_device(inp) for inp in cases]
    dys = [torch.randn(inp.T, inp.d, device="cuda").to(torch.bfloat16) for inp in cases]

    def fwd(dev, stream=None):
        return bmoe.forward(dev["x"], dev["ids"], dev["gates"], dev["theta"], dev["phi"],
                            dev["w_packed"], dev["alpha"], stream=stream)

    def bwd(dev, dy, stream=None):
        return bmoe.backward(dev["x"], dev["ids"], dev["gates"], dev["theta"], dev["phi"],
                             dev["w_packed"], dev["alpha"], dy, stream=stream)

    alone_y = [fwd(dev) for dev in devs]
    alone_g = [bwd(dev, dy) for dev, dy in zip(devs, dys)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in cases]
    torch.cuda.synchronize()
    ys, gs = [], []
    for _ in range(3):
        for dev, dy, st in zip(devs, dys, streams):
            with torch.cuda.stream(st):
                ys.append(fwd(dev, st))
                gs.append(bwd(dev, dy, st))
    torch.cuda.synchronize()
    for i, (y, g) in enumerate(zip(ys, gs)):
        c = i % len(cases)
        assert torch.equal(y, alone_y[c])
        for key in ("dx", "dgates", "dtheta", "dphi", "dw"):
            assert torch.equal(g[key], alone_g[c][key]), (c, key)


def test_duplicate_experts_in_a_token():
    inp = W.make_inputs("custom", d=64, N=4, k=3, T=50, seed=5, dtype="f32")
    inp.ids[:, 1] = inp.ids[:, 0]
    dev = to_device(inp)
    y, route = run_forward(dev, inp)
    check_route(inp, route)
    ref = O.forward(inp.x, inp.ids, inp.gates, inp.theta, inp.phi, inp.w, inp.alpha)
    assert O.max_rel_err(y, ref) <= TOL["f32"]


def test_bitwise_deterministic():
    inp = W.make_inputs(W.HEADLINE, T=1500)
    dev = to_device(inp)
    y1, r1 = run_forward(dev, inp)
    y2, r2 = run_forward(dev, inp)
    assert np.array_equal(y1, y2)
    for a, b in zip(r1, r2):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("d,bad", [(64, 4), (512, 4), (512, -1)])
def test_out_of_range_expert_is_reported(d, bad):
    """d = 512 routes inside the fused kernel, d = 64 in the prep kernel;
    ids past either end are clamped for addressing and reported."""
    inp = W.make_inputs("custom", d=d, N=4, k=2, T=20, seed=6, dtype="bf16")
    dev = to_device(inp)
    dev["ids"][3, 1] = bad
    ws = bmoe.Workspace(bmoe.BMOE_BF16, inp.T, inp.d, inp.N, inp.k)
    bmoe.forward(dev["x"], dev["ids"], dev["gates"], dev["theta"], dev["phi"], dev["w_packed"],
                 dev["alpha"], ws=ws)
    assert bmoe.bmoe_sync_status(ws.buf) == 5
    # a clean call on the same workspace clears it
    dev["ids"][3, 1] = 0
    bmoe.forward(dev["x"], dev["ids"], dev["gates"], dev["theta"], dev["phi"], dev["w_packed"],
                 dev["alpha"], ws=ws)
    assert bmoe.bmoe_sync_status(ws.buf) == 0


def test_small_workspace_and_alignment_rejected():
    inp = W.make_inputs("custom", d=64, N=4, k=2, T=20, seed=7, dtype="bf16")
    dev = to_device(inp)
    need = bmoe.bmoe_workspace_bytes(bmoe.BMOE_BF16, inp.T, inp.d, inp.N, inp.k)
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(dev["x"])
    rc = bmoe.bmoe_forward(bmoe.BMOE_BF16, inp.T, inp.d, inp.N, inp.k, dev["x"], dev["ids"],
                           dev["gates"], dev["theta"], dev["phi"], dev["w_packed"], dev["alpha"],
                           y, small)
    assert rc == 6
    ws = torch.empty(need + 64, dtype=torch.uint8, device="cuda")
    rc = bmoe.lib().bmoe_forward(bmoe.BMOE_BF16, inp.T, inp.d, inp.N, inp.k,
                                 bmoe._ptr(dev["x"]), bmoe._ptr(dev["ids"]), bmoe._ptr(dev["gates"]),
                                 bmoe._ptr(dev["theta"]), bmoe._ptr(dev["phi"]),
                                 bmoe._ptr(dev["w_packed"]), 1.0, bmoe._ptr(y),
                                 bmoe.ctypes.c_void_p(ws.data_ptr() + 8), need, None, None)
    assert rc == 8


@pytest.mark.parametrize("name", [W.HEADLINE, "d2048_e64_top2_outliers_bf16"])
def test_timed_forward_matches_untimed(name):
    """bmoe_forward_timed (per-dispatch start/stop events) computes exactly
    what bmoe_forward does, and every kernel reports a positive duration."""
    import ctypes
    inp = W.make_inputs(name, T=300)
    dev = to_device(inp)
    T, d, N, k = inp.T, inp.d, inp.N, inp.k
    y_ref, _ = run_forward(dev, inp, with_route=False)
    dt = bmoe.BMOE_BF16 if inp.dtype == "bf16" else bmoe.BMOE_F32
    nk = bmoe.bmoe_forward_kernel_count(dt, T, d, N, k)
    assert nk in (2, 3, 5)
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = []
    for _ in range(2 * nk):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    ws = bmoe.Workspace(dt, T, d, N, k, device=dev["x"].device)
    y = torch.empty_like(dev["x"])
    rc = bmoe.bmoe_forward_timed(dt, T, d, N, k, dev["x"], dev["ids"], dev["gates"], dev["theta"],
                                 dev["phi"], dev["w_packed"], dev["alpha"], y, ws.buf, None,
                                 torch.cuda.current_stream(), evs)
    assert rc == 0
    torch.cuda.synchronize()
    assert np.array_equal(y.float().cpu().numpy().astype(np.float64), y_ref)
    for i in range(nk):
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), evs[2 * i], evs[2 * i + 1]) == 0
        assert 0.0 < ms.value < 1000.0
    for e in evs:
        hip.hipEventDestroy(e)
