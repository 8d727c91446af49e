"""bench.py's host-side model: the algorithmic work of a launch, the roofline
choice, the stored counter lookup and the one-GPU contract. CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

T, D, N, K = 4096, 512, 64, 2          # the d = 512 workload
M = T * K
L = 9
A = N * L * (D // 2)                   # angles per side


def test_routed_fused_bytes_follow_the_stated_per_unit_figures():
    # per token 2d B of x; per routed row 2d B of U, 4 B id, 4 B gate, 12 B of
    # tables written; per call d^2/4 B of packed W, 4 B per angle on both
    # sides, (N+1) * 4 B of offsets
    want = T * 2 * D + M * (2 * D + 4 + 4 + 12) + D * D // 4 + 2 * A * 4 + (N + 1) * 4
    w = bench.kernel_work("fused_wave_kernel", 2, T, D, N, K, routed=True)
    assert w["bytes"] == want == 13_992_196
    assert w["mfma_flops"] == 2 * M * D * D
    assert w["valu_flops"] == 2 * M * L * (D // 2) * 6


def test_prep_path_fused_bytes_differ_from_the_routed_ones():
    routed = bench.kernel_work("fused_wave_kernel", 2, T, D, N, K, routed=True)["bytes"]
    after_prep = bench.kernel_work("fused_wave_kernel", 2, T, D, N, K)["bytes"]
    # after prep: packed W and both angle sets in, perm, slot_e and gates per
    # routed row; nothing written back but U
    assert after_prep == (T * 2 * D + M * 2 * D + D * D // 4 + 2 * A * 4 + 3 * M * 4)
    assert after_prep != routed


def test_prep_writes_tables_only_where_no_fused_kernel_follows():
    routing = M * 4 + 3 * M * 4 + (N + 1) * 4
    assert bench.kernel_work("prep_kernel", 2, T, D, N, K)["bytes"] == routing
    assert bench.kernel_work("prep_kernel", 2, T, D, N, K, trig=True)["bytes"] == (
        routing + 2 * A * 4 + 2 * A * 8)
    # d = 4096, T = 32768, top-4: 1024 row tiles x 8 column tiles of the large
    # product, which reads a tile-major copy of the packed substrate
    d, n, k, t = 4096, 256, 4, 32768
    a = n * 12 * (d // 2)
    want = t * k * 16 + (n + 1) * 4 + 2 * a * 12 + 2 * (d * d // 4)
    assert bench.kernel_work("prep_kernel", 2, t, d, n, k)["bytes"] == want


def test_roofline_takes_the_resource_with_the_largest_ideal_time():
    work = {"bytes": 8e9, "mfma_flops": 1e12, "valu_flops": 0}   # 1 ms HBM, 0.4 ms MFMA
    r = bench.roofline(work, 2e-3, bench.PEAK_BF16_TFLOPS)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(4000.0)
    assert r["frac"] == pytest.approx(0.5)
    work = {"bytes": 8e6, "mfma_flops": 5e12, "valu_flops": 0}   # 1 us HBM, 2 ms MFMA
    r = bench.roofline(work, 4e-3, bench.PEAK_BF16_TFLOPS)
    assert r["bound"] == "mfma" and r["frac"] == pytest.approx(0.5)


def test_alu_peak_and_per_resource_fractions():
    # 256 CU x 4 SIMD x 32 lanes x 2 flop x 2.4 GHz
    assert bench.PEAK_VALU_F32_TFLOPS == pytest.approx(157.2864)
    # the routed d = 512 fused kernel: its bytes at 8 TB/s (1.75 us) take
    # longer than its product at 2.5 PFLOP/s (1.72 us) or its rotations at
    # 157 TFLOP/s (1.44 us)
    w = bench.kernel_work("fused_wave_kernel", 2, T, D, N, K, routed=True)
    r = bench.roofline(w, 26e-6, bench.PEAK_BF16_TFLOPS)
    assert r["bound"] == "hbm"
    assert r["frac_by_resource"]["mfma"] == pytest.approx(2 * M * D * D / 2.5e15 / 26e-6)
    assert r["frac_by_resource"]["alu"] == pytest.approx(w["valu_flops"] / 157.2864e12 / 26e-6)
    assert r["frac"] == pytest.approx(r["frac_by_resource"]["hbm"])


def test_stored_traffic_requires_the_current_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    f = prof / "fused_kernel_w.traffic.txt"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda: "abc")
    f.write_text("# header\nsource_sha256: abc\ntraffic_bytes_per_launch: 123\n")
    assert bench.stored_traffic("fused_kernel", "w") == 123.0
    f.write_text("source_sha256: other\ntraffic_bytes_per_launch: 123\n")
    assert bench.stored_traffic("fused_kernel", "w") is None
    assert bench.stored_traffic("gemm_kernel", "w") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "--gpus 1" in (r.stdout + r.stderr)


def test_backward_partials_follow_the_tile_rows():
    # 16-row tiles at d = 512: M / 16 + N tiles, each one [L][d/2] fp32 partial
    tiles = M // 16 + N
    w = bench.backward_work("finish_kernel", 2, T, D, N, K)
    slices = bench.dw_slices(M, D)
    want = (M + T) * D * 2 + 2 * (tiles * L * (D // 2) * 4 + A * 4)
    if slices > 1:
        want += (slices + 1) * D * D * 4
    assert w["bytes"] == want
