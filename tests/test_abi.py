"""The C-ABI library loads and exports every entry point include/bmoe.h
declares; the host-only size queries behave as documented (no GPU needed)."""
import ctypes
import os
import re

import pytest

from butterfly_rotated_ternary_amd import bmoe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bmoe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bmoe_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["bmoe_forward", "bmoe_pack_ternary", "bmoe_workspace_bytes", "bmoe_sync_status",
              "bmoe_packed_words", "bmoe_param_count", "bmoe_status_str",
              "bmoe_pack_workspace_bytes"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(bmoe._LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n
    # and the binding wraps each under the same name
    for n in declared_functions():
        assert callable(getattr(bmoe, n)), n


def test_param_count_matches_fixture(golden_dir):
    for line in open(os.path.join(golden_dir, "param_counts.txt")):
        if line.startswith("#") or not line.strip():
            continue
        d, N, cnt = map(int, line.split())
        assert bmoe.bmoe_param_count(d, N) == cnt


def test_packed_words():
    assert bmoe.bmoe_packed_words(16) == 16
    assert bmoe.bmoe_packed_words(512) == 512 * 32
    assert bmoe.bmoe_packed_words(4096) == 4096 * 256
    # d = 2, 4, 8: one zero-padded word per row
    for d in (2, 4, 8):
        assert bmoe.bmoe_packed_words(d) == d
    for bad in (0, 1, 6, 24, 16384, -16):
        assert bmoe.bmoe_packed_words(bad) == 0


def test_small_d_contract():
    """d = 2, 4, 8: the forward and the pack step take them; the entry points
    that need whole 16-column words per row reject them."""
    bf, f32 = bmoe.BMOE_BF16, bmoe.BMOE_F32
    for d in (2, 4, 8):
        for dt in (bf, f32):
            assert bmoe.bmoe_workspace_bytes(dt, 100, d, 3, 2) > 0
            assert bmoe.bmoe_forward_kernel_count(dt, 100, d, 3, 2) == 2
            assert [bmoe.bmoe_forward_kernel_name(dt, 100, d, 3, 2, i) for i in range(2)] == \
                ["prep_kernel", "small_kernel"]
            assert bmoe.bmoe_backward_workspace_bytes(dt, 100, d, 3, 2) == 0
            assert bmoe.bmoe_forward_keep_workspace_bytes(dt, 100, d, 3, 2) == 0
            assert bmoe.bmoe_rotate_in_workspace_bytes(dt, 100, d, 3, 2) == 0
            assert bmoe.bmoe_router_workspace_bytes(dt, 100, d, 3, 2) == 0
        assert bmoe.bmoe_packed3_bytes(d) == 0
        assert bmoe.bmoe_param_count(d, 5) == d * d + 2 * 5 * (d.bit_length() - 1) * (d // 2)
    lib = bmoe.lib()
    a = [None] * 10
    assert lib.bmoe_backward(1, 4, 8, 8, 2, *a[:6], 1.0, *a[:7], 0, None) == 2
    assert lib.bmoe_forward(1, 4, 8, 8, 2, None, None, None, None, None, None, 1.0, None, None,
                            0, None, None) == 1     # shape accepted, pointers checked next


def test_workspace_bytes_validates_shape():
    # d = 512 bf16 keeps Z and H on chip: at least U (bf16) over M = T*k rows
    ok = bmoe.bmoe_workspace_bytes(bmoe.BMOE_BF16, 4096, 512, 64, 2)
    assert ok >= 8192 * 512 * 2
    # split path: Z, H and U over M rows
    big = bmoe.bmoe_workspace_bytes(bmoe.BMOE_BF16, 4096, 2048, 64, 2)
    assert big >= 8192 * 2048 * 2 * 3
    f32 = bmoe.bmoe_workspace_bytes(bmoe.BMOE_F32, 256, 64, 8, 2)
    assert f32 >= 512 * 64 * 4 * 3
    assert bmoe.bmoe_workspace_bytes(bmoe.BMOE_BF16, 0, 512, 64, 2) > 0
    for args in [(bmoe.BMOE_BF16, 16, 500, 64, 2),   # d not a power of two
                 (bmoe.BMOE_BF16, 16, 512, 64, 65),  # k > N
                 (bmoe.BMOE_BF16, 16, 512, 0, 1),    # N < 1
                 (bmoe.BMOE_BF16, -1, 512, 64, 2),   # T < 0
                 (bmoe.BMOE_BF16, 16, 512, 5000, 2),  # N too large
                 (7, 16, 512, 64, 2)]:               # bad dtype
        assert bmoe.bmoe_workspace_bytes(*args) == 0


def test_product_validation_needs_no_gpu():
    lib = bmoe.lib()
    assert lib.bmoe_product(4, 512, None, None, 9, 1.0, None, None, None) == 3
    assert lib.bmoe_product(4, 96, None, None, 0, 1.0, None, None, None) == 2
    assert lib.bmoe_product(-1, 512, None, None, 0, 1.0, None, None, None) == 2
    assert lib.bmoe_product(4, 512, None, None, 1, 1.0, None, None, None) == 1
    assert lib.bmoe_product(0, 512, None, None, 1, 1.0, None, None, None) == 0


def test_status_strings():
    for code in range(9):
        assert bmoe.bmoe_status_str(code)


def test_host_validation_needs_no_gpu():
    # These return before any HIP call: shape, dtype and null checks.
    lib = bmoe.lib()
    assert lib.bmoe_forward(9, 4, 512, 8, 2, None, None, None, None, None, None, 1.0, None, None,
                            0, None, None) == 3
    assert lib.bmoe_forward(1, 4, 500, 8, 2, None, None, None, None, None, None, 1.0, None, None,
                            0, None, None) == 2
    assert lib.bmoe_forward(1, 4, 512, 8, 2, None, None, None, None, None, None, 1.0, None, None,
                            0, None, None) == 1
    assert lib.bmoe_forward(1, 0, 512, 8, 2, None, None, None, None, None, None, 1.0, None, None,
                            0, None, None) == 0     # T = 0 is a no-op
    assert lib.bmoe_pack_ternary(None, 16, None, None, 0, None) == 1


def test_forward_launch_table():
    bf, f32 = bmoe.BMOE_BF16, bmoe.BMOE_F32

    def names(dt, T, d, N, k):
        return [bmoe.bmoe_forward_kernel_name(dt, T, d, N, k, i)
                for i in range(bmoe.bmoe_forward_kernel_count(dt, T, d, N, k))]
    # fused with routing inside: up to 8192 routed rows, and 256 experts at
    # d = 512 or 512 at d = 256
    assert names(bf, 4096, 512, 64, 2) == ["fused_wave_kernel", "combine_kernel"]
    assert names(bf, 4096, 512, 256, 2) == ["fused_wave_kernel", "combine_kernel"]
    assert names(bf, 4096, 256, 512, 2) == ["fused_wave_kernel", "combine_kernel"]
    # beyond either limit the prep kernel routes
    assert names(bf, 4097, 512, 64, 2) == ["prep_kernel", "fused_wave_kernel", "combine_kernel"]
    assert names(bf, 64, 512, 257, 2) == ["prep_kernel", "fused_wave_kernel", "combine_kernel"]
    assert names(bf, 64, 256, 513, 2) == ["prep_kernel", "fused_wave_kernel", "combine_kernel"]
    # split path
    assert names(f32, 64, 512, 8, 2) == ["prep_kernel", "bfly_in_kernel", "gemm_kernel",
                                         "bfly_out_kernel", "combine_kernel"]
    assert names(bf, 64, 1024, 8, 2)[0] == "prep_kernel"
    assert bmoe.bmoe_forward_kernel_name(bf, 4096, 512, 64, 2, 2) == ""


def test_backward_launch_table_and_validation():
    bf = bmoe.BMOE_BF16
    def names(dt, d):
        return [bmoe.bmoe_backward_kernel_name(dt, 64, d, 8, 2, i)
                for i in range(bmoe.bmoe_backward_kernel_count(dt, 64, d, 8, 2))]
    # bf16 d = 256, 512: Z and H recomputed by the fused kernel in one launch
    fused = names(bf, 512)
    assert fused == names(bf, 256)
    assert fused == ["prep_kernel", "fused_wave_kernel", "bfly_bwd_out_kernel", "dw_kernel",
                     "gemm_t_kernel", "bfly_bwd_in_kernel", "finish_kernel"]
    for other in (names(bf, 1024), names(bmoe.BMOE_F32, 512), names(bf, 128)):
        assert len(other) == 8 and len(set(other)) == 8
        assert other[1:3] == ["bfly_in_kernel", "gemm_kernel"]
        assert "bfly_bwd_out_kernel" in other and "gemm_t_kernel" in other
        assert other[0] == "prep_kernel" and other[-1] == "finish_kernel"
    assert bmoe.bmoe_backward_kernel_count(bf, 64, 8192, 8, 2) == 0   # d > 4096
    assert bmoe.bmoe_backward_kernel_count(bf, 0, 512, 8, 2) == 0
    assert bmoe.bmoe_backward_kernel_name(bf, 64, 512, 8, 2, 7) == ""
    assert bmoe.bmoe_backward_kernel_name(bf, 64, 1024, 8, 2, 8) == ""
    assert bmoe.bmoe_backward_workspace_bytes(bf, 64, 8192, 8, 2) == 0
    assert bmoe.bmoe_backward_workspace_bytes(bf, 64, 4096, 8, 2) > 0
    lib = bmoe.lib()
    a = [None] * 10
    assert lib.bmoe_backward(9, 4, 512, 8, 2, *a[:6], 1.0, *a[:7], 0, None) == 3
    assert lib.bmoe_backward(1, 4, 8192, 8, 2, *a[:6], 1.0, *a[:7], 0, None) == 2
    assert lib.bmoe_backward(1, 4, 512, 8, 2, *a[:6], 1.0, *a[:7], 0, None) == 1
    assert lib.bmoe_backward(1, 0, 512, 8, 2, *a[:6], 1.0, *a[:7], 0, None) == 0


def test_router_validation_needs_no_gpu():
    bf = bmoe.BMOE_BF16
    assert bmoe.bmoe_router_workspace_bytes(bf, 100, 512, 64, 2) >= 100 * 64 * 4
    assert bmoe.bmoe_router_workspace_bytes(bf, 100, 512, 128, 65) == 0   # k > 64
    assert bmoe.bmoe_router_workspace_bytes(bf, 100, 500, 64, 2) == 0
    lib = bmoe.lib()
    assert lib.bmoe_router(9, 4, 512, 8, 2, None, None, None, None, None, None, 0, None) == 3
    assert lib.bmoe_router(1, 4, 512, 80, 65, None, None, None, None, None, None, 0, None) == 2
    assert lib.bmoe_router(1, 4, 512, 8, 2, None, None, None, None, None, None, 0, None) == 1
    assert lib.bmoe_router(1, 0, 512, 8, 2, None, None, None, None, None, None, 0, None) == 0
