"""The generated gfx950 code of the hand-pipelined kernels keeps the issue
order their hand-counted waits rely on (CPU only: compiles the sources to
AMD assembly, no GPU).

The global->LDS rings wait with `s_waitcnt vmcnt(N)` before a barrier,
counting the N newest vector-memory operations as ones the barrier need not
cover: in `gemm_dl_kernel` the packed-word loads of the next step, in
`gemm_rb_kernel` and `dw_kernel` the DMA of the two steps still in flight.
Empty `asm volatile("" ::: "memory")` fences hold that order in the source;
these tests check it in what the compiler emitted, and that those kernels do
not spill (a scratch reload is a vector-memory operation the compiler waits
for with vmcnt(0), draining the ring)."""
import os
import re
import shutil
import subprocess

import pytest

from butterfly_rotated_ternary_amd import build as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC) and not shutil.which("hipcc"),
                                reason="hipcc not available")


def _asm(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [B.HIPCC, *[f for f in B.FLAGS if f != "-fPIC"], "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out.read_text()


def _functions(text):
    """Kernel symbol -> its instruction lines (labels kept)."""
    funcs, cur = {}, None
    for line in text.splitlines():
        m = re.match(r"^(_Z[^:\s]+):", line)
        if m:
            cur = m.group(1)
            funcs[cur] = []
            continue
        if cur is None:
            continue
        s = line.strip()
        if not s or s.startswith(";"):
            continue
        if line.startswith("\t") or s.startswith(".LBB"):
            funcs[cur].append(s)
        if s.startswith("s_endpgm"):
            cur = None
    return funcs


def _is_vmem(ins):
    return ins.startswith(("global_load", "global_store", "buffer_", "scratch_", "flat_"))


def _counted_waits(ins):
    """(N, the N newest vector-memory ops before it) for every
    `s_waitcnt vmcnt(N)`, N > 0, that sits right before a barrier, when
    those N ops lie in the same basic block."""
    out = []
    for i, s in enumerate(ins):
        # vmcnt alone, or merged with the lgkmcnt / expcnt wait of the barrier
        m = re.match(r"s_waitcnt vmcnt\((\d+)\)(?: (?:lgkmcnt|expcnt)\(\d+\))*$", s)
        if not m or int(m.group(1)) == 0:
            continue
        if not any(x.startswith("s_barrier") for x in ins[i + 1:i + 4]):
            continue
        n, ops = int(m.group(1)), []
        for s2 in reversed(ins[:i]):
            if s2.startswith((".LBB", "s_cbranch", "s_branch")):
                break
            if _is_vmem(s2):
                ops.append(s2.split()[0])
                if len(ops) == n:
                    break
        if len(ops) == n:
            out.append((n, ops))
    return out


def _kernels(funcs, name):
    ks = {k: v for k, v in funcs.items() if name in k}
    assert ks, f"no {name} in the generated code"
    return ks


def test_gemm_dl_counts_only_packed_word_loads(tmp_path):
    funcs = _functions(_asm("gemm.hip", tmp_path))
    checked = 0
    for k, ins in _kernels(funcs, "gemm_dl_kernel").items():
        for n, ops in _counted_waits(ins):
            # the N newest are plain loads (registers), never the stage DMA
            assert all(o.startswith("global_load") and "lds" not in o for o in ops), (k, n, ops)
            checked += 1
    assert checked > 0


def test_dma_rings_count_only_dma(tmp_path):
    checked = 0
    for src, name in (("gemm.hip", "gemm_rb_kernel"), ("dw.hip", "dw_kernel")):
        funcs = _functions(_asm(src, tmp_path))
        for k, ins in _kernels(funcs, name).items():
            if "dw_f32_kernel" in k:
                continue
            for n, ops in _counted_waits(ins):
                # the steps still in flight: DMA only (a plain load or store
                # among them would shift what the count waits for)
                if any(o.startswith("global_store") for o in ops):
                    continue  # the tile-boundary wait that allows for stores
                assert all(o == "global_load_lds_dwordx4" for o in ops), (k, n, ops)
                checked += 1
    assert checked > 0


@pytest.mark.parametrize("src,name", [("gemm.hip", "gemm_rb_kernel"), ("gemm.hip", "gemm_dl_kernel"),
                                      ("dw.hip", "dw_kernel"), ("bfly_wave.hip", "bfly_wave_kernel"),
                                      ("fused_wave.hip", "fused_wave_kernel")])
def test_pipelined_kernels_do_not_spill(src, name, tmp_path):
    funcs = _functions(_asm(src, tmp_path))
    for k, ins in _kernels(funcs, name).items():
        assert not any(s.startswith("scratch_") for s in ins), k
