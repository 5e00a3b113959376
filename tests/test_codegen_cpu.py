"""Code-generation checks of the grouped GEMM kernels (CPU only: hipcc cross-compiles gfx950).

The big-tile kernels stream operand tiles into an LDS ring with direct-to-LDS
buffer loads and synchronise it with explicit vmcnt waits.  The compiler also
tracks those loads, and when LDS accesses carry alias-scope metadata (which
restrict-qualified LDS pointers produce after inlining) it may decide that a
read of one ring buffer depends on a load still in flight into another and
insert a full `s_waitcnt vmcnt(0)` before the read.  Inside the K loop that
drains the prefetch every stage and serialises loads with the matrix-core
work.  This test compiles the kernels to assembly and fails if any such drain
appears inside a K loop (a loop nested in the per-item loop).
"""
from __future__ import annotations

import os
import re
import subprocess

import pytest

from mixture_experts_layer_moe_amd import build as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not available")


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "grouped_gemm.s"
    cmd = [B.HIPCC, *[f for f in B.CFLAGS if f != "-fPIC"], "--cuda-device-only", "-S",
           os.path.join(B.CSRC, "grouped_gemm.hip"), "-o", str(out)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    return out.read_text()


def _functions(asm: str):
    for m in re.finditer(r"^(_Z\S+):", asm, re.M):
        end = asm.index(".Lfunc_end", m.start())
        yield m.group(1), asm[m.start():end]


def _vmcnt_zero(line: str) -> bool:
    return line.startswith("s_waitcnt") and "vmcnt(0)" in line


def _inner_loop_drains(body: str):
    """(block label, read) pairs where a K-loop LDS read directly follows a vmcnt(0) wait."""
    lines = [ln for ln in body.split("\n") if ln.strip() and not ln.strip().startswith(";")]
    label, hits = "", []
    for i, ln in enumerate(lines[:-1]):
        if ln.startswith(".LBB"):
            label = ln
        if _vmcnt_zero(ln.strip()) and "Parent Loop" in label:
            nxt = [x.strip() for x in lines[i + 1:i + 3]]
            if any(x.startswith("ds_read") for x in nxt):
                hits.append((label.split(":")[0], nxt[0]))
    return hits


def test_big_tile_kernels_present(gemm_asm):
    names = [n for n, _ in _functions(gemm_asm) if "gemm_mfma32_kernel" in n]
    # layer0 (SwiGLU, GELU) and layer1 for the 256- and 128-row tiles, plus the 128-column layer1 fallbacks
    assert len(names) >= 8, names


def test_no_prefetch_drain_inside_k_loops(gemm_asm):
    bad = {}
    for name, body in _functions(gemm_asm):
        if "gemm_mfma32_kernel" not in name:
            continue
        hits = _inner_loop_drains(body)
        if hits:
            bad[name] = hits
    assert not bad, f"vmcnt(0) before LDS reads inside K loops: {bad}"


def test_drain_detector_sees_a_drain():
    """The detector itself flags a K-loop read that follows a full vmcnt drain."""
    body = "\n".join([
        ".LBB0_5:                                ;   Parent Loop BB0_2 Depth=1",
        "\ts_waitcnt lgkmcnt(1)",
        "\ts_waitcnt vmcnt(0)",
        "\tds_read_b128 v[0:3], v52",
        "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[0:3], a[0:15]",
    ])
    assert _inner_loop_drains(body) == [(".LBB0_5", "ds_read_b128 v[0:3], v52")]
    clean = body.replace("vmcnt(0)", "vmcnt(8)")
    assert _inner_loop_drains(clean) == []
