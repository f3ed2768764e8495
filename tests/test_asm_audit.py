"""Audit of the GEMM's hand-placed m0 writes (no GPU needed).

The LDS-staged FP6 GEMM issues its global->LDS copies from inline assembly
that sets m0 (the copies' LDS base) itself, a register the compiler treats as
reserved. That is only sound while no compiler-generated code in the same
kernels keeps a value in m0, so this test compiles the GEMM source for gfx950
and checks that every instruction touching m0 is one of those writes, each
directly followed by its copy.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "rotation_w4a4_quantized_amd", "csrc", "gemm6.hip")


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc") or ""):
        if c and os.path.exists(c):
            return c
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_gemm_m0_only_feeds_lds_copies(tmp_path):
    from rotation_w4a4_quantized_amd import build as B
    out = tmp_path / "gemm6.s"
    cmd = [_hipcc(), "-x", "hip", *B.FLAGS, "--cuda-device-only", "-S", SRC, "-o", str(out)]
    p = subprocess.run(cmd, capture_output=True, text=True)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [ln.strip() for ln in out.read_text().splitlines()]
    code = [ln for ln in lines if ln and not ln.startswith((";", ".", "//")) and not ln.endswith(":")]
    writes = 0
    for i, ln in enumerate(code):
        if not re.search(r"\bm0\b", ln):
            continue
        assert re.match(r"s_mov_b32 m0, s\d+$", ln), ln
        nxt = code[i + 1]
        assert nxt.startswith(("global_load_lds_dwordx4 ", "global_load_lds_dword ")), (ln, nxt)
        writes += 1
    assert writes > 0                                    # the kernels were compiled
