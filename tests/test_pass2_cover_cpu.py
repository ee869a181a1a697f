"""The fused variant's pass-2 work dealing, checked on the host (CPU only): tests/c/pass2_cover.cpp
includes the library's own StepPlan functions and checks, over a grid of launch shapes, block shapes,
step sizes and workgroup groupings, that every logits tile is recomputed exactly once and every dx
tile gets one product per vocabulary block and every dW tile one per token block (a duplicate would
add a contribution twice; a gap would drop one), each dealt to exactly one workgroup."""
import os
import subprocess

import pytest

from linear_cross_entropy_token_amd import build as B

SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "pass2_cover.cpp")


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")
def test_pass2_pieces_cover_every_cell_once(tmp_path):
    exe = str(tmp_path / "pass2_cover")
    r = subprocess.run([B.HIPCC, "-O2", "-std=c++17", "-I", B.CSRC, SRC, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and "PASS pass2" in out.stdout, out.stdout + out.stderr
