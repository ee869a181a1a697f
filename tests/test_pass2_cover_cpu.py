"""The fused variant's pass-2 work decomposition, checked on the host (CPU only): tests/c/pass2_cover.cpp
includes the library's own span_piece and checks, over a grid of shapes, row heights, piece widths and
workgroup counts in both dealing modes, that every cell is covered exactly once by pieces inside the
grid and no wider than allowed (an overlap would make two workgroups add the same dlogits twice; a
gap would drop a tile's dx and dW contributions)."""
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
