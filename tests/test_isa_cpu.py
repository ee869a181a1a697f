"""The device code as built (same hipcc flags as the package build) contains no scalar-cache
writes (scalar stores, scalar atomics, scalar-cache write-back or discard) and no packed fp32
VALU operations: every HIP source is compiled to gfx950 assembly here and scanned.  CPU only."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from linear_cross_entropy_token_amd import build as B

FORBIDDEN = re.compile(r"^\s*(s_store|s_buffer_store|s_atomic|s_buffer_atomic|s_dcache_wb|s_dcache_discard|"
                       r"s_scratch_store|v_pk_add_f32|v_pk_mul_f32|v_pk_fma_f32)\b", re.M)


def _asm(src, tmp):
    out = os.path.join(tmp, os.path.basename(src) + ".s")
    cmd = [B.HIPCC, *B.FLAGS, "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read()


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")
def test_device_code_has_no_forbidden_instructions(tmp_path):
    assert "-packed-fp32-ops" in B.FLAGS
    srcs = [os.path.join(B.CSRC, s) for s in B.SOURCES]
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        asms = list(ex.map(lambda s: _asm(s, str(tmp_path)), srcs))
    for src, asm in zip(srcs, asms):
        assert "v_mfma" in asm or "flce_api" in src or "rmsnorm" in src, f"{src}: no MFMA in the build?"
        bad = FORBIDDEN.findall(asm)
        assert not bad, f"{os.path.basename(src)}: {sorted(set(bad))}"
