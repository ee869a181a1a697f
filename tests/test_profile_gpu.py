"""The library's tracing (flce_profile_enable / flce_profile_read): every launch is timed with HIP
events on the caller's stream, and the GEMM kernels also time their workgroups with the shader-clock
and 100 MHz real-time counters, giving the shader clock they ran at.  Checked for consistency: the
three GEMMs report a clock in the part's range and no GEMM's achieved rate exceeds the dense bf16
peak scaled to its own clock; other kernels report none; enabling again resets everything."""
import pytest

from flce_inputs import make_inputs
from flce_testlib import require_gpu, to_device

pytestmark = pytest.mark.gpu


def test_profile_counts_times_and_shader_clock():
    torch = require_gpu()
    from linear_cross_entropy_token_amd import FusedLinearCrossEntropy
    N, H, V, C = 2048, 1024, 8000, 1024
    x, W, t = to_device(make_inputs(N, H, V, "bf16", seed=201))
    f = FusedLinearCrossEntropy()
    f.profile_enable(True)
    for _ in range(3):
        f.forward_backward(x, W, t, chunk=C)
    torch.cuda.synchronize()
    st = f.profile_read()
    chunks = N // C
    for k in ("logits_lse", "dx", "dw"):
        s = st[k]
        assert s["launches"] == 3 * chunks and s["total_ms"] > 0 and s["flops"] == 3 * chunks * 2.0 * C * V * H
        assert 500.0 <= s["sclk_mhz"] <= 2600.0, (k, s["sclk_mhz"])
        tflops = s["flops"] / (s["total_ms"] * 1e-3) / 1e12
        assert tflops <= 2500.0 * s["sclk_mhz"] / 2400.0 * 1.02, (k, tflops, s["sclk_mhz"])
    for k in ("lse_combine", "dlogits", "finalize"):
        assert st[k]["launches"] > 0 and st[k]["sclk_mhz"] == 0.0
    f.profile_enable(True)                                   # resets the statistics and the counters
    f.forward_backward(x, W, t, chunk=C)
    torch.cuda.synchronize()
    st2 = f.profile_read()
    assert st2["dx"]["launches"] == chunks and 500.0 <= st2["dx"]["sclk_mhz"] <= 2600.0
    f.profile_enable(False)
    f.close()
