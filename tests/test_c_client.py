"""The C ABI from plain C: tests/c/flce_c_client.c (C99, no C++ or Python in its process), built by
the package build next to libflce.so.  Host mode runs here; device mode checks the W = 0 closed
form (loss = ln V, dx = 0, dW per row) for fp32 and bf16 inputs, and the argument and data errors."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "c", "flce_c_client")


def _run(mode, timeout):
    if not os.path.exists(CLIENT):
        pytest.fail(f"{CLIENT} is missing: build it with `python -m linear_cross_entropy_token_amd.build`")
    print(f"[c client] {mode}", flush=True)
    r = subprocess.run([CLIENT, mode], capture_output=True, text=True, timeout=timeout)
    assert r.returncode == 0 and f"PASS {mode}" in r.stdout, f"rc={r.returncode}\n{r.stdout}\n{r.stderr}"
    return r.stdout


def test_c_client_host():
    _run("host", 60)


@pytest.mark.gpu
def test_c_client_device():
    out = _run("device", 120)
    assert out.count("ok  W = 0 closed form") == 2
