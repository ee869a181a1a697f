"""The fused (two-pass, no logits buffer) variant vs the CPU oracle (GPU only).

Same tolerances as the chunked variant: loss relative error <= 1e-4, dx and dW
relative Frobenius error <= 2e-2 (bf16 inputs), also on never-targeted dW rows.
The fused variant adds dx/dW partials with fp32 atomics, so it is compared
within tolerance, never bitwise.
"""
import math

import numpy as np
import pytest

import oracle
from flce_inputs import make_inputs, WORKLOADS
from flce_testlib import require_gpu, run_flce, compare, oracle_full, rel_fro

pytestmark = pytest.mark.gpu
FUSED = 1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


CASES = [
    # id, N, H, V, chunk, grads fp32
    ("ragged", 1000, 512, 5000, 384, False),
    ("ragged_fp32_grads", 1000, 512, 5000, 384, True),
    ("N1", 1, 64, 1001, 0, False),
    ("H64_V1001", 300, 64, 1001, 128, False),
    ("one_chunk", 512, 256, 3000, 0, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_fused_small_vs_oracle(case):
    import torch
    name, N, H, V, chunk, g32 = case
    d = make_inputs(N, H, V, "bf16", seed=N + V)
    gd = torch.float32 if g32 else None
    got = run_flce(d, chunk=chunk, dx_dtype=gd, dw_dtype=gd, variant=FUSED)
    got["handle"].close()
    compare(got, oracle_full(d), d["t"], V, 2e-2, 1e-4, "fused " + name)


def test_fused_full_vocab_reduced_tokens():
    d = make_inputs(256, 4096, 128256, "bf16", seed=31)
    got = run_flce(d, chunk=128, with_lse=True, variant=FUSED)
    got["handle"].close()
    want = oracle_full(d)
    compare(got, want, d["t"], 128256, 2e-2, 1e-4, "fused V=128256")
    assert np.max(np.abs(got["lse"] - want["lse"])) <= 1e-4


def test_fused_matches_chunked():
    import torch
    N, H, V = 1024, 512, 6000
    d = make_inputs(N, H, V, "bf16", seed=32)
    a = run_flce(d, chunk=512, dx_dtype=torch.float32, dw_dtype=torch.float32)
    b = run_flce(d, chunk=512, dx_dtype=torch.float32, dw_dtype=torch.float32, variant=FUSED)
    a["handle"].close()
    b["handle"].close()
    assert a["loss"] == b["loss"]            # pass 1 is the same statistics kernel
    assert rel_fro(b["dx"], a["dx"]) <= 1e-2 and rel_fro(b["dW"], a["dW"]) <= 1e-2


def test_fused_out_of_range_target_flags():
    from linear_cross_entropy_token_amd import FusedLinearCrossEntropy
    d = make_inputs(300, 64, 500, "bf16", seed=33)
    d["t"][7] = 500
    f = FusedLinearCrossEntropy(variant=FUSED)
    r = run_flce(d, chunk=128, handle=f)
    assert math.isnan(r["loss"]) and np.all(np.isfinite(r["dW"]))
    assert f.check() == 5
    f.close()
