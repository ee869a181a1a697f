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


def test_fused_full_size_sampled_llama3():
    """Llama-3-vocabulary workload at full size with the fused variant (fp32 gradients, so the
    exact invariants apply): sampled lse / dx rows against the oracle, dW column sums and
    <x,dx> = <W,dW>."""
    import torch
    w = WORKLOADS["llama3_vocab"]
    print(f"[fused full-size] {w.name} N={w.N} H={w.H} V={w.V} chunk={w.chunk}", flush=True)
    d = make_inputs(w.N, w.H, w.V, w.dtype, w.seed, w.targets)
    got = run_flce(d, chunk=w.chunk, with_lse=True, dx_dtype=torch.float32, dw_dtype=torch.float32,
                   variant=FUSED)
    got["handle"].close()
    rows = [0, 1, 777, w.chunk - 1, w.chunk, w.N // 2, w.N - 1]
    W64 = oracle.widen(d["W"], "bf16")
    want = oracle.flce_rows(oracle.widen(d["x"][rows], "bf16"), W64, d["t"][rows], range(len(rows)), w.N)
    assert np.max(np.abs(got["lse"][rows] - want["lse"])) <= 1e-4 * np.max(np.abs(want["lse"]))
    assert rel_fro(got["dx"][rows], want["dx"]) <= 2e-2
    assert abs(got["loss"] - (math.log(w.V) + 2e-4 * w.H)) < 0.1
    dW = got["dW"]
    assert np.linalg.norm(dW.sum(axis=0)) <= 1e-3 * np.linalg.norm(dW)
    x64 = oracle.widen(d["x"], "bf16")
    a = float(np.sum(x64 * got["dx"]))
    b = float(np.sum(W64 * dW))
    assert abs(a - b) <= 1e-3 * max(abs(a), abs(b))
