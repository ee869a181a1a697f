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
    # id, N, H, V, chunk, fp32 gradients: "" (bf16 dx and dW: pass 2 per chunk, dW stored by its one
    # product), "dx+dW" (one pass 2 over all tokens, atomics into both), "dx" or "dW" (per chunk)
    ("ragged", 1000, 512, 5000, 384, ""),
    ("ragged_fp32_grads", 1000, 512, 5000, 384, "dx+dW"),
    ("ragged_fp32_dx_bf16_dW", 1000, 512, 5000, 384, "dx"),
    ("ragged_bf16_dx_fp32_dW", 1000, 512, 5000, 384, "dW"),
    ("N1", 1, 64, 1001, 0, ""),
    ("H64_V1001", 300, 64, 1001, 128, ""),
    ("H320_V2049", 700, 320, 2049, 256, ""),
    ("one_chunk", 512, 256, 3000, 0, "dx+dW"),
    # a 20,000-token chunk with bf16 dW: pass 2 in launches of at most 16,384 tokens (one token block
    # each), the second adding into the dW tiles the first stored
    ("long_chunk_bf16", 20000, 128, 3000, 20000, ""),
    ("long_chunk_fp32_dx", 20000, 128, 3000, 20000, "dx"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_fused_small_vs_oracle(case):
    import torch
    name, N, H, V, chunk, g32 = case
    d = make_inputs(N, H, V, "bf16", seed=N + V)
    gx = torch.float32 if "dx" in g32 else None
    gw = torch.float32 if "dW" in g32 else None
    got = run_flce(d, chunk=chunk, dx_dtype=gx, dw_dtype=gw, variant=FUSED)
    got["handle"].close()
    compare(got, oracle_full(d), d["t"], V, 2e-2, 1e-4, "fused " + name)


def test_fused_workspace_within_the_memory_bar():
    """Peak extra HBM of the fused variant at the Llama-3 size stays within 2 GB for every gradient
    dtype: bf16 dW is stored by its one product per chunk (no V x H fp32 accumulator)."""
    import torch
    from linear_cross_entropy_token_amd import FusedLinearCrossEntropy
    w = WORKLOADS["llama3_vocab"]
    for gx, gw in ((None, None), (torch.float32, None), (None, torch.float32), (torch.float32, torch.float32)):
        f = FusedLinearCrossEntropy(dx_dtype=gx, dw_dtype=gw, variant=FUSED)
        ws = f.workspace_bytes(w.N, w.H, w.V, w.chunk)
        f.close()
        print(f"[fused workspace] dx {gx} dW {gw}: {ws / 1e9:.3f} GB", flush=True)
        assert 0 < ws <= 1.7e9


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
