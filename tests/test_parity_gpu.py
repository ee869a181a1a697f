"""HIP path vs the CPU oracle (GPU only).

Element-wise comparisons at sizes the oracle finishes in seconds (several
tiles, ragged chunk and vocabulary tails, edge cases), and the exact W = 0
closed form at the Llama-3-vocabulary size (the full-size comparisons with the
whole oracle are in tests/test_full_size_gpu.py).

Tolerances (written in each assert): loss relative error <= 1e-4; dx and dW
relative Frobenius error <= 2e-2 for bf16 inputs and <= 1e-5 for fp32 inputs,
also on the dW rows no target hits (pure softmax part).
"""
import math
import zlib

import numpy as np
import pytest

import oracle
from flce_inputs import make_inputs, WORKLOADS
from flce_testlib import (require_gpu, run_flce, compare, oracle_full, rel_fro, to_device, to_f64)

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp32": 1e-5}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


SMALL = [
    # id, N, H, V, dtype, chunk, grads dtype
    ("tiny_fp32_C256", 256, 256, 4096, "fp32", 256, None),
    ("tiny_fp32_C64", 256, 256, 4096, "fp32", 64, None),
    ("fp32_ragged", 333, 96, 777, "fp32", 100, None),
    ("bf16_ragged", 1000, 512, 5000, "bf16", 384, None),
    ("bf16_ragged_fp32_grads", 1000, 512, 5000, "bf16", 384, "fp32"),
    ("bf16_N1", 1, 64, 1001, "bf16", 0, None),
    ("bf16_H64_V1001", 300, 64, 1001, "bf16", 128, None),
    ("bf16_one_chunk", 512, 256, 3000, "bf16", 0, None),
    # H = 264: a partial last k-slice in the logits GEMM and a partial second column tile in
    # the dx and dW epilogues (dW read-modify-write over three chunks)
    ("bf16_H264", 520, 264, 1300, "bf16", 200, None),
    ("bf16_H264_fp32_grads", 520, 264, 1300, "bf16", 200, "fp32"),
    ("fp32_H264", 200, 264, 900, "fp32", 64, None),
    # contractions of one or two k-slices in both LDS rings: H = 32 / 64 / 128 for the logits,
    # a vocabulary of one or two tiles for dx, chunks of 40 / 64 / 96 / 100 tokens for dW
    ("bf16_V50_H64", 64, 64, 50, "bf16", 0, None),
    ("bf16_V300_H128_N100", 100, 128, 300, "bf16", 0, None),
    ("fp32_V50_H32", 40, 32, 50, "fp32", 0, None),
    ("bf16_C96_V700", 300, 192, 700, "bf16", 96, None),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c[0])
def test_small_vs_oracle(case):
    name, N, H, V, dt, chunk, gdt = case
    d = make_inputs(N, H, V, dt, seed=zlib.crc32(name.encode()) % 1000)
    import torch
    gd = {"fp32": torch.float32, None: None}[gdt]
    got = run_flce(d, chunk=chunk, dx_dtype=gd, dw_dtype=gd)
    want = oracle_full(d)
    compare(got, want, d["t"], V, TOL[dt], 1e-4, name)


def test_tiny_fp32_workload_exact_config():
    """The tiny fp32 workload as named (N=256, H=256, V=4096, seeded), tolerance 1e-5."""
    w = WORKLOADS["tiny_fp32"]
    d = make_inputs(w.N, w.H, w.V, w.dtype, w.seed, w.targets)
    got = run_flce(d, chunk=w.chunk, with_lse=True)
    want = oracle_full(d)
    compare(got, want, d["t"], w.V, 1e-5, 1e-5, "tiny_fp32")
    assert np.max(np.abs(got["lse"] - want["lse"])) <= 1e-5 * np.max(np.abs(want["lse"]))


@pytest.mark.parametrize("V,zipf", [(128256, False), (151936, True)])
def test_full_vocab_reduced_tokens(V, zipf):
    """Full H and V of the Llama-3 / Qwen3 workloads at N=256 (two chunks of 128)."""
    d = make_inputs(256, 4096, V, "bf16", seed=V, targets="zipf" if zipf else "uniform")
    got = run_flce(d, chunk=128, with_lse=True)
    want = oracle_full(d)
    compare(got, want, d["t"], V, 2e-2, 1e-4, f"V={V}")
    assert np.max(np.abs(got["lse"] - want["lse"])) <= 1e-4


def test_target_extremes_and_collisions():
    N, H, V = 600, 128, 2000
    d = make_inputs(N, H, V, "bf16", seed=21)
    d["t"] = np.where(np.arange(N) % 2 == 0, 0, V - 1).astype(np.int64)
    compare(run_flce(d, chunk=256), oracle_full(d), d["t"], V, 2e-2, 1e-4, "targets {0,V-1}")
    d["t"] = np.full(N, 7, dtype=np.int64)
    compare(run_flce(d, chunk=256), oracle_full(d), d["t"], V, 2e-2, 1e-4, "all targets equal")


def test_zero_target_row_isolates_softmax_part():
    """Append a zero row to W and aim every target at it: the one-hot part of dx is
    -W[t]/N = 0, so dx is pure softmax and the 2e-2 bound tests that part alone."""
    N, H, V = 512, 256, 3000
    d = make_inputs(N, H, V - 1, "bf16", seed=22)
    d["W"] = np.concatenate([d["W"], np.zeros((1, H), dtype=np.uint16)], axis=0)
    d["t"] = np.full(N, V - 1, dtype=np.int64)
    got = run_flce(d, chunk=200)
    want = oracle_full(d)
    assert rel_fro(got["dx"], want["dx"]) <= 2e-2
    compare(got, want, d["t"], V, 2e-2, 1e-4, "zero target row")


def test_chunk_invariance_and_determinism():
    N, H, V = 1024, 256, 4000
    d = make_inputs(N, H, V, "bf16", seed=23)
    want = oracle_full(d)
    outs = []
    for c in (1024, 384, 100):
        r = run_flce(d, chunk=c)
        compare(r, want, d["t"], V, 2e-2, 1e-4, f"chunk={c}")
        outs.append(r)
    again = run_flce(d, chunk=384)
    assert again["loss"] == outs[1]["loss"]
    assert np.array_equal(again["dx"], outs[1]["dx"]) and np.array_equal(again["dW"], outs[1]["dW"])
    # the chunk size changes only rounding order (dW accumulation across chunks)
    assert rel_fro(outs[0]["dW"], outs[2]["dW"]) <= 1e-2
    assert rel_fro(outs[0]["dx"], outs[2]["dx"]) <= 1e-3


def test_out_of_range_target_sets_flag_without_fault():
    from linear_cross_entropy_token_amd import FusedLinearCrossEntropy
    N, H, V = 300, 64, 500
    d = make_inputs(N, H, V, "bf16", seed=24)
    for bad in (V, -1):
        d["t"][5] = bad
        f = FusedLinearCrossEntropy()
        r = run_flce(d, chunk=128, handle=f)
        assert math.isnan(r["loss"])
        assert np.all(np.isfinite(r["dx"])) and np.all(np.isfinite(r["dW"]))
        assert f.check() == 5          # FLCE_ERR_DATA
        assert f.check() == 0          # the flag is cleared by the check
        f.close()


def test_reuse_handle_across_shapes():
    from linear_cross_entropy_token_amd import FusedLinearCrossEntropy
    f = FusedLinearCrossEntropy()
    for (N, H, V, c) in ((700, 128, 3000, 256), (200, 64, 900, 0), (900, 256, 5000, 512)):
        d = make_inputs(N, H, V, "bf16", seed=N)
        compare(run_flce(d, chunk=c, handle=f), oracle_full(d), d["t"], V, 2e-2, 1e-4, f"{N},{H},{V}")
    f.close()


# ---- full workload sizes: tests/test_full_size_gpu.py holds the whole-oracle comparisons ----

def test_full_size_zero_weight_closed_form():
    """W = 0 at the Llama-3-vocabulary size: loss = ln V, dx = 0 and
    dW[v] = (1/V) mean_n x_n - (1/N) sum_{n: t_n = v} x_n, exactly in the mathematics."""
    w = WORKLOADS["llama3_vocab"]
    d = make_inputs(w.N, w.H, w.V, w.dtype, w.seed, w.targets)
    d["W"] = np.zeros_like(d["W"])
    got = run_flce(d, chunk=w.chunk)
    assert abs(got["loss"] - math.log(w.V)) <= 1e-4 * math.log(w.V)
    assert np.all(got["dx"] == 0.0)
    x64 = oracle.widen(d["x"], "bf16")
    expect = np.empty((w.V, w.H))
    expect[:] = x64.mean(axis=0) / w.V
    np.subtract.at(expect, d["t"], x64 / w.N)
    assert rel_fro(got["dW"], expect) <= 2e-2
    untargeted = np.ones(w.V, dtype=bool)
    untargeted[d["t"]] = False
    assert rel_fro(got["dW"][untargeted], expect[untargeted]) <= 2e-2
    got["handle"].close()


@pytest.mark.parametrize("variant", [0, 1], ids=["chunked", "fused"])
@pytest.mark.parametrize("scale", [25.0, 100.0])
def test_large_logits(variant, scale):
    """W scaled so that |z| reaches ~40 / ~160 (a peaked softmax).  The chunked variant's bf16
    buffer holds z minus the row's 256-column tile maximum, so its accuracy does not depend on the
    logit scale (rounding z itself would put the gradients 3% / 13% off at these scales); the
    fused variant forms G from the fp32 accumulators."""
    from flce_inputs import bf16_bits_from_f32
    d = make_inputs(512, 256, 4096, "bf16", seed=211)
    d["W"] = bf16_bits_from_f32((oracle.widen(d["W"], "bf16") * scale).astype(np.float32))
    want = oracle_full(d)
    got = run_flce(d, chunk=256, variant=variant)
    got["handle"].close()
    compare(got, want, d["t"], 4096, 2e-2, 1e-4, f"scale {scale}, variant {variant}")
