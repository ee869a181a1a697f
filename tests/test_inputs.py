"""The seeded input generator (CPU only)."""
import numpy as np

from flce_inputs import (bf16_bits_from_f32, f32_from_bf16_bits, make_inputs, zipf_targets,
                         digest, WORKLOADS)


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,
                     -2.5, 65504.0, 1e-40], dtype=np.float32)
    bits = bf16_bits_from_f32(vals)
    back = f32_from_bf16_bits(bits)
    assert back[0] == 1.0
    assert back[1] == 1.0                      # tie -> even
    assert back[2] == 1.0 + 4 * 2 ** -8        # tie -> even (up)
    assert back[3] == 1.0 + 2 * 2 ** -8        # above the tie -> up
    assert back[4] == -2.5
    assert back[5] == 65536.0
    # every result is within half a bf16 ulp
    rel = np.abs(back[:6] - vals[:6]) / np.abs(vals[:6])
    assert np.all(rel <= 2.0 ** -8)


def test_bf16_nan_stays_nan():
    bits = bf16_bits_from_f32(np.array([np.nan, np.inf, -np.inf], dtype=np.float32))
    back = f32_from_bf16_bits(bits)
    assert np.isnan(back[0]) and back[1] == np.inf and back[2] == -np.inf


def test_deterministic_and_seed_sensitive():
    a = make_inputs(16, 8, 100, "bf16", seed=3)
    b = make_inputs(16, 8, 100, "bf16", seed=3)
    c = make_inputs(16, 8, 100, "bf16", seed=4)
    assert digest(a) == digest(b) != digest(c)
    assert a["x"].dtype == np.uint16 and a["t"].dtype == np.int64
    assert a["t"].min() >= 0 and a["t"].max() < 100


def test_token_prefix_is_stable():
    """Drawing fewer tokens yields the first rows of the larger draw (bounded samples)."""
    a = make_inputs(64, 8, 50, "fp32", seed=9)
    b = make_inputs(16, 8, 50, "fp32", seed=9)
    assert np.array_equal(a["x"][:16], b["x"]) and np.array_equal(a["t"][:16], b["t"])
    assert np.array_equal(a["W"], b["W"])


def test_distributions():
    d = make_inputs(4096, 64, 1000, "fp32", seed=0)
    assert abs(d["x"].std() - 1.0) < 0.02
    assert abs(d["W"].std() - 0.02) < 0.001


def test_zipf_skew():
    rng = np.random.Generator(np.random.PCG64(0))
    V = 151936
    t = zipf_targets(rng, 200000, V, 1.1)
    top = np.mean(t == 0)
    w = np.arange(1, V + 1, dtype=np.float64) ** -1.1
    assert abs(top - w[0] / w.sum()) < 0.005
    assert t.min() >= 0 and t.max() < V


def test_workload_table():
    w = WORKLOADS["llama3_vocab"]
    assert (w.N, w.H, w.V, w.dtype) == (16384, 4096, 128256, "bf16")
    assert WORKLOADS["qwen3_vocab"].targets == "zipf"
    assert WORKLOADS["tiny_fp32"].dtype == "fp32"
    # one GPU's shares of the Llama-3 workload split 8 ways: by tokens and by vocabulary
    dp, tp = WORKLOADS["llama3_dp8_share"], WORKLOADS["llama3_tp8_share"]
    assert (dp.N * 8, dp.H, dp.V) == (w.N, w.H, w.V)
    assert (tp.N, tp.H, tp.V * 8) == (w.N, w.H, w.V)
