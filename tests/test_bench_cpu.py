"""Host-side logic of bench.py (no GPU): the one-GPU contract, the source fingerprint that
ties stored traffic counters to the kernels, and the CPU-baseline sample sizing."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _write(d, name, text):
    with open(os.path.join(d, name), "w") as f:
        f.write(text)


def test_source_hash_ignores_comments_and_layout(tmp_path):
    d = str(tmp_path)
    _write(d, "a.hip", "int f(int x) {\n  return x + 1;  // one\n}\n")
    _write(d, "b.hpp", "/* header */\nconstexpr int k = 4;\n")
    h0 = bench.kernel_source_hash(d)
    _write(d, "a.hip", "// new comment\nint f(int x) {\n    return x + 1;  /* still one */\n}\n")
    assert bench.kernel_source_hash(d) == h0
    _write(d, "a.hip", "int f(int x) {\n  return x + 2;\n}\n")
    assert bench.kernel_source_hash(d) != h0
    _write(d, "notes.txt", "ignored: not a kernel source")
    _write(d, "a.hip", "int f(int x) {\n  return x + 1;\n}\n")
    assert bench.kernel_source_hash(d) == h0


def test_traffic_record_matches_current_sources_only(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    rec = {"llama3_vocab/4096/dw": {"bytes_per_launch": 123, "source_hash": bench.kernel_source_hash()},
           "llama3_vocab/4096/dx": {"bytes_per_launch": 456, "source_hash": "stale"}}
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("dw", "llama3_vocab", 4096) == 123
    assert bench.measured_traffic("dx", "llama3_vocab", 4096) is None       # taken on other code
    assert bench.measured_traffic("logits_lse", "llama3_vocab", 4096) is None


def test_committed_traffic_records_carry_a_hash():
    with open(bench.TRAFFIC_FILE) as fh:
        rec = json.load(fh)
    assert rec, "profiles/traffic.json is empty"
    for k, e in rec.items():
        assert len(k.split("/")) == 3 and e["bytes_per_launch"] > 0 and len(e["source_hash"]) == 16


def test_cpu_baseline_sample_is_a_prefix_of_the_workload():
    """The timed oracle sample uses the workload's first tokens (seeded draws are prefix-stable)."""
    import numpy as np
    from flce_inputs import make_inputs
    small, large = make_inputs(32, 16, 50, "bf16", 3), make_inputs(100, 16, 50, "bf16", 3)
    assert np.array_equal(small["x"], large["x"][:32]) and np.array_equal(small["t"], large["t"][:32])


def test_host_info_fields():
    info = bench.host_info()
    assert set(info) == {"cpu_model", "blas", "host_ram_gb"}
    assert info["host_ram_gb"] is None or info["host_ram_gb"] > 0


if __name__ == "__main__":
    sys.exit(pytest.main([__file__, "-q"]))
