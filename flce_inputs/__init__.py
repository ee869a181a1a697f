"""Seeded synthetic inputs for fused linear cross-entropy (FLCE).

This module is shared by the CPU oracle (``oracle/``), the tests and the
benchmark.  It holds no arithmetic of the method itself: it only draws
random numbers and converts them to the storage formats the GPU path reads
(bf16 bit patterns or fp32), so that the oracle and the HIP library see
byte-identical inputs.

Workloads (hidden states x[N,H], LM-head weight W[V,H], targets t[N]):
x ~ N(0,1), W ~ N(0, 0.02^2), targets uniform in [0,V) (or truncated Zipf
with exponent 1.1 over vocabulary ids for the Qwen3-vocabulary workload).
The vocabulary sizes are the ones the "Unsloth deep architecture" page
(techknowgenie.com) lists under "vocabulary explosion" (Llama 2: 32,000;
Llama 3: 128,256) and the Qwen3 size from the "Fused Linear Cross-Entropy"
page (42jerrykim.github.io), section "why the logits tensor is so large"
(151,936 with hidden 4,096).

Generation: numpy ``Generator(PCG64)`` seeded with ``SeedSequence(seed)``
spawned into three independent streams (x, W, t).  Floats are drawn in
fp32 and rounded to bf16 with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "bf16_bits_from_f32", "f32_from_bf16_bits",
    "make_inputs", "zipf_targets", "digest",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    N: int
    H: int
    V: int
    dtype: str            # "fp32" or "bf16": storage/compute type of x, W
    targets: str          # "uniform" or "zipf"
    chunk: int            # token chunk used by the chunked variant
    seed: int
    desc: str


# The five synthetic workloads (sizes as named; data is random, no dataset).
WORKLOADS: Dict[str, Workload] = {
    "tiny_fp32": Workload("tiny_fp32", 256, 256, 4096, "fp32", "uniform", 256, 1,
                          "tiny FLCE, fp32, N=256 H=256 V=4096"),
    "llama2_vocab": Workload("llama2_vocab", 8192, 4096, 32000, "bf16", "uniform", 2048, 2,
                             "Llama-2 vocab, bf16, N=8192 (2x4096) H=4096 V=32000, C=2048"),
    "llama3_vocab": Workload("llama3_vocab", 16384, 4096, 128256, "bf16", "uniform", 4096, 3,
                             "Llama-3 vocab, bf16, N=16384 (1x16384) H=4096 V=128256"),
    "qwen3_vocab": Workload("qwen3_vocab", 16384, 4096, 151936, "bf16", "zipf", 4096, 4,
                            "Qwen3 vocab, bf16, N=16384 (4x4096) H=4096 V=151936, Zipf(1.1) targets"),
    "long_context": Workload("long_context", 131072, 4096, 128256, "bf16", "uniform", 4096, 5,
                             "long context, bf16, N=131072 (1x128K) H=4096 V=128256"),
    # one GPU's share of the Llama-3 workload when it is split 8 ways (the path itself runs on one
    # GPU): by tokens (data parallel: N/8 rows, all of W) or by vocabulary (V/8 rows of W, all N)
    "llama3_dp8_share": Workload("llama3_dp8_share", 2048, 4096, 128256, "bf16", "uniform", 2048, 6,
                                 "Llama-3 vocab, token shard of 8: N=2048 H=4096 V=128256"),
    "llama3_tp8_share": Workload("llama3_tp8_share", 16384, 4096, 16032, "bf16", "uniform", 4096, 7,
                                 "Llama-3 vocab, vocabulary shard of 8: N=16384 H=4096 V=16032"),
}


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round-to-nearest-even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    out = np.empty(a.shape, dtype=np.uint16)
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_u.size, step):
        b = flat_u[s:s + step]
        r = (b + (np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
        nan = (b & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
        if nan.any():
            r = np.where(nan, (b >> np.uint32(16)) | np.uint32(0x40), r)
        flat_o[s:s + step] = r.astype(np.uint16)
    return out


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def zipf_targets(rng: np.random.Generator, n: int, V: int, s: float = 1.1) -> np.ndarray:
    """Truncated Zipf over ids 0..V-1: p(k) proportional to (k+1)^-s, by inverse CDF."""
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(n)
    idx = np.searchsorted(cdf, u, side="right")
    return np.minimum(idx, V - 1).astype(np.int64)


def _normal_f32(rng: np.random.Generator, shape, scale: float) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return a


def make_inputs(N: int, H: int, V: int, dtype: str = "bf16", seed: int = 0,
                targets: str = "uniform", w_std: float = 0.02,
                x_std: float = 1.0) -> Dict[str, np.ndarray]:
    """Draw one seeded input set.

    Returns a dict with
      ``x``: [N,H] and ``W``: [V,H] in storage form (uint16 bf16 bits for
             dtype "bf16", float32 for dtype "fp32"),
      ``t``: [N] int64 targets,
      ``dtype``: the storage dtype string.
    """
    if dtype not in ("bf16", "fp32"):
        raise ValueError(f"unknown dtype {dtype!r}")
    ss = np.random.SeedSequence(seed)
    sx, sw, st = ss.spawn(3)
    rx, rw, rt = (np.random.Generator(np.random.PCG64(s)) for s in (sx, sw, st))
    x = _normal_f32(rx, (N, H), x_std)
    W = _normal_f32(rw, (V, H), w_std)
    if targets == "uniform":
        t = rt.integers(0, V, size=N, dtype=np.int64)
    elif targets == "zipf":
        t = zipf_targets(rt, N, V, 1.1)
    else:
        raise ValueError(f"unknown target distribution {targets!r}")
    if dtype == "bf16":
        x = bf16_bits_from_f32(x)
        W = bf16_bits_from_f32(W)
    return {"x": x, "W": W, "t": t, "dtype": dtype}


def workload_inputs(w: Workload, N: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Inputs of a named workload, optionally with only the first N tokens' draw size."""
    return make_inputs(N if N is not None else w.N, w.H, w.V, w.dtype, w.seed, w.targets)


def as_float(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Storage form -> float32 values (exact)."""
    if dtype == "bf16":
        return f32_from_bf16_bits(arr)
    return np.asarray(arr, dtype=np.float32)


def digest(d: Dict[str, np.ndarray]) -> str:
    """SHA-256 over the stored bytes of x, W, t (a manifest fingerprint)."""
    h = hashlib.sha256()
    for k in ("x", "W", "t"):
        h.update(np.ascontiguousarray(d[k]).tobytes())
    return h.hexdigest()
