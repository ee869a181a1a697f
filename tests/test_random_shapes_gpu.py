"""Seeded random shapes and options against the oracle: sizes drawn around the tile and slice
boundaries (multiples of 256 and 64, plus and minus a little), both variants, both input dtypes,
ignore_index and the sum reduction.  Every case prints its parameters before it runs."""
import numpy as np
import pytest

import oracle
from flce_inputs import make_inputs
from flce_testlib import rel_fro, require_gpu, to_device, to_f64

pytestmark = pytest.mark.gpu


def _draw(k):
    rng = np.random.default_rng(1000 + k)
    pick = lambda base: int(max(8, base + rng.integers(-9, 10)))
    N = int(rng.choice([1, 7, 64, 200, 255, 256, 257, 511, 640]))
    H = 8 * max(1, pick(int(rng.choice([32, 64, 96, 256, 264, 512]))) // 8)
    V = pick(int(rng.choice([50, 256, 300, 1000, 2048, 3000])))
    dtype = "fp32" if rng.random() < 0.25 else "bf16"
    variant = 1 if (dtype == "bf16" and rng.random() < 0.3) else 0
    chunk = int(rng.choice([0, 64, 100, 256]))
    reduction = "sum" if rng.random() < 0.3 else "mean"
    ignore = -100 if rng.random() < 0.4 else None
    return N, H, V, dtype, variant, chunk, reduction, ignore


CASES = [_draw(k) for k in range(32)]


@pytest.mark.parametrize("k", range(len(CASES)))
def test_random_case(k):
    N, H, V, dtype, variant, chunk, reduction, ignore = CASES[k]
    print(f"[random {k}] N={N} H={H} V={V} {dtype} variant={variant} chunk={chunk} "
          f"{reduction} ignore={ignore}", flush=True)
    torch = require_gpu()
    from linear_cross_entropy_token_amd import FusedLinearCrossEntropy
    d = make_inputs(N, H, V, dtype, seed=2000 + k)
    if ignore is not None and N > 1:
        d["t"] = d["t"].copy()
        d["t"][np.random.default_rng(k).random(N) < 0.25] = ignore
    want = oracle.flce_ext(oracle.widen(d["x"], dtype), oracle.widen(d["W"], dtype), d["t"],
                           reduction=reduction, ignore_index=ignore)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    f = FusedLinearCrossEntropy(in_dtype=tdt, dx_dtype=tdt, dw_dtype=tdt, variant=variant)
    x, W, t = to_device(d)
    loss, dx, dW = f.forward_backward(x, W, t, chunk=chunk, reduction=reduction, ignore_index=ignore)
    assert f.check() == 0
    f.close()
    tol = 1e-5 if dtype == "fp32" else 2e-2
    gl = float(loss.item())
    if np.isnan(want["loss"]):
        assert np.isnan(gl)
    else:
        assert abs(gl - want["loss"]) <= 1e-4 * max(abs(want["loss"]), 1e-30), (gl, want["loss"])
    if np.linalg.norm(want["dx"]) == 0:
        assert float(dx.abs().max().item()) == 0.0 and float(dW.abs().max().item()) == 0.0
        return
    edx, edw = rel_fro(to_f64(dx), want["dx"]), rel_fro(to_f64(dW), want["dW"])
    assert edx <= tol and edw <= tol, (edx, edw)
