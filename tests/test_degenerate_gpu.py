"""Degenerate shapes of the method, both variants, through the C ABI:
  * one class (V = 1): every token's softmax is 1 at its target, so the loss is exactly 0 and
    dx = dW = 0 exactly (lse = z_t in fp32: the tile's sum of exp(z - max) is exactly 1);
  * two classes (V = 2): per token the loss is softplus(z_other - z_target);
  * the smallest hidden size the ABI takes (H = 8) and a single token (N = 1);
each against the oracle at the stated tolerances (loss <= 1e-4 relative or, where the loss is 0,
exactly 0; dx, dW <= 2e-2 relative Frobenius for bf16 inputs, <= 1e-5 for fp32)."""
import numpy as np
import pytest

from flce_inputs import make_inputs
from flce_testlib import require_gpu, run_flce, oracle_full, rel_fro

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp32": 1e-5}


# the fused variant takes bf16 inputs only
@pytest.mark.parametrize("variant,dtype", [(0, "bf16"), (0, "fp32"), (1, "bf16")],
                         ids=["chunked-bf16", "chunked-fp32", "fused-bf16"])
def test_one_class(variant, dtype):
    require_gpu()
    for N, H in ((300, 64), (1, 8)):
        d = make_inputs(N, H, 1, dtype, seed=191 + N)
        r = run_flce(d, chunk=128, with_lse=True, variant=variant)
        assert r["handle"].check() == 0
        assert r["loss"] == 0.0, r["loss"]
        assert np.all(r["dx"] == 0.0) and np.all(r["dW"] == 0.0)
        r["handle"].close()


SMALL = [(500, 64, 2, "bf16"), (300, 32, 2, "fp32"), (700, 8, 3000, "bf16"), (1, 8, 5, "fp32"),
         (1, 8, 1001, "bf16")]


@pytest.mark.parametrize("variant,N,H,V,dtype",
                         [(0, *c) for c in SMALL] + [(1, *c) for c in SMALL if c[3] == "bf16"])
def test_small_classes_and_hidden(variant, N, H, V, dtype):
    require_gpu()
    d = make_inputs(N, H, V, dtype, seed=197 + N + V)
    want = oracle_full(d)
    r = run_flce(d, chunk=256, variant=variant)
    assert r["handle"].check() == 0
    assert abs(r["loss"] - want["loss"]) <= 1e-4 * abs(want["loss"]), (r["loss"], want["loss"])
    assert rel_fro(r["dx"], want["dx"]) <= TOL[dtype]
    assert rel_fro(r["dW"], want["dW"]) <= TOL[dtype]
    r["handle"].close()
