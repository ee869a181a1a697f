"""Metamorphic relations of the definition on the HIP path (GPU only).

* Shift invariance: W -> W + 1 u^T adds <x_n, u> to every logit of token n, which softmax
  cross-entropy ignores (the per-row shift of the CE equations on the "Unsloth deep
  architecture" page).  With fp32 inputs and |z| past 100, a kernel without the running-maximum
  subtraction would overflow exp (e^89 > fp32 max); the chunked path's buffer stores z minus
  the tile maximum and must stay exact.
* Token permutation: permuting the rows of x (and t) permutes the rows of dx and leaves the loss
  and dW unchanged; vocabulary permutation: permuting the rows of W (relabelling t) permutes the
  rows of dW and leaves the loss and dx unchanged.
* The chunk size changes nothing but rounding (the FLCE page's core idea; tests/test_parity_gpu.py).

Tolerances.  Unshifted fp32: 1e-5 (the fp32 bar).  Shifted fp32: the logits are ~190, so the fp32
sum that forms each of them carries an absolute error of up to ~sqrt(H) |z| 2^-24 ~ 1e-4, which
moves each softmax entry by that much relatively; the bound for the shifted case is therefore
2e-4 on the loss and 1e-3 on the gradients, against both the oracle on the shifted inputs and
the unshifted run.  bf16 permutations: the stated bf16 bars (loss 1e-4, gradients 2e-2); dx under
a token permutation is compared bitwise, because every dx row depends on its own token alone
and each kernel treats every row alike.
"""
import numpy as np
import pytest

from flce_inputs import make_inputs
from flce_testlib import require_gpu, run_flce, compare, oracle_full, rel_fro

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_shift_invariance_fp32_chunked():
    N, H, V = 512, 256, 4096
    d = make_inputs(N, H, V, "fp32", seed=401)
    base = run_flce(d, chunk=192, with_lse=True)
    base["handle"].close()
    compare(base, oracle_full(d), d["t"], V, 1e-5, 1e-5, "unshifted")
    # x gets mean 1 so that <x_n, u> ~ 0.75 H = 192 for u = 0.75: |z| past 100 on every row
    sh = dict(d)
    sh["x"] = (d["x"] + np.float32(1.0)).astype(np.float32)
    u = np.full(H, 0.75, dtype=np.float32)
    plain = dict(sh)
    sh["W"] = (d["W"] + u[None, :]).astype(np.float32)
    z_abs = np.abs(sh["x"].astype(np.float64) @ sh["W"].astype(np.float64).T).min()
    assert z_abs > 100, z_abs
    got = run_flce(sh, chunk=192, with_lse=True)
    got["handle"].close()
    ref = run_flce(plain, chunk=192, with_lse=True)       # the same x without the shift
    ref["handle"].close()
    errs = compare(got, oracle_full(sh), sh["t"], V, 1e-3, 2e-4, "shifted vs oracle")
    print(f"[shift] |z| >= {z_abs:.1f}; against the oracle: {errs}", flush=True)
    # the relation itself: shifted and unshifted runs agree
    assert abs(got["loss"] - ref["loss"]) <= 2e-4 * abs(ref["loss"])
    assert rel_fro(got["dx"], ref["dx"]) <= 1e-3
    assert rel_fro(got["dW"], ref["dW"]) <= 1e-3
    assert np.max(np.abs((got["lse"] - ref["lse"]) - (sh["x"].astype(np.float64) @ u))) <= 1e-3


@pytest.mark.parametrize("variant", [0, 1], ids=["chunked", "fused"])
def test_token_permutation(variant):
    N, H, V, C = 1000, 512, 5000, 384
    d = make_inputs(N, H, V, "bf16", seed=402)
    p = np.random.default_rng(402).permutation(N)
    a = run_flce(d, chunk=C, variant=variant)
    a["handle"].close()
    dp = dict(d, x=d["x"][p], t=d["t"][p])
    b = run_flce(dp, chunk=C, variant=variant)
    b["handle"].close()
    assert abs(b["loss"] - a["loss"]) <= 1e-4 * abs(a["loss"])
    if variant == 0:
        assert np.array_equal(b["dx"], a["dx"][p])
    else:   # fp32 atomics add the partials in any order
        assert rel_fro(b["dx"], a["dx"][p]) <= 2e-2
    err_w = rel_fro(b["dW"], a["dW"])
    print(f"[token permutation] variant {variant}: dW {err_w:.2e}", flush=True)
    assert err_w <= 2e-2
    compare(b, oracle_full(dp), dp["t"], V, 2e-2, 1e-4, "token-permuted vs oracle")


@pytest.mark.parametrize("variant", [0, 1], ids=["chunked", "fused"])
def test_vocabulary_permutation(variant):
    N, H, V, C = 1000, 512, 5000, 384
    d = make_inputs(N, H, V, "bf16", seed=403)
    pv = np.random.default_rng(403).permutation(V)
    inv = np.argsort(pv)
    a = run_flce(d, chunk=C, variant=variant)
    a["handle"].close()
    dv = dict(d, W=d["W"][pv], t=inv[d["t"]])
    b = run_flce(dv, chunk=C, variant=variant)
    b["handle"].close()
    err_x, err_w = rel_fro(b["dx"], a["dx"]), rel_fro(b["dW"], a["dW"][pv])
    print(f"[vocabulary permutation] variant {variant}: dx {err_x:.2e} dW {err_w:.2e}", flush=True)
    assert abs(b["loss"] - a["loss"]) <= 1e-4 * abs(a["loss"])
    assert err_x <= 2e-2 and err_w <= 2e-2
    compare(b, oracle_full(dv), dv["t"], V, 2e-2, 1e-4, "vocabulary-permuted vs oracle")
