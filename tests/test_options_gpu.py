"""GPU parity of the loss options (flce_forward_backward_opt) against the oracle's flce_ext.

Options: reduction "mean" / "sum", ignore_index (tokens whose target equals it count for
nothing), accumulation into dx / dW, and forward only.  Every case goes through the C ABI
(via the binding) and compares with the fp64 oracle on the same seeded inputs.
"""
import math

import numpy as np
import pytest

import oracle
from flce_inputs import make_inputs
from flce_testlib import rel_fro, require_gpu, to_device, to_f64

pytestmark = pytest.mark.gpu

BF16_GRAD_TOL = 2e-2
FP32_GRAD_TOL = 1e-5
LOSS_TOL = 1e-4


def _inputs(N, H, V, dtype, seed, ignore=None, frac=0.3):
    d = make_inputs(N, H, V, dtype, seed)
    if ignore is not None:
        rng = np.random.default_rng(seed + 1000)
        d["t"] = d["t"].copy()
        d["t"][rng.random(N) < frac] = ignore
    return d


def _oracle(d, reduction, ignore):
    return oracle.flce_ext(oracle.widen(d["x"], d["dtype"]), oracle.widen(d["W"], d["dtype"]), d["t"],
                           reduction=reduction, ignore_index=ignore)


def _handle(d, variant, grad_dtype=None):
    torch = require_gpu()
    from linear_cross_entropy_token_amd import FusedLinearCrossEntropy
    tdt = torch.bfloat16 if d["dtype"] == "bf16" else torch.float32
    g = grad_dtype or tdt
    return FusedLinearCrossEntropy(in_dtype=tdt, dx_dtype=g, dw_dtype=g, variant=variant)


def _check(got_loss, dx, dW, want, tol_grad, what):
    if math.isnan(want["loss"]):
        assert math.isnan(got_loss), f"{what}: loss {got_loss}, expected NaN"
    else:
        err = abs(got_loss - want["loss"]) / max(abs(want["loss"]), 1e-30)
        assert err <= LOSS_TOL, f"{what}: loss rel err {err}"
    if np.linalg.norm(want["dx"]) == 0:
        assert np.all(dx == 0) and np.all(dW == 0), f"{what}: gradients should be exactly zero"
        return
    edx, edw = rel_fro(dx, want["dx"]), rel_fro(dW, want["dW"])
    assert edx <= tol_grad and edw <= tol_grad, f"{what}: dx {edx} dW {edw}"


CASES = [
    # name, N, H, V, dtype, chunk, reduction, ignore, variant
    ("chunked_mean_ign-100", 700, 256, 3000, "bf16", 256, "mean", -100, 0),
    ("chunked_sum_ign-100", 700, 256, 3000, "bf16", 256, "sum", -100, 0),
    ("chunked_sum_noign", 300, 128, 1000, "bf16", 128, "sum", None, 0),
    ("chunked_mean_ign_in_range", 513, 64, 777, "bf16", 200, "mean", 5, 0),
    ("chunked_fp32_mean_ign", 256, 256, 4096, "fp32", 64, "mean", -1, 0),
    ("chunked_fp32_sum", 256, 256, 4096, "fp32", 256, "sum", None, 0),
    ("fused_mean_ign-100", 700, 256, 3000, "bf16", 256, "mean", -100, 1),
    ("fused_sum_ign-100", 600, 256, 2100, "bf16", 300, "sum", -100, 1),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_options_vs_oracle(case):
    name, N, H, V, dtype, chunk, reduction, ign, variant = case
    print(f"[options] {name}", flush=True)
    d = _inputs(N, H, V, dtype, seed=31 + CASES.index(case), ignore=ign)
    want = _oracle(d, reduction, ign)
    f = _handle(d, variant)
    x, W, t = to_device(d)
    loss, dx, dW = f.forward_backward(x, W, t, chunk=chunk, reduction=reduction, ignore_index=ign)
    assert f.check() == 0
    dxn, dWn = to_f64(dx), to_f64(dW)
    _check(float(loss.item()), dxn, dWn, want, FP32_GRAD_TOL if dtype == "fp32" else BF16_GRAD_TOL, name)
    if ign is not None:   # an ignored token's gradient row is exactly zero
        assert np.all(dxn[d["t"] == ign] == 0), f"{name}: nonzero dx row of an ignored token"


@pytest.mark.parametrize("variant", [0, 1], ids=["chunked", "fused"])
@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_all_tokens_ignored(variant, reduction):
    d = _inputs(300, 128, 1000, "bf16", seed=41, ignore=-100, frac=1.1)
    f = _handle(d, variant)
    x, W, t = to_device(d)
    loss, dx, dW = f.forward_backward(x, W, t, chunk=128, reduction=reduction, ignore_index=-100)
    assert f.check() == 0, "an ignored target must not raise the data flag"
    lv = float(loss.item())
    if reduction == "mean":
        assert math.isnan(lv), f"mean over zero counted tokens should be NaN, got {lv}"
    else:
        assert lv == 0.0
    assert float(dx.abs().max().item()) == 0.0 and float(dW.abs().max().item()) == 0.0


ACC_CASES = [
    # name, N, H, V, dtype, chunk, grad dtype, variant
    ("chunked_bf16_split", 700, 256, 3000, "bf16", 256, None, 0),
    ("chunked_bf16_fp32grads", 700, 256, 3000, "bf16", 256, "fp32", 0),
    ("chunked_fp32", 256, 256, 4096, "fp32", 64, None, 0),
    ("chunked_bf16_nosplit", 4096, 4096, 2048, "bf16", 4096, None, 0),
    ("fused_bf16", 600, 256, 2100, "bf16", 300, None, 1),
    ("fused_fp32grads", 600, 256, 2100, "bf16", 300, "fp32", 1),
]


@pytest.mark.parametrize("case", ACC_CASES, ids=[c[0] for c in ACC_CASES])
def test_accumulate(case):
    """dx, dW start from nonzero values of the gradients' size; the call adds its gradients."""
    name, N, H, V, dtype, chunk, gdt, variant = case
    print(f"[accumulate] {name}", flush=True)
    torch = require_gpu()
    d = _inputs(N, H, V, dtype, seed=51 + ACC_CASES.index(case), ignore=-100, frac=0.1)
    want = _oracle(d, "mean", -100)
    f = _handle(d, variant, torch.float32 if gdt == "fp32" else None)
    x, W, t = to_device(d)
    gen = torch.Generator(device="cuda").manual_seed(5)
    sx = float(np.sqrt(np.mean(want["dx"] ** 2)))
    sw = float(np.sqrt(np.mean(want["dW"] ** 2)))
    dx0 = (torch.randn(x.shape, device="cuda", generator=gen) * sx).to(f.dx_dtype)
    dW0 = (torch.randn(W.shape, device="cuda", generator=gen) * sw).to(f.dw_dtype)
    dx, dW = dx0.clone(), dW0.clone()
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    f.forward_backward(x, W, t, chunk=chunk, out=(loss, dx, dW, None), ignore_index=-100, accumulate=True)
    assert f.check() == 0
    # bf16 inputs keep a bf16 dlogits tile on either path, so fp32 outputs do not tighten the
    # gradient tolerance; only fp32 inputs do
    tol = FP32_GRAD_TOL if dtype == "fp32" else BF16_GRAD_TOL
    gx = to_f64(dx) - to_f64(dx0)
    gw = to_f64(dW) - to_f64(dW0)
    # bf16 outputs: one rounding of (start + gradient), relative to the gradient's size
    edx, edw = rel_fro(gx, want["dx"]), rel_fro(gw, want["dW"])
    assert edx <= tol and edw <= tol, f"{name}: accumulated dx {edx} dW {edw}"
    assert abs(float(loss.item()) - want["loss"]) / abs(want["loss"]) <= LOSS_TOL


@pytest.mark.parametrize("variant", [0, 1], ids=["chunked", "fused"])
def test_forward_only(variant):
    d = _inputs(700, 256, 3000, "bf16", seed=61, ignore=-100, frac=0.2)
    f = _handle(d, variant)
    x, W, t = to_device(d)
    for reduction in ("mean", "sum"):
        want = _oracle(d, reduction, -100)
        loss, lse = f.forward(x, W, t, chunk=256, with_lse=True, reduction=reduction, ignore_index=-100)
        loss_full, _, _, lse_full = f.forward_backward(x, W, t, chunk=256, with_lse=True, reduction=reduction,
                                                       ignore_index=-100)
        assert f.check() == 0
        err = abs(float(loss.item()) - want["loss"]) / abs(want["loss"])
        assert err <= LOSS_TOL, f"forward-only {reduction} loss rel err {err}"
        # the statistics pass is the same computation with or without gradients
        assert float(loss.item()) == float(loss_full.item())
        assert np.array_equal(to_f64(lse), to_f64(lse_full))
        assert np.max(np.abs(to_f64(lse) - want["lse"])) <= 1e-3


def test_forward_only_full_vocab():
    """Forward only at the Llama-3 vocabulary (no logits buffer), sum reduction, vs the oracle."""
    d = _inputs(512, 4096, 128256, "bf16", seed=71, ignore=-100, frac=0.25)
    f = _handle(d, 0)
    x, W, t = to_device(d)
    loss, lse = f.forward(x, W, t, chunk=256, with_lse=True, reduction="sum", ignore_index=-100)
    assert f.check() == 0
    want = _oracle(d, "sum", -100)
    err = abs(float(loss.item()) - want["loss"]) / abs(want["loss"])
    assert err <= LOSS_TOL, f"loss rel err {err}"
    assert np.max(np.abs(to_f64(lse) - want["lse"])) <= 1e-3


def test_option_validation():
    torch = require_gpu()
    import linear_cross_entropy_token_amd as flce
    d = _inputs(64, 64, 300, "bf16", seed=81)
    f = _handle(d, 0)
    x, W, t = to_device(d)
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    dx = torch.empty_like(x)
    dW = torch.empty_like(W)
    s = torch.cuda.current_stream().cuda_stream

    def call(opt, dxp=dx.data_ptr(), dWp=dW.data_ptr()):
        return flce.flce_forward_backward_opt(f.handle, x.data_ptr(), W.data_ptr(), t.data_ptr(), 64, 64, 300,
                                              0, opt, loss.data_ptr(), dxp, dWp, None, s)
    assert call(None) == 0
    assert call(flce.Options(2, 0, 0, 0, 0)) == 1                                    # unknown reduction
    assert call(flce.Options(0, 4, 0, 0, 0)) == 1                                    # unknown flag
    assert call(flce.Options(0, flce.FLCE_ACCUMULATE | flce.FLCE_FORWARD_ONLY, 0, 0, 0)) == 1
    assert call(flce.Options(0, 0, 2, 0, 0)) == 1                                    # ignore_on not 0/1
    assert call(flce.Options(0, 0, 0, 1, 0)) == 1                                    # reserved
    assert call(flce.Options(0, 0, 0, 0, 0), dxp=None) == 1                          # gradients need dx
    assert call(flce.Options(0, flce.FLCE_FORWARD_ONLY, 0, 0, 0), dxp=None, dWp=None) == 0
    torch.cuda.synchronize()
    # forward only needs neither the logits buffer nor gradient accumulators
    full = f.workspace_bytes(4096, 4096, 128256, 2048)
    fwd = f.workspace_bytes(4096, 4096, 128256, 2048, forward_only=True)
    assert 0 < fwd < full - 2048 * 128256 * 2 + 4096, (fwd, full)
