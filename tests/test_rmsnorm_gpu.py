"""GPU parity of the RMSNorm-in-front-of-the-head entry point (flce_rmsnorm_forward_backward)
against the oracle's rmsnorm_flce (fp64, pinned to torch rms_norm + cross_entropy)."""
import numpy as np
import pytest

import oracle
from flce_inputs import make_inputs
from flce_testlib import rel_fro, require_gpu, to_f64

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
FP32_TOL = 1e-5
LOSS_TOL = 1e-4


def _inputs(N, H, V, dtype, seed, ignore=None, frac=0.25):
    """hidden ~ N(0, 1.5^2), gamma ~ 1 + 0.2 N(0, 1), W and targets from the seeded generator."""
    d = make_inputs(N, H, V, dtype, seed)
    rng = np.random.default_rng(seed + 500)
    hidden = (rng.standard_normal((N, H), dtype=np.float32) * np.float32(1.5))
    gamma = (1.0 + 0.2 * rng.standard_normal(H)).astype(np.float32)
    t = d["t"].copy()
    if ignore is not None:
        t[rng.random(N) < frac] = ignore
    if dtype == "bf16":
        from flce_inputs import bf16_bits_from_f32
        hidden, gamma = bf16_bits_from_f32(hidden), bf16_bits_from_f32(gamma)
    return {"h": hidden, "g": gamma, "W": d["W"], "t": t, "dtype": dtype}


def _dev(d):
    torch = require_gpu()
    conv = (lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)) if d["dtype"] == "bf16" \
        else (lambda a: torch.from_numpy(a))
    return (conv(d["h"]).cuda(), conv(d["g"]).cuda(), conv(d["W"]).cuda(), torch.from_numpy(d["t"]).cuda())


def _oracle(d, eps, reduction="mean", ignore=None):
    w = (lambda a: oracle.widen(a, d["dtype"]))
    return oracle.rmsnorm_flce(w(d["h"]), w(d["g"]), eps, w(d["W"]), d["t"], reduction=reduction,
                               ignore_index=ignore)


def _handle(dtype, grad=None, variant=0):
    torch = require_gpu()
    from linear_cross_entropy_token_amd import FusedLinearCrossEntropy
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = grad or tdt
    return FusedLinearCrossEntropy(in_dtype=tdt, dx_dtype=g, dw_dtype=g, variant=variant)


CASES = [
    # name, N, H, V, dtype, chunk, grads, reduction, ignore, eps
    ("bf16_ragged", 700, 256, 3000, "bf16", 256, None, "mean", None, 1e-6),
    ("bf16_fp32_grads", 700, 256, 3000, "bf16", 256, "fp32", "mean", None, 1e-6),
    ("bf16_H264", 520, 264, 1300, "bf16", 200, None, "mean", None, 1e-5),
    ("bf16_sum_ign", 600, 512, 2100, "bf16", 300, None, "sum", -100, 1e-6),
    ("fp32_tiny", 256, 256, 4096, "fp32", 64, None, "mean", None, 1e-6),
    ("fp32_H264_eps", 200, 264, 900, "fp32", 64, None, "mean", -1, 0.5),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_rmsnorm_vs_oracle(case):
    name, N, H, V, dtype, chunk, gdt, reduction, ign, eps = case
    print(f"[rmsnorm] {name}", flush=True)
    torch = require_gpu()
    d = _inputs(N, H, V, dtype, seed=91 + CASES.index(case), ignore=ign)
    want = _oracle(d, eps, reduction, ign)
    f = _handle(dtype, torch.float32 if gdt == "fp32" else None)
    h, g, W, t = _dev(d)
    loss, dh, dg, dW, lse = f.rmsnorm_forward_backward(h, g, W, t, eps=eps, chunk=chunk, with_lse=True,
                                                       reduction=reduction, ignore_index=ign)
    assert f.check() == 0
    tol = FP32_TOL if dtype == "fp32" else BF16_TOL
    err = abs(float(loss.item()) - want["loss"]) / abs(want["loss"])
    assert err <= LOSS_TOL, f"{name}: loss rel err {err}"
    e = {"dh": rel_fro(to_f64(dh), want["dh"]), "dgamma": rel_fro(to_f64(dg), want["dgamma"]),
         "dW": rel_fro(to_f64(dW), want["dW"])}
    assert all(v <= tol for v in e.values()), f"{name}: {e}"
    assert np.max(np.abs(to_f64(lse) - want["lse"])) <= (1e-4 if dtype == "fp32" else 2e-2)
    if ign is not None:
        assert np.all(to_f64(dh)[d["t"] == ign] == 0), f"{name}: nonzero dhidden row of an ignored token"


def test_rmsnorm_full_vocab():
    """Llama-3 vocabulary and hidden size at 256 tokens, two chunks."""
    d = _inputs(256, 4096, 128256, "bf16", seed=97)
    want = _oracle(d, 1e-6)
    f = _handle("bf16")
    h, g, W, t = _dev(d)
    loss, dh, dg, dW = f.rmsnorm_forward_backward(h, g, W, t, eps=1e-6, chunk=128)
    assert f.check() == 0
    assert abs(float(loss.item()) - want["loss"]) / abs(want["loss"]) <= LOSS_TOL
    e = {"dh": rel_fro(to_f64(dh), want["dh"]), "dgamma": rel_fro(to_f64(dg), want["dgamma"]),
         "dW": rel_fro(to_f64(dW), want["dW"])}
    assert all(v <= BF16_TOL for v in e.values()), e


@pytest.mark.parametrize("dtype,gdt", [("bf16", None), ("bf16", "fp32"), ("fp32", None)])
def test_rmsnorm_accumulate(dtype, gdt):
    torch = require_gpu()
    d = _inputs(600, 256, 2100, dtype, seed=101)
    want = _oracle(d, 1e-6)
    f = _handle(dtype, torch.float32 if gdt == "fp32" else None)
    h, g, W, t = _dev(d)
    gen = torch.Generator(device="cuda").manual_seed(9)

    def start(shape, ref, dt):
        return (torch.randn(shape, device="cuda", generator=gen) * float(np.sqrt(np.mean(ref ** 2)))).to(dt)
    dh0, dg0, dW0 = start(h.shape, want["dh"], f.dx_dtype), start(g.shape, want["dgamma"], f.dw_dtype), \
        start(W.shape, want["dW"], f.dw_dtype)
    dh, dg, dW = dh0.clone(), dg0.clone(), dW0.clone()
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    f.rmsnorm_forward_backward(h, g, W, t, eps=1e-6, chunk=256, out=(loss, dh, dg, dW, None), accumulate=True)
    assert f.check() == 0
    tol = FP32_TOL if dtype == "fp32" else BF16_TOL
    e = {"dh": rel_fro(to_f64(dh) - to_f64(dh0), want["dh"]),
         "dgamma": rel_fro(to_f64(dg) - to_f64(dg0), want["dgamma"]),
         "dW": rel_fro(to_f64(dW) - to_f64(dW0), want["dW"])}
    assert all(v <= tol for v in e.values()), e


def test_rmsnorm_forward_only_matches_full_call():
    d = _inputs(700, 256, 3000, "bf16", seed=103, ignore=-100, frac=0.2)
    f = _handle("bf16")
    h, g, W, t = _dev(d)
    loss, lse = f.rmsnorm_forward(h, g, W, t, eps=1e-6, chunk=256, with_lse=True, ignore_index=-100)
    loss2, _, _, _, lse2 = f.rmsnorm_forward_backward(h, g, W, t, eps=1e-6, chunk=256, with_lse=True,
                                                      ignore_index=-100)
    assert f.check() == 0
    assert float(loss.item()) == float(loss2.item())
    assert np.array_equal(to_f64(lse), to_f64(lse2))
    want = _oracle(d, 1e-6, ignore=-100)
    assert abs(float(loss.item()) - want["loss"]) / abs(want["loss"]) <= LOSS_TOL


def test_rmsnorm_validation():
    torch = require_gpu()
    import linear_cross_entropy_token_amd as flce
    d = _inputs(64, 64, 300, "bf16", seed=107)
    h, g, W, t = _dev(d)
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    dh, dg, dW = torch.empty_like(h), torch.empty_like(g), torch.empty_like(W)
    s = torch.cuda.current_stream().cuda_stream

    def call(f, eps=1e-6, H=64, dgp=dg.data_ptr(), hp=h.data_ptr()):
        return flce.flce_rmsnorm_forward_backward(f.handle, hp, g.data_ptr(), eps, W.data_ptr(), t.data_ptr(),
                                                  64, H, 300, 0, None, loss.data_ptr(), dh.data_ptr(), dgp,
                                                  dW.data_ptr(), None, s)
    f = _handle("bf16")
    assert call(f) == 0
    assert call(f, eps=-1.0) == 1                      # negative eps
    assert call(f, eps=float("nan")) == 1              # NaN eps
    assert call(f, dgp=None) == 1                      # gradients need dgamma
    assert call(f, H=32776) == 2                       # beyond the backward's LDS row (checked before any launch)
    assert call(_handle("bf16", variant=1)) == 2       # chunked variant only
    assert f.workspace_bytes(64, 64, 300) > 0
    assert flce.flce_rmsnorm_workspace_bytes(f.handle, 4096, 4096, 128256, 2048, None) > \
        flce.flce_workspace_bytes(f.handle, 4096, 4096, 128256, 2048)
    torch.cuda.synchronize()
