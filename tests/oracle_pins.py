"""Pins for the FLCE oracle: checks that tie it to facts other than itself.

Each ``check_*`` takes an ``flce(x, W, t) -> dict`` implementation (the
oracle, or a copy of it with a planted mistake) and raises AssertionError
when the implementation disagrees with

  * hand-derived worked examples (tests/golden/worked_examples.json),
  * closed forms (W = 0; two classes reduce to softplus),
  * central finite differences of the loss in fp64,
  * invariants of the definition (dlogits rows sum to zero, dW column sums
    vanish, <x,dx> = <W,dW>, per-row logit shift, permutations),
  * an independent library routine (torch.nn.functional.cross_entropy with
    autograd, fp64, CPU).

The definition being pinned: loss = mean_n(lse_n - z[n,t_n]),
G = (softmax(z) - onehot(t))/N, dx = G W, dW = G^T x with z = x W^T
(cross-entropy and gradient equations of the "Unsloth deep architecture"
page, streaming Fast CrossEntropy section; mean reduction with 1/N on the
gradients from the code sample of the "core idea" section of the "Fused
Linear Cross-Entropy" page).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _eval(expr: str) -> float:
    return float(eval(expr, {"__builtins__": {}}, {"log": math.log, "exp": math.exp}))


def _mat(rows):
    return np.array([[_eval(e) for e in r] for r in rows], dtype=np.float64)


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    assert np.allclose(a, b, rtol=rtol, atol=atol), \
        f"{what}: max abs diff {np.max(np.abs(a - b))}"


def check_worked_examples(flce):
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        ex = json.load(f)["examples"]
    for e in ex:
        x, W = _mat(e["x"]), _mat(e["W"])
        t = np.array(e["t"], dtype=np.int64)
        r = flce(x, W, t)
        _close(r["loss"], _eval(e["loss"]), 1e-12, 1e-12, e["name"] + " loss")
        _close(r["dx"], _mat(e["dx"]), 1e-12, 1e-12, e["name"] + " dx")
        _close(r["dW"], _mat(e["dW"]), 1e-12, 1e-12, e["name"] + " dW")


def check_zero_weight(flce, N=37, H=11, V=29, seed=0):
    """W = 0: every logit is 0, softmax is uniform 1/V.

    loss = ln V exactly; dx = G W = 0; dW[v] = (1/V) mean_n x_n - (1/N) sum_{n: t_n = v} x_n.
    """
    rng = _rng(seed)
    x = rng.standard_normal((N, H))
    t = rng.integers(0, V, N)
    t[:3] = [0, V - 1, 5]
    r = flce(x, np.zeros((V, H)), t)
    _close(r["loss"], math.log(V), 1e-15, 0, "W=0 loss")
    assert np.all(r["dx"] == 0.0), "W=0 dx must be exactly 0"
    expect = np.tile(x.mean(axis=0) / V, (V, 1))
    for n in range(N):
        expect[t[n]] -= x[n] / N
    _close(r["dW"], expect, 1e-12, 1e-14, "W=0 dW")


def check_two_classes(flce, N=50, H=7, seed=1):
    """V = 2: the per-row loss is softplus(z_other - z_target) = log(1 + e^d)."""
    rng = _rng(seed)
    x = rng.standard_normal((N, H))
    W = rng.standard_normal((2, H))
    t = rng.integers(0, 2, N)
    z = np.einsum("nh,vh->nv", x, W)
    d = z[np.arange(N), 1 - t] - z[np.arange(N), t]
    want = np.logaddexp(0.0, d).mean()
    r = flce(x, W, t)
    _close(r["loss"], want, 1e-13, 0, "V=2 softplus")


def _loss_only(flce, x, W, t):
    return flce(x, W, t)["loss"]


def check_finite_differences(flce, N=3, H=5, V=7, seed=2, eps=1e-6):
    """dx and dW against central differences of the loss (fp64, O(eps^2) error)."""
    rng = _rng(seed)
    x = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H)) * 0.5
    t = rng.integers(0, V, N)
    r = flce(x, W, t)
    fdx = np.zeros_like(x)
    for i in range(N):
        for j in range(H):
            xp, xm = x.copy(), x.copy()
            xp[i, j] += eps
            xm[i, j] -= eps
            fdx[i, j] = (_loss_only(flce, xp, W, t) - _loss_only(flce, xm, W, t)) / (2 * eps)
    fdW = np.zeros_like(W)
    for i in range(V):
        for j in range(H):
            Wp, Wm = W.copy(), W.copy()
            Wp[i, j] += eps
            Wm[i, j] -= eps
            fdW[i, j] = (_loss_only(flce, x, Wp, t) - _loss_only(flce, x, Wm, t)) / (2 * eps)
    _close(r["dx"], fdx, 1e-6, 1e-9, "dx vs finite differences")
    _close(r["dW"], fdW, 1e-6, 1e-9, "dW vs finite differences")


def check_invariants(flce, N=40, H=16, V=33, seed=3):
    """Row sums of G vanish, so dW's column sums vanish and <x,dx> = <W,dW>."""
    rng = _rng(seed)
    x = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H)) * 0.3
    t = rng.integers(0, V, N)
    r = flce(x, W, t)
    scale = np.abs(r["dW"]).max()
    assert np.abs(r["dW"].sum(axis=0)).max() <= 1e-13 * max(scale, 1.0) * V, "dW column sums"
    a = float(np.sum(x * r["dx"]))
    b = float(np.sum(W * r["dW"]))
    _close(a, b, 1e-12, 1e-15, "<x,dx> vs <W,dW>")
    # lse is at least the row max and at most max + ln V
    z = x @ W.T
    assert np.all(r["lse"] >= z.max(axis=1) - 1e-12)
    assert np.all(r["lse"] <= z.max(axis=1) + math.log(V) + 1e-12)


def check_shift_invariance(flce, N=20, H=9, V=17, seed=4, shift=300.0):
    """W -> W + 1 u^T adds <x_n, u> to every logit of row n: nothing changes."""
    rng = _rng(seed)
    x = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H)) * 0.2
    t = rng.integers(0, V, N)
    u = rng.standard_normal(H) * shift
    r0 = flce(x, W, t)
    r1 = flce(x, W + u[None, :], t)
    _close(r1["loss"], r0["loss"], 1e-9, 0, "shifted loss")
    _close(r1["dW"], r0["dW"], 1e-9, 1e-12, "shifted dW")
    _close(r1["dx"], r0["dx"], 1e-7, 1e-9, "shifted dx")


def check_permutations(flce, N=25, H=6, V=19, seed=5):
    """Permuting tokens permutes dx; permuting vocabulary rows (and relabelling targets) permutes dW."""
    rng = _rng(seed)
    x = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H)) * 0.4
    t = rng.integers(0, V, N)
    r = flce(x, W, t)
    pn = rng.permutation(N)
    rn = flce(x[pn], W, t[pn])
    _close(rn["dx"], r["dx"][pn], 1e-12, 1e-15, "token permutation dx")
    _close(rn["loss"], r["loss"], 1e-13, 0, "token permutation loss")
    pv = rng.permutation(V)
    inv = np.argsort(pv)
    rv = flce(x, W[pv], inv[t])
    _close(rv["dW"], r["dW"][pv], 1e-12, 1e-15, "vocab permutation dW")
    _close(rv["dx"], r["dx"], 1e-12, 1e-15, "vocab permutation dx")


def check_torch_autograd(flce, N=31, H=12, V=45, seed=6):
    """Independent library routine: torch cross_entropy + autograd in fp64 on the CPU."""
    import torch
    import torch.nn.functional as F
    rng = _rng(seed)
    x = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H)) * 0.5
    t = rng.integers(0, V, N)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    loss = F.cross_entropy(xt @ Wt.T, torch.tensor(t), reduction="mean")
    loss.backward()
    r = flce(x, W, t)
    _close(r["loss"], loss.item(), 1e-13, 0, "torch loss")
    _close(r["dx"], xt.grad.numpy(), 1e-11, 1e-15, "torch dx")
    _close(r["dW"], Wt.grad.numpy(), 1e-11, 1e-15, "torch dW")


ALL_CHECKS = [check_worked_examples, check_zero_weight, check_two_classes,
              check_finite_differences, check_invariants, check_shift_invariance,
              check_permutations, check_torch_autograd]


# ---- pins of the loss options (flce_ext) -------------------------------------
# Each check_ext_* takes an ``ext(x, W, t, reduction, ignore_index) -> dict``.

def _ext_inputs(seed, N, H, V, ignore, frac=0.3):
    rng = _rng(seed)
    x = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H)) * 0.5
    t = rng.integers(0, V, N)
    if ignore is not None:
        t[rng.random(N) < frac] = ignore
    return x, W, t


def check_ext_torch(ext, N=29, H=10, V=37, seed=7):
    """Library routine: torch cross_entropy(reduction=..., ignore_index=...) with autograd,
    fp64 on the CPU, including an in-range ignore_index and an all-ignored batch."""
    import torch
    import torch.nn.functional as F
    cases = [(r, ign, 0.3) for r in ("mean", "sum") for ign in (None, -100, 5)]
    cases += [("mean", -1, 1.0), ("sum", -1, 1.0)]
    for k, (reduction, ign, frac) in enumerate(cases):
        x, W, t = _ext_inputs(seed + k, N, H, V, ign, frac)
        xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
        Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
        loss = F.cross_entropy(xt @ Wt.T, torch.tensor(t), reduction=reduction,
                               ignore_index=-100 if ign is None else ign)
        loss.backward()
        r = ext(x, W, t, reduction, ign)
        what = f"torch {reduction} ignore={ign} frac={frac}"
        if math.isnan(loss.item()):
            assert math.isnan(r["loss"]), f"{what}: loss {r['loss']} (expected NaN)"
        else:
            _close(r["loss"], loss.item(), 1e-13, 1e-15, what + " loss")
        _close(r["dx"], xt.grad.numpy(), 1e-11, 1e-15, what + " dx")
        _close(r["dW"], Wt.grad.numpy(), 1e-11, 1e-15, what + " dW")


def check_ext_drop_rows(ext, N=40, H=8, V=23, seed=8):
    """Ignoring tokens is dropping them: against the plain definition (the pinned ``flce``)
    on the kept rows, with zero gradient rows for the ignored ones; a sum is the mean times
    the count."""
    import oracle
    x, W, t = _ext_inputs(seed, N, H, V, -7, 0.4)
    kept = t != -7
    ref = oracle.flce(x[kept], W, t[kept])
    n = int(kept.sum())
    for reduction, f in (("mean", 1.0), ("sum", float(n))):
        r = ext(x, W, t, reduction, -7)
        _close(r["loss"], ref["loss"] * f, 1e-12, 0, f"drop rows {reduction} loss")
        _close(r["dx"][kept], ref["dx"] * f, 1e-11, 1e-15, f"drop rows {reduction} dx")
        _close(r["dx"][~kept], np.zeros((N - n, H)), 0, 0, f"drop rows {reduction} ignored dx")
        _close(r["dW"], ref["dW"] * f, 1e-11, 1e-15, f"drop rows {reduction} dW")


def check_ext_defaults(ext, N=18, H=7, V=13, seed=9):
    """No ignored token and the mean: the plain definition."""
    import oracle
    x, W, t = _ext_inputs(seed, N, H, V, None)
    r, ref = ext(x, W, t, "mean", None), oracle.flce(x, W, t)
    _close(r["loss"], ref["loss"], 1e-14, 0, "defaults loss")
    _close(r["dx"], ref["dx"], 1e-13, 1e-16, "defaults dx")
    _close(r["dW"], ref["dW"], 1e-13, 1e-16, "defaults dW")


EXT_CHECKS = [check_ext_torch, check_ext_drop_rows, check_ext_defaults]


# ---- pins of the RMSNorm in front of the head (rmsnorm_flce) ---------------
# Each check_rms_* takes ``rf(h, gamma, eps, W, t, reduction, ignore_index) -> dict`` with
# loss, dh, dgamma, dW.

def _rms_inputs(seed, N, H, V):
    rng = _rng(seed)
    h = rng.standard_normal((N, H)) * 1.7
    g = 1.0 + 0.3 * rng.standard_normal(H)
    W = rng.standard_normal((V, H)) * 0.4
    t = rng.integers(0, V, N)
    return h, g, W, t


def check_rms_torch(rf, N=23, H=12, V=19, seed=21):
    """Library routines: torch rms_norm, then cross_entropy, with autograd, fp64 on the CPU
    (a large eps so that a dropped eps shows)."""
    import torch
    import torch.nn.functional as F
    for k, (reduction, ign, eps) in enumerate([("mean", None, 1e-2), ("sum", -100, 1e-6), ("mean", 3, 0.5)]):
        h, g, W, t = _rms_inputs(seed + k, N, H, V)
        if ign is not None:
            t[_rng(seed + 50 + k).random(N) < 0.3] = ign
        ht = torch.tensor(h, requires_grad=True)
        gt = torch.tensor(g, requires_grad=True)
        Wt = torch.tensor(W, requires_grad=True)
        x = F.rms_norm(ht, (H,), gt, eps)
        loss = F.cross_entropy(x @ Wt.T, torch.tensor(t), reduction=reduction,
                               ignore_index=-100 if ign is None else ign)
        loss.backward()
        r = rf(h, g, eps, W, t, reduction, ign)
        what = f"rms torch {reduction} ignore={ign} eps={eps}"
        _close(r["loss"], loss.item(), 1e-12, 1e-15, what + " loss")
        _close(r["dh"], ht.grad.numpy(), 1e-10, 1e-14, what + " dh")
        _close(r["dgamma"], gt.grad.numpy(), 1e-10, 1e-14, what + " dgamma")
        _close(r["dW"], Wt.grad.numpy(), 1e-10, 1e-14, what + " dW")


def check_rms_finite_differences(rf, N=3, H=5, V=4, seed=22, eps=1e-6):
    """Central differences of the loss in h and gamma (fp64)."""
    h, g, W, t = _rms_inputs(seed, N, H, V)
    r = rf(h, g, 1e-3, W, t, "mean", None)
    num_h = np.zeros_like(h)
    for i in range(N):
        for j in range(H):
            hp, hm = h.copy(), h.copy()
            hp[i, j] += eps
            hm[i, j] -= eps
            num_h[i, j] = (rf(hp, g, 1e-3, W, t, "mean", None)["loss"]
                           - rf(hm, g, 1e-3, W, t, "mean", None)["loss"]) / (2 * eps)
    num_g = np.zeros_like(g)
    for j in range(H):
        gp, gm = g.copy(), g.copy()
        gp[j] += eps
        gm[j] -= eps
        num_g[j] = (rf(h, gp, 1e-3, W, t, "mean", None)["loss"] - rf(h, gm, 1e-3, W, t, "mean", None)["loss"]) / (2 * eps)
    _close(r["dh"], num_h, 1e-6, 1e-9, "rms finite differences dh")
    _close(r["dgamma"], num_g, 1e-6, 1e-9, "rms finite differences dgamma")


def check_rms_scale_invariance(rf, N=17, H=9, V=11, seed=23, c=7.5):
    """With eps = 0, scaling h by c > 0 leaves x, the loss, dW and dgamma unchanged and divides dh by c."""
    h, g, W, t = _rms_inputs(seed, N, H, V)
    a = rf(h, g, 0.0, W, t, "mean", None)
    b = rf(c * h, g, 0.0, W, t, "mean", None)
    _close(b["loss"], a["loss"], 1e-13, 0, "rms scale loss")
    _close(b["dW"], a["dW"], 1e-11, 1e-15, "rms scale dW")
    _close(b["dgamma"], a["dgamma"], 1e-11, 1e-15, "rms scale dgamma")
    _close(b["dh"] * c, a["dh"], 1e-11, 1e-15, "rms scale dh")


def check_rms_zero_gamma(rf, N=13, H=6, V=10, seed=24):
    """gamma = 0: x = 0, so the loss is ln V exactly, dW = 0 and dh = 0."""
    h, g, W, t = _rms_inputs(seed, N, H, V)
    r = rf(h, np.zeros_like(g), 1e-5, W, t, "mean", None)
    _close(r["loss"], math.log(V), 1e-14, 0, "rms zero gamma loss")
    _close(r["dW"], np.zeros_like(W), 0, 1e-17, "rms zero gamma dW")
    _close(r["dh"], np.zeros_like(h), 0, 1e-17, "rms zero gamma dh")


RMS_CHECKS = [check_rms_torch, check_rms_finite_differences, check_rms_scale_invariance, check_rms_zero_gamma]
