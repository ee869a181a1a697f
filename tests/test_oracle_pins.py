"""The CPU oracle against its pins (CPU only).

Also plants plausible mistakes in copies of the oracle and checks that at
least one pin catches each one, so the pins are known to be sensitive.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import flce_oracle as fo
import oracle_pins as pins
from flce_inputs import make_inputs, WORKLOADS


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle.flce)


# ---- planted mistakes ------------------------------------------------------

def _mutant(kind):
    def flce(x, W, t):
        x = np.asarray(x, dtype=np.float64)
        W = np.asarray(W, dtype=np.float64)
        t = np.asarray(t, dtype=np.int64)
        N, V = x.shape[0], W.shape[0]
        tt = (t + 1) % V if kind == "target_off_by_one" else t
        Z = x @ W.T
        if kind == "no_max_subtraction":
            lse = np.log(np.exp(Z).sum(axis=1))
        elif kind == "lse_missing_log":
            m = Z.max(axis=1)
            lse = m + np.exp(Z - m[:, None]).sum(axis=1)
        else:
            lse = fo.row_logsumexp(Z)
        losses = lse - Z[np.arange(N), tt]
        loss = losses.sum() if kind == "sum_not_mean" else losses.mean()
        G = np.exp(Z - lse[:, None])
        if kind == "no_onehot":
            pass
        elif kind == "onehot_wrong_sign":
            G[np.arange(N), tt] += 1.0
        else:
            G[np.arange(N), tt] -= 1.0
        if kind != "no_1_over_N":
            G /= N
        dx = G @ W
        if kind == "dx_uses_WT_rows_reversed":
            dx = G @ W[::-1]
        dW = G.T @ x
        if kind == "dW_tokens_reversed":
            dW = G.T @ x[::-1]
        return {"loss": float(loss), "dx": dx, "dW": dW, "lse": lse, "losses": losses}
    return flce


MUTANTS = ["target_off_by_one", "no_max_subtraction", "lse_missing_log", "sum_not_mean",
           "no_onehot", "onehot_wrong_sign", "no_1_over_N", "dx_uses_WT_rows_reversed",
           "dW_tokens_reversed"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistake(kind):
    bad = _mutant(kind)
    caught = []
    with np.errstate(all="ignore"):
        for check in pins.ALL_CHECKS:
            try:
                check(bad)
            except (AssertionError, FloatingPointError, ValueError, IndexError):
                caught.append(check.__name__)
    assert caught, f"no pin caught the planted mistake {kind!r}"


def test_unmutated_copy_passes_all_pins():
    good = _mutant("none")
    for check in pins.ALL_CHECKS:
        check(good)


# ---- loss options (flce_ext) -------------------------------------------------

def _ext(x, W, t, reduction, ignore_index):
    return oracle.flce_ext(x, W, t, reduction=reduction, ignore_index=ignore_index)


@pytest.mark.parametrize("check", pins.EXT_CHECKS, ids=lambda c: c.__name__)
def test_ext_pin(check):
    check(_ext)


def _ext_mutant(kind):
    def ext(x, W, t, reduction, ignore_index):
        x = np.asarray(x, dtype=np.float64)
        W = np.asarray(W, dtype=np.float64)
        t = np.asarray(t, dtype=np.int64)
        N = x.shape[0]
        counted = np.ones(N, bool) if ignore_index is None else t != ignore_index
        tt = np.where(counted, t, 0)
        Z = x @ W.T
        lse = fo.row_logsumexp(Z)
        losses = lse - Z[np.arange(N), tt]
        if kind != "ignored_rows_keep_loss":
            losses = np.where(counted, losses, 0.0)
        n = int(counted.sum())
        denom = float(N) if kind == "mean_over_all_tokens" else float(n)
        if reduction == "sum" and kind != "sum_divides":
            denom = 1.0
        if n == 0 and reduction == "mean":
            loss = 0.0 if kind == "all_ignored_zero_loss" else float("nan")
        else:
            loss = float(losses.sum() / denom)
        G = np.exp(Z - lse[:, None])
        G[np.arange(N), tt] -= 1.0
        if kind != "ignored_rows_keep_grad":
            G[~counted] = 0.0
        G /= max(denom, 1.0) if n == 0 else denom
        return {"loss": loss, "dx": G @ W, "dW": G.T @ x}
    return ext


EXT_MUTANTS = ["mean_over_all_tokens", "ignored_rows_keep_grad", "ignored_rows_keep_loss",
               "sum_divides", "all_ignored_zero_loss"]


@pytest.mark.parametrize("kind", EXT_MUTANTS)
def test_ext_pins_catch_planted_mistake(kind):
    bad = _ext_mutant(kind)
    caught = []
    with np.errstate(all="ignore"):
        for check in pins.EXT_CHECKS:
            try:
                check(bad)
            except (AssertionError, FloatingPointError, ValueError, IndexError):
                caught.append(check.__name__)
    assert caught, f"no pin caught the planted mistake {kind!r}"


def test_ext_unmutated_copy_passes():
    good = _ext_mutant("none")
    for check in pins.EXT_CHECKS:
        check(good)


# ---- RMSNorm in front of the head (rmsnorm_flce) ---------------------------

def _rf(h, g, eps, W, t, reduction, ignore_index):
    return oracle.rmsnorm_flce(h, g, eps, W, t, reduction=reduction, ignore_index=ignore_index)


@pytest.mark.parametrize("check", pins.RMS_CHECKS, ids=lambda c: c.__name__)
def test_rms_pin(check):
    check(_rf)


def _rms_mutant(kind):
    def rf(h, g, eps, W, t, reduction, ignore_index):
        h = np.asarray(h, dtype=np.float64)
        g = np.asarray(g, dtype=np.float64)
        d = h.shape[1]
        ms = (h * h).mean(axis=1) + (0.0 if kind == "no_eps" else eps)
        rstd = 1.0 / (ms if kind == "rms_no_sqrt" else np.sqrt(ms))
        x = h * rstd[:, None] * g[None, :]
        r = oracle.flce_ext(x, W, t, reduction=reduction, ignore_index=ignore_index)
        dx = r["dx"]
        s = (dx * g[None, :] * h).sum(axis=1)
        dd = 1.0 if kind == "dh_missing_1_over_d" else float(d)
        sign = 1.0 if kind == "dh_plus" else -1.0
        dh = rstd[:, None] * (dx * g[None, :] + sign * h * (rstd ** 2 * s / dd)[:, None])
        dgamma = (dx * h * (1.0 if kind == "dgamma_no_rstd" else rstd[:, None])).sum(axis=0)
        return {"loss": r["loss"], "dh": dh, "dgamma": dgamma, "dW": r["dW"]}
    return rf


RMS_MUTANTS = ["no_eps", "rms_no_sqrt", "dh_missing_1_over_d", "dh_plus", "dgamma_no_rstd"]


@pytest.mark.parametrize("kind", RMS_MUTANTS)
def test_rms_pins_catch_planted_mistake(kind):
    bad = _rms_mutant(kind)
    caught = []
    with np.errstate(all="ignore"):
        for check in pins.RMS_CHECKS:
            try:
                check(bad)
            except (AssertionError, FloatingPointError, ValueError, IndexError):
                caught.append(check.__name__)
    assert caught, f"no pin caught the planted mistake {kind!r}"


def test_rms_unmutated_copy_passes():
    good = _rms_mutant("none")
    for check in pins.RMS_CHECKS:
        check(good)


# ---- other properties of the oracle ---------------------------------------

def test_rows_match_full():
    d = make_inputs(64, 32, 300, "bf16", seed=11)
    x = oracle.widen(d["x"], "bf16")
    W = oracle.widen(d["W"], "bf16")
    r = oracle.flce(x, W, d["t"])
    rows = [0, 7, 63]
    rr = oracle.flce_rows(x, W, d["t"], rows, 64)
    np.testing.assert_allclose(rr["lse"], r["lse"][rows], rtol=1e-14)
    np.testing.assert_allclose(rr["loss"], r["losses"][rows], rtol=1e-13)
    np.testing.assert_allclose(rr["dx"], r["dx"][rows], rtol=1e-11, atol=1e-17)


@pytest.mark.parametrize("case", ["mixed", "targets_only_in_zero_rows", "targets_only_in_nonzero_rows",
                                  "no_zero_rows", "all_zero"])
def test_sparse_weight_matches_dense(case):
    """flce_sparse_weight against flce on the dense weight it stands for (zero outside nz)."""
    rng = np.random.default_rng(17)
    N, H, V = 48, 24, 300
    x = rng.standard_normal((N, H))
    if case == "no_zero_rows":
        nz = np.arange(V)
    elif case == "all_zero":
        nz = np.array([], dtype=np.int64)
    else:
        nz = np.unique(np.concatenate([rng.choice(V, 40, replace=False), [V - 1, V - 2]]))
    W_nz = rng.standard_normal((len(nz), H)) * 0.7      # large enough logits to matter
    zero = np.setdiff1d(np.arange(V), nz)
    if case == "targets_only_in_zero_rows":
        t = rng.choice(zero, N)
    elif case == "targets_only_in_nonzero_rows":
        t = rng.choice(nz, N)
    else:
        t = rng.integers(0, V, N)
    W = np.zeros((V, H))
    W[nz] = W_nz
    want = oracle.flce(x, W, t)
    rows = np.unique(np.concatenate([t[:5], zero[:3], nz[:3], [V - 1]]))
    got = oracle.flce_sparse_weight(x, W_nz, nz, V, t, rows)
    np.testing.assert_allclose(got["loss"], want["loss"], rtol=1e-13)
    np.testing.assert_allclose(got["lse"], want["lse"], rtol=1e-13)
    np.testing.assert_allclose(got["dx"], want["dx"], rtol=1e-10, atol=1e-15)
    np.testing.assert_allclose(got["dW_rows"], want["dW"][rows], rtol=1e-10, atol=1e-15)
    if case == "all_zero":                                 # the W = 0 closed form
        assert abs(got["loss"] - np.log(V)) <= 1e-14 * np.log(V)


def test_statistical_expectation_of_loss():
    """x ~ N(0,1), W ~ N(0,0.02^2): logits ~ N(0, 4e-4 |x|^2), so E[loss] ~ ln V + 2e-4 H."""
    w = WORKLOADS["tiny_fp32"]
    d = make_inputs(w.N, w.H, w.V, w.dtype, w.seed, w.targets)
    r = oracle.flce(oracle.widen(d["x"], "fp32"), oracle.widen(d["W"], "fp32"), d["t"])
    assert abs(r["loss"] - (math.log(w.V) + 2e-4 * w.H)) < 0.1


def test_widen_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0001, 0x7F7F, 0x4049], dtype=np.uint16)
    got = oracle.widen(bits, "bf16")
    assert got[0] == 1.0 and got[1] == -1.0
    assert got[2] == 2.0 ** -133      # smallest bf16 subnormal
    assert got[3] == (2 - 2 ** -7) * 2.0 ** 127
    assert got[4] == 3.140625


def test_rejects_empty_and_bad_targets():
    with pytest.raises(ValueError):
        oracle.flce(np.zeros((0, 3)), np.zeros((4, 3)), np.zeros(0, dtype=np.int64))
    with pytest.raises(ValueError):
        oracle.flce(np.zeros((2, 3)), np.zeros((4, 3)), np.array([0, 4]))


def test_page_logit_sizes():
    with open(os.path.join(pins.GOLDEN, "page_logit_sizes.json")) as f:
        figs = json.load(f)["figures"]
    for fgr in figs:
        b = oracle.logits_bytes(fgr["tokens"], fgr["vocab"], fgr["bytes_per_elem"])
        if "elements" in fgr:
            assert fgr["tokens"] * fgr["vocab"] == fgr["elements"], fgr["cite"]
        unit = 1e9 if fgr["unit"] == "GB" else 2.0 ** 30
        assert abs(b / unit - fgr["printed"]) <= fgr["rel_tol"] * fgr["printed"], fgr["cite"]


# ---- the row-blocked driver (flce_blocked) ---------------------------------
# The full-size GPU parity tests compare against flce_blocked, which runs the definition one
# block of token rows at a time.  It is pinned the way flce is (every check of the pin suite,
# with blocks that split every pin's tokens, ragged last block included), against flce itself,
# and by planted mistakes of the kind a blocked loop invites.

def _blocked(block):
    def f(x, W, t):
        return oracle.flce_blocked(x, W, t, block=block)
    return f


@pytest.mark.parametrize("block", [1, 2, 3])
@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_blocked_pin(check, block):
    check(_blocked(block))


@pytest.mark.parametrize("N,block", [(1, 1), (7, 3), (64, 64), (64, 100), (65, 16), (200, 7)])
def test_blocked_matches_flce(N, block):
    rng = np.random.default_rng(N * 1000 + block)
    H, V = 24, 301
    x = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H)) * 0.6
    t = rng.integers(0, V, N)
    want = oracle.flce(x, W, t)
    got = oracle.flce_blocked(x, W, t, block=block)
    np.testing.assert_allclose(got["loss"], want["loss"], rtol=1e-14)
    np.testing.assert_allclose(got["lse"], want["lse"], rtol=1e-14)
    np.testing.assert_allclose(got["losses"], want["losses"], rtol=1e-13)
    np.testing.assert_array_equal(got["dx_rows"], np.arange(N))
    np.testing.assert_allclose(got["dx"], want["dx"], rtol=1e-11, atol=1e-17)
    np.testing.assert_allclose(got["dW"], want["dW"], rtol=1e-11, atol=1e-17)


def test_blocked_storage_forms_and_selected_blocks():
    """bf16 / fp32 storage widened block by block equals the widened whole; dx of selected blocks."""
    for dt in ("bf16", "fp32"):
        d = make_inputs(150, 40, 500, dt, seed=41)
        want = oracle.flce(oracle.widen(d["x"], dt), oracle.widen(d["W"], dt), d["t"])
        got = oracle.flce_blocked(d["x"], d["W"], d["t"], block=64, dtype=dt, dx_blocks=[2, 0])
        assert got["loss"] == pytest.approx(want["loss"], rel=1e-14)
        rows = np.concatenate([np.arange(0, 64), np.arange(128, 150)])
        np.testing.assert_array_equal(got["dx_rows"], rows)
        np.testing.assert_allclose(got["dx"], want["dx"][rows], rtol=1e-11, atol=1e-17)
        np.testing.assert_allclose(got["dW"], want["dW"], rtol=1e-11, atol=1e-17)
    seen = []
    oracle.flce_blocked(d["x"], d["W"], d["t"], block=64, dtype="fp32", dx_blocks=[],
                        progress=lambda b, n: seen.append((b, n)))
    assert seen == [(0, 3), (1, 3), (2, 3)]


def _blocked_mutant(kind, block=2):
    """Copies of the blocked loop with one plausible mistake each."""
    def f(x, W, t):
        x = np.asarray(x, dtype=np.float64)
        W = np.asarray(W, dtype=np.float64)
        t = np.asarray(t, dtype=np.int64)
        N = x.shape[0]
        lse, losses = np.empty(N), np.empty(N)
        dW = np.zeros_like(W)
        dx = np.zeros_like(x)
        means = []
        for s in range(0, N, block):
            e = min(N, s + block)
            xb = x[s:e]
            Z = fo.logits(xb, W)
            lse[s:e] = fo.row_logsumexp(Z)
            losses[s:e] = fo.row_losses(Z, t[s:e], lse[s:e])
            means.append(losses[s:e].mean())
            G = fo.dlogits(Z, t[s:e], lse[s:e], e - s if kind == "block_local_N" else N)
            dx[s:e] = G @ W
            if kind == "dx_rows_shifted" and s > 0:
                dx[s - 1:e - 1] = G @ W
            if kind == "dW_overwritten":
                dW = G.T @ xb
            else:
                dW += G.T @ xb
        loss = float(np.mean(means)) if kind == "mean_of_block_means" else float(losses.mean())
        return {"loss": loss, "lse": lse, "losses": losses, "dx": dx, "dW": dW}
    return f


BLOCKED_MUTANTS = ["block_local_N", "dx_rows_shifted", "dW_overwritten", "mean_of_block_means"]


@pytest.mark.parametrize("kind", BLOCKED_MUTANTS)
def test_blocked_pins_catch_planted_mistake(kind):
    bad = _blocked_mutant(kind)
    caught = []
    with np.errstate(all="ignore"):
        for check in pins.ALL_CHECKS:
            try:
                check(bad)
            except (AssertionError, FloatingPointError, ValueError, IndexError):
                caught.append(check.__name__)
    assert caught, f"no pin caught the planted mistake {kind!r}"


def test_blocked_unmutated_copy_passes():
    good = _blocked_mutant("none")
    for check in pins.ALL_CHECKS:
        check(good)
