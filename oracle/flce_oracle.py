"""CPU oracle for fused linear cross-entropy (FLCE).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or
runs this module; only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may.  It shares no code with the HIP
library: the only common dependency is the seeded input generator
(``flce_inputs``), which holds none of the method's arithmetic.

What it computes is the plain, materialised definition that FLCE reaches
exactly (up to rounding order): the pages present FLCE as a memory
optimisation that yields the same loss and gradients as projecting every
token through the LM head and applying softmax cross-entropy
("Fused Linear Cross-Entropy", 42jerrykim.github.io, introduction and the
section on the core idea; the "Unsloth deep architecture" page,
techknowgenie.com, describes its streaming CE kernel as exact, not an
approximation).  So the oracle materialises the full [N,V] logits in fp64.

Notation: hidden states x[N,H], LM-head weight W[V,H] (row-major, one row per
vocabulary id, as in the code sample of the "core idea" section), targets
t[N] (int64 ids in [0,V)).

Readings taken where the pages are silent or disagree:
  * reduction is the mean over all N tokens, and dx, dW carry the same 1/N:
    the code sample of the "core idea" section sums per chunk and divides
    loss, dx and dw by the global token count at the end;
  * no bias and no label smoothing (neither is mentioned; the projection in
    the code sample has no bias); masked tokens (ignore_index) and the sum
    reduction exist only in ``flce_ext``, which states its own readings;
  * W is [V,H] (the 128K-context guide at sigco.tistory.com prints an [H,V]
    weight in its chunked-CE snippet; the [V,H] layout of the FLCE page is
    taken).
Every function below is pinned by tests against closed forms, invariants,
finite differences and a hand-derived worked example (tests/golden).
"""
from __future__ import annotations

from typing import Callable, Dict, Iterable, Optional

import numpy as np

__all__ = ["widen", "logits", "row_logsumexp", "row_losses", "dlogits", "flce", "flce_blocked",
           "flce_rows", "flce_sparse_weight", "flce_ext", "rmsnorm", "rmsnorm_backward", "rmsnorm_flce",
           "logits_bytes"]


def widen(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Storage form -> fp64, exactly (bf16 bit patterns or fp32 values)."""
    if dtype == "bf16":
        bits = np.ascontiguousarray(arr, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "fp32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "fp64":
        return np.asarray(arr, dtype=np.float64)
    raise ValueError(dtype)


def logits(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Z = x W^T, [N,V]: the LM-head projection (FLCE page, core idea, step 1)."""
    return x @ W.T


def row_logsumexp(Z: np.ndarray) -> np.ndarray:
    """lse_n = m_n + ln sum_v exp(Z[n,v] - m_n), m_n = max_v Z[n,v].

    The log-sum-exp term of the cross-entropy equation on the Unsloth page
    ("streaming chunked Fast CrossEntropy loss kernel"); the max is
    subtracted first, as that page's online-softmax description keeps a
    running maximum for numerical stability.
    """
    m = Z.max(axis=1)
    return m + np.log(np.exp(Z - m[:, None]).sum(axis=1))


def row_losses(Z: np.ndarray, t: np.ndarray, lse: np.ndarray) -> np.ndarray:
    """L_n = -Z[n, t_n] + lse_n (Unsloth page, cross-entropy loss equation)."""
    return lse - Z[np.arange(Z.shape[0]), t]


def dlogits(Z: np.ndarray, t: np.ndarray, lse: np.ndarray, n_total: int) -> np.ndarray:
    """G = (softmax(Z) - onehot(t)) / N.

    dL/dz_i = softmax(z)_i - [i = y] (Unsloth page, gradient equation; the
    FLCE page's step 2 overwrites the logits with softmax - one_hot), scaled
    by 1/N for the mean reduction (FLCE page, code sample, final division by
    the token count).
    """
    G = np.exp(Z - lse[:, None])
    G[np.arange(Z.shape[0]), t] -= 1.0
    G /= float(n_total)
    return G


def flce(x: np.ndarray, W: np.ndarray, t: np.ndarray) -> Dict[str, np.ndarray]:
    """The whole materialised computation in fp64.

    Returns loss (mean over N), dx = G W [N,H], dW = G^T x [V,H], and the
    per-row lse [N] and losses [N].  Steps 3 and 4 of the FLCE page's core
    idea (dx = dlogits x weight; dw = dlogits^T x hidden), here over all N at
    once instead of per chunk.
    """
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    t = np.asarray(t, dtype=np.int64)
    N = x.shape[0]
    if N == 0:
        raise ValueError("N must be positive (the mean over zero tokens is undefined)")
    if t.min() < 0 or t.max() >= W.shape[0]:
        raise ValueError("targets out of range")
    Z = logits(x, W)
    lse = row_logsumexp(Z)
    losses = row_losses(Z, t, lse)
    G = dlogits(Z, t, lse, N)
    del Z
    dx = G @ W
    dW = G.T @ x
    return {"loss": float(losses.mean()), "dx": dx, "dW": dW, "lse": lse, "losses": losses}


def flce_blocked(x: np.ndarray, W: np.ndarray, t: np.ndarray, block: int, dtype: str = "fp64",
                 dx_blocks: Optional[Iterable[int]] = None,
                 progress: Optional[Callable[[int, int], None]] = None) -> Dict[str, np.ndarray]:
    """``flce`` computed one block of ``block`` token rows at a time.

    This is the token-chunk loop of the FLCE page's core idea, in fp64 and
    with the plain functions above: for the rows [s, e) of a block, the
    logits Z_b = x_b W^T, their log-sum-exp and losses, the block's rows of
    G (scaled by 1/N for the GLOBAL token count N, as the page divides by
    the whole batch's token count), the block's rows of dx = G_b W, and the
    block's term G_b^T x_b of dW, which is summed over the blocks.  Every
    quantity is the same as ``flce``'s up to the order of the dW sum; only
    one block's logits exist at a time, so problems whose [N,V] logits do
    not fit in host memory can be checked whole.

    ``x`` and ``W`` may be in storage form (``dtype`` "bf16" bit patterns,
    "fp32"), widened exactly block by block.  ``dx_blocks``: indices of the
    blocks whose dx rows are formed (default: all); their rows are returned
    in ``dx`` (stacked in block order) with their row ids in ``dx_rows``.
    ``progress(b, n_blocks)`` is called after each block.
    """
    W = widen(W, dtype)
    t = np.asarray(t, dtype=np.int64)
    N, V = x.shape[0], W.shape[0]
    if N == 0:
        raise ValueError("N must be positive (the mean over zero tokens is undefined)")
    if block < 1:
        raise ValueError("block must be positive")
    if t.shape != (N,) or t.min() < 0 or t.max() >= V:
        raise ValueError("targets out of range")
    n_blocks = (N + block - 1) // block
    want_dx = set(range(n_blocks)) if dx_blocks is None else set(int(b) for b in dx_blocks)
    lse = np.empty(N)
    losses = np.empty(N)
    dW = np.zeros_like(W)
    dx_parts, dx_rows = [], []
    for b in range(n_blocks):
        s, e = b * block, min(N, (b + 1) * block)
        xb = widen(x[s:e], dtype)
        Z = logits(xb, W)
        lse[s:e] = row_logsumexp(Z)
        losses[s:e] = row_losses(Z, t[s:e], lse[s:e])
        G = dlogits(Z, t[s:e], lse[s:e], N)
        del Z
        if b in want_dx:
            dx_parts.append(G @ W)
            dx_rows.append(np.arange(s, e))
        dW += G.T @ xb
        del G
        if progress is not None:
            progress(b, n_blocks)
    H = W.shape[1]
    return {"loss": float(losses.mean()), "lse": lse, "losses": losses, "dW": dW,
            "dx": np.concatenate(dx_parts) if dx_parts else np.zeros((0, H)),
            "dx_rows": np.concatenate(dx_rows) if dx_rows else np.zeros(0, dtype=np.int64)}


def flce_ext(x: np.ndarray, W: np.ndarray, t: np.ndarray, reduction: str = "mean",
             ignore_index=None) -> Dict[str, np.ndarray]:
    """The same materialised computation with the loss options a training loop asks for.

    The 128K-context training guide (sigco.tistory.com), strategy 1 (chunked
    cross-entropy), computes the loss alone, summing per chunk and dividing
    by the token count, through PyTorch's cross_entropy; its tips section
    recommends gradient accumulation.  The pages define no masking, so the
    conventions of that cross_entropy call are taken:

      * a token whose target equals ``ignore_index`` counts for nothing: its
        loss is 0 and its row of G is 0;
      * ``reduction="mean"`` divides the summed loss and every counted row of
        G by the number of counted tokens (0 counted tokens: the loss is
        0 / 0 = NaN and G is all zero); ``"sum"`` divides by nothing.

    With ``ignore_index=None`` and ``"mean"`` this is ``flce``.  Counted
    targets must lie in [0, V).
    """
    if reduction not in ("mean", "sum"):
        raise ValueError(reduction)
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    t = np.asarray(t, dtype=np.int64)
    N = x.shape[0]
    if N == 0:
        raise ValueError("N must be positive")
    counted = np.ones(N, dtype=bool) if ignore_index is None else (t != ignore_index)
    tc = t[counted]
    if tc.size and (tc.min() < 0 or tc.max() >= W.shape[0]):
        raise ValueError("targets out of range")
    n_counted = int(counted.sum())
    Z = logits(x, W)
    lse = row_logsumexp(Z)
    losses = np.zeros(N)
    rows = np.nonzero(counted)[0]
    losses[rows] = lse[rows] - Z[rows, tc]
    if reduction == "sum":
        denom = 1.0
        loss = float(losses.sum())
    else:
        denom = float(n_counted)
        loss = float(losses.sum() / denom) if n_counted else float("nan")
    G = np.zeros_like(Z)
    if n_counted:
        Gc = np.exp(Z[rows] - lse[rows, None])
        Gc[np.arange(rows.size), tc] -= 1.0
        G[rows] = Gc / denom
    del Z
    return {"loss": loss, "dx": G @ W, "dW": G.T @ x, "lse": lse, "losses": losses,
            "counted": n_counted}


def rmsnorm(h: np.ndarray, gamma: np.ndarray, eps: float):
    """x = h / RMS(h) * gamma with RMS(h) = sqrt(mean_k h_k^2 + eps), per row; returns (x, rstd).

    The RMSNorm definition of the "Unsloth deep architecture" page (section on RMSNorm and its
    backward as one kernel); rstd = 1 / RMS(h) is the one value per row that page keeps for the
    backward pass.
    """
    h = np.asarray(h, dtype=np.float64)
    rstd = 1.0 / np.sqrt((h * h).mean(axis=1) + float(eps))
    return h * rstd[:, None] * np.asarray(gamma, dtype=np.float64)[None, :], rstd


def rmsnorm_backward(dx: np.ndarray, h: np.ndarray, gamma: np.ndarray, rstd: np.ndarray):
    """(dh, dgamma) for x = rmsnorm(h, gamma) given dL/dx.

    dh_i = rstd (dx_i g_i - h_i rstd^2 / d * sum_k dx_k g_k h_k): the simplified input derivative
    the same section gives (with 1 / RMS = rstd); dgamma_i = sum_n dx[n,i] h[n,i] rstd_n, the
    derivative of x = h rstd gamma in gamma (the page names dgamma as the kernel's second output
    but prints no formula for it).
    """
    dx = np.asarray(dx, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float64)
    d = h.shape[1]
    s = (dx * g[None, :] * h).sum(axis=1)
    dh = rstd[:, None] * (dx * g[None, :] - h * (rstd ** 2 * s / d)[:, None])
    dgamma = (dx * h * rstd[:, None]).sum(axis=0)
    return dh, dgamma


def rmsnorm_flce(h: np.ndarray, gamma: np.ndarray, eps: float, W: np.ndarray, t: np.ndarray,
                 reduction: str = "mean", ignore_index=None) -> Dict[str, np.ndarray]:
    """The final RMSNorm in front of the LM head, then the loss: x = rmsnorm(h), loss of x W^T.

    Returns loss, dh = dL/dh, dgamma = dL/dgamma, dW, lse and x (all fp64).
    """
    x, rstd = rmsnorm(h, gamma, eps)
    r = flce_ext(x, W, t, reduction=reduction, ignore_index=ignore_index)
    dh, dgamma = rmsnorm_backward(r["dx"], h, gamma, rstd)
    return {"loss": r["loss"], "dh": dh, "dgamma": dgamma, "dW": r["dW"], "lse": r["lse"], "x": x,
            "rstd": rstd, "dx": r["dx"]}


def flce_rows(x: np.ndarray, W: np.ndarray, t: np.ndarray, rows: Iterable[int],
              n_total: int) -> Dict[str, np.ndarray]:
    """lse_n, loss_n and dx_n for selected token rows only.

    The same definition as ``flce`` restricted to the selected rows (a row of
    dx depends only on that token's logits row), so full-size problems can be
    checked on sampled rows; ``n_total`` is the N of the whole problem.
    """
    W = np.asarray(W, dtype=np.float64)
    rows = np.asarray(list(rows), dtype=np.int64)
    xs = np.asarray(x[rows], dtype=np.float64)
    ts = np.asarray(t, dtype=np.int64)[rows]
    Z = logits(xs, W)
    lse = row_logsumexp(Z)
    loss = row_losses(Z, ts, lse)
    G = dlogits(Z, ts, lse, n_total)
    del Z
    return {"lse": lse, "loss": loss, "dx": G @ W}


def flce_sparse_weight(x: np.ndarray, W_nz: np.ndarray, nz: np.ndarray, V: int, t: np.ndarray,
                       dw_rows: Iterable[int]) -> Dict[str, np.ndarray]:
    """``flce`` for a [V,H] weight that is zero outside the rows ``nz``, without forming it.

    The same definition, evaluated where the zero rows make it explicit: a zero row's logit is 0
    for every token, so lse_n = ln(sum_{r in nz} e^{z[n,r]} + (V - |nz|) e^0) with z = x W_nz^T;
    a zero row adds nothing to dx = G W; and a zero row v has G[n,v] = (e^{-lse_n} - [t_n = v]) / N,
    so dW[v] = sum_n G[n,v] x_n needs no logits of its own.  Returns the loss (mean over N), lse
    [N], dx [N,H], and dW for the rows ``dw_rows`` (in that order).  For checking weights too
    large for ``flce`` to hold in host memory; pinned against ``flce`` on small dense cases.
    """
    x = np.asarray(x, dtype=np.float64)
    W_nz = np.asarray(W_nz, dtype=np.float64)
    nz = np.asarray(nz, dtype=np.int64)
    t = np.asarray(t, dtype=np.int64)
    if np.any(np.diff(nz) <= 0) or (len(nz) and (nz[0] < 0 or nz[-1] >= V)):
        raise ValueError("nz must be increasing ids in [0, V)")
    if t.min() < 0 or t.max() >= V:
        raise ValueError("targets out of range")
    N, k = x.shape[0], len(nz)
    n_zero = V - k
    Zs = logits(x, W_nz)                                           # [N, k]
    m = Zs.max(axis=1) if k else np.full(N, -np.inf)
    if n_zero > 0:
        m = np.maximum(m, 0.0)
    lse = m + np.log(np.exp(Zs - m[:, None]).sum(axis=1) + n_zero * np.exp(-m))
    j_t = np.searchsorted(nz, t)
    hit = (j_t < k) & (nz[np.minimum(j_t, max(k - 1, 0))] == t) if k else np.zeros(N, dtype=bool)
    z_t = np.where(hit, Zs[np.arange(N), np.minimum(j_t, max(k - 1, 0))] if k else 0.0, 0.0)
    loss = float((lse - z_t).mean())
    Gs = np.exp(Zs - lse[:, None])
    Gs[np.arange(N)[hit], j_t[hit]] -= 1.0
    Gs /= N
    dx = Gs @ W_nz
    base = (np.exp(-lse) / N) @ x                                  # sum_n e^{-lse_n} x_n / N
    out = []
    for v in dw_rows:
        j = int(np.searchsorted(nz, v))
        if j < k and nz[j] == v:
            out.append(Gs[:, j] @ x)
        else:
            out.append(base - x[t == v].sum(axis=0) / N)
    return {"loss": loss, "lse": lse, "dx": dx, "dW_rows": np.array(out).reshape(len(out), x.shape[1])}


def logits_bytes(n_tokens: int, vocab: int, bytes_per_elem: int) -> int:
    """Size of a materialised [N,V] logits tensor, the footprint FLCE avoids."""
    return int(n_tokens) * int(vocab) * int(bytes_per_elem)
