"""Helpers shared by the GPU tests: device upload, library calls, error metrics."""
from __future__ import annotations

import numpy as np

import oracle


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X; torch.cuda.is_available() is False")
    return torch


def to_device(d, dev="cuda:0"):
    """Storage-form inputs -> torch device tensors (bf16 bits are reinterpreted, not converted)."""
    import torch
    if d["dtype"] == "bf16":
        x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16)
        W = torch.from_numpy(d["W"].view(np.int16)).view(torch.bfloat16)
    else:
        x = torch.from_numpy(d["x"])
        W = torch.from_numpy(d["W"])
    t = torch.from_numpy(np.ascontiguousarray(d["t"]))
    return x.to(dev), W.to(dev), t.to(dev)


def to_f64(ten):
    import torch
    return ten.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def run_flce(d, chunk=0, dx_dtype=None, dw_dtype=None, with_lse=False, dev="cuda:0", handle=None,
             variant=0):
    import torch
    from linear_cross_entropy_token_amd import FusedLinearCrossEntropy
    x, W, t = to_device(d, dev)
    f = handle or FusedLinearCrossEntropy(in_dtype=x.dtype, dx_dtype=dx_dtype, dw_dtype=dw_dtype,
                                          variant=variant)
    out = f.forward_backward(x, W, t, chunk=chunk, with_lse=with_lse)
    torch.cuda.synchronize()
    res = {"loss": float(out[0].item()), "dx": to_f64(out[1]), "dW": to_f64(out[2])}
    if with_lse:
        res["lse"] = to_f64(out[3])
    res["handle"] = f
    return res


def rel_fro(a, b):
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def oracle_full(d):
    return oracle.flce(oracle.widen(d["x"], d["dtype"]), oracle.widen(d["W"], d["dtype"]), d["t"])


def compare(got, want, t, V, tol_grad, tol_loss=1e-4, what=""):
    """Loss relative error, dx/dW relative Frobenius error, and dW on never-targeted rows
    (pure softmax part, which the one-hot term would otherwise dominate)."""
    errs = {
        "loss": abs(got["loss"] - want["loss"]) / abs(want["loss"]),
        "dx": rel_fro(got["dx"], want["dx"]),
        "dW": rel_fro(got["dW"], want["dW"]),
    }
    untargeted = np.ones(V, dtype=bool)
    untargeted[np.asarray(t)] = False
    if untargeted.any():
        errs["dW_untargeted"] = rel_fro(got["dW"][untargeted], want["dW"][untargeted])
    msg = f"{what}: {errs}"
    assert np.isfinite(got["loss"]), msg
    assert errs["loss"] <= tol_loss, msg
    assert errs["dx"] <= tol_grad, msg
    assert errs["dW"] <= tol_grad, msg
    if "dW_untargeted" in errs:
        assert errs["dW_untargeted"] <= tol_grad, msg
    return errs
