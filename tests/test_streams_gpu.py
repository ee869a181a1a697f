"""Handles are independent and every kernel runs on the caller's stream: two handles driven on two
side streams at once give bitwise the results each gives alone (the chunked path is
deterministic), and both match the oracle.  Streams are created at the default priority."""
import pytest

from flce_inputs import make_inputs
from flce_testlib import require_gpu, to_device, to_f64, oracle_full, compare

pytestmark = pytest.mark.gpu

# (N, H, V, chunk, dW dtype): two chunked calls of different shapes, several chunks each
CASES = [(900, 264, 3000, 256, None), (700, 512, 2500, 300, "fp32")]


def _setup(torch):
    from linear_cross_entropy_token_amd import FusedLinearCrossEntropy
    runs = []
    for k, (N, H, V, C, dw) in enumerate(CASES):
        d = make_inputs(N, H, V, "bf16", seed=151 + k)
        x, W, t = to_device(d)
        f = FusedLinearCrossEntropy(dw_dtype=torch.float32 if dw == "fp32" else None)
        f.reserve(N, H, V, C)
        out = (torch.empty((), dtype=torch.float32, device="cuda"), torch.empty_like(x),
               torch.empty(W.shape, dtype=torch.float32 if dw == "fp32" else W.dtype, device="cuda"),
               torch.empty(N, dtype=torch.float32, device="cuda"))
        runs.append(dict(d=d, x=x, W=W, t=t, C=C, f=f, out=out))
    return runs


def _call(r, stream):
    r["f"].forward_backward(r["x"], r["W"], r["t"], chunk=r["C"], with_lse=True, out=r["out"], stream=stream)


def test_two_handles_on_two_streams():
    torch = require_gpu()
    runs = _setup(torch)
    # each call alone, on the default stream
    alone = []
    for r in runs:
        _call(r, torch.cuda.current_stream())
        torch.cuda.synchronize()
        alone.append([o.clone() for o in r["out"]])
        assert r["f"].check() == 0
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for r in runs:                          # scribble over the outputs first
            for o in r["out"]:
                o.fill_(float(rep + 3))
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        # interleave the two calls' enqueueing so that their kernels overlap on the device
        for r, s in zip(runs, streams):
            with torch.cuda.stream(s):
                _call(r, s)
        for s in streams:
            torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for k, (r, want) in enumerate(zip(runs, alone)):
            for name, e, g in zip(("loss", "dx", "dW", "lse"), want, r["out"]):
                assert torch.equal(e, g), f"repeat {rep}, call {k}: {name} differs from the call alone"
    for r, (N, H, V, C, dw) in zip(runs, CASES):
        want = oracle_full(r["d"])
        got = {"loss": float(r["out"][0].item()), "dx": to_f64(r["out"][1]), "dW": to_f64(r["out"][2])}
        compare(got, want, r["d"]["t"], V, tol_grad=2e-2, what=f"N={N} H={H} V={V} C={C} dW={dw or 'bf16'}")


def test_fused_and_chunked_handles_on_two_streams():
    """A fused call (its pass-2 kernels hold no waits on other workgroups, so they may share the
    device with any other kernel) overlapping a chunked call on another stream: both match the
    oracle, and the chunked one is bitwise what it gives alone."""
    import torch as _t
    torch = require_gpu()
    from linear_cross_entropy_token_amd import FusedLinearCrossEntropy, FLCE_FUSED
    shapes = [(900, 264, 3000, 256), (1000, 512, 5000, 384)]
    runs = []
    for k, (N, H, V, C) in enumerate(shapes):
        d = make_inputs(N, H, V, "bf16", seed=171 + k)
        x, W, t = to_device(d)
        fused = k == 1
        f = FusedLinearCrossEntropy(variant=FLCE_FUSED if fused else 0,
                                    dx_dtype=_t.float32 if fused else None, dw_dtype=_t.float32 if fused else None)
        f.reserve(N, H, V, C)
        gd = _t.float32 if fused else x.dtype
        out = (torch.empty((), dtype=torch.float32, device="cuda"), torch.empty(x.shape, dtype=gd, device="cuda"),
               torch.empty(W.shape, dtype=gd, device="cuda"), torch.empty(N, dtype=torch.float32, device="cuda"))
        runs.append(dict(d=d, x=x, W=W, t=t, C=C, f=f, out=out, fused=fused))
    _call(runs[0], torch.cuda.current_stream())
    torch.cuda.synchronize()
    alone = [o.clone() for o in runs[0]["out"]]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for r, s in zip(runs, streams):
        with torch.cuda.stream(s):
            _call(r, s)
    for s in streams:
        torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for name, e, g in zip(("loss", "dx", "dW", "lse"), alone, runs[0]["out"]):
        assert torch.equal(e, g), f"chunked call next to a fused one: {name} differs from the call alone"
    for r, (N, H, V, C) in zip(runs, shapes):
        assert r["f"].check() == 0
        want = oracle_full(r["d"])
        got = {"loss": float(r["out"][0].item()), "dx": to_f64(r["out"][1]), "dW": to_f64(r["out"][2])}
        compare(got, want, r["d"]["t"], V, tol_grad=2e-2, what=f"{'fused' if r['fused'] else 'chunked'} N={N}")
