"""Boundary behaviour of the C ABI that needs a device (GPU only).

Failures forced from the host (a workspace limit), the asynchrony of a call (it returns
after enqueueing, before the stream has run its kernels: the default-stream and events
sections of the async continuous-batching page), and the graph-capture rules the header
states (nothing allocated under capture; a captured workspace never moves)."""
import time

import numpy as np
import pytest

import linear_cross_entropy_token_amd as flce
from flce_inputs import make_inputs, WORKLOADS
from flce_testlib import require_gpu, to_device

pytestmark = pytest.mark.gpu

OK, INVALID, UNSUPPORTED, OOM = 0, 1, 2, 3


def _bufs(torch, N, H, V, dt):
    loss = torch.full((), 123.0, dtype=torch.float32, device="cuda")
    dx = torch.full((N, H), 7.0, dtype=dt, device="cuda")
    dW = torch.full((V, H), -3.0, dtype=dt, device="cuda")
    return loss, dx, dW


def _raw_call(f, x, W, t, chunk, loss, dx, dW, stream):
    N, H = x.shape
    return flce.flce_forward_backward(f.handle, x.data_ptr(), W.data_ptr(), t.data_ptr(), N, H, W.shape[0],
                                      chunk, loss.data_ptr(), dx.data_ptr(), dW.data_ptr(), stream.cuda_stream)


def test_workspace_limit_gives_oom_and_leaves_outputs_untouched():
    torch = require_gpu()
    N, H, V, C = 600, 256, 3000, 256
    d = make_inputs(N, H, V, "bf16", seed=301)
    x, W, t = to_device(d)
    probe = flce.FusedLinearCrossEntropy()
    need = probe.workspace_bytes(N, H, V, C)
    probe.close()
    assert need > 0
    for variant in (flce.FLCE_CHUNKED, flce.FLCE_FUSED):
        f = flce.FusedLinearCrossEntropy(variant=variant, workspace_limit=1024)
        loss, dx, dW = _bufs(torch, N, H, V, torch.bfloat16)
        s = torch.cuda.current_stream()
        assert _raw_call(f, x, W, t, C, loss, dx, dW, s) == OOM
        assert flce.flce_reserve(f.handle, N, H, V, C) == OOM
        torch.cuda.synchronize()
        assert loss.item() == 123.0
        assert bool((dx == 7.0).all()) and bool((dW == -3.0).all())
        f.close()
    # a limit just large enough lets the same call through
    f = flce.FusedLinearCrossEntropy(workspace_limit=need)
    loss, dx, dW = _bufs(torch, N, H, V, torch.bfloat16)
    assert _raw_call(f, x, W, t, C, loss, dx, dW, torch.cuda.current_stream()) == OK
    torch.cuda.synchronize()
    assert np.isfinite(loss.item()) and loss.item() != 123.0
    f.close()


def test_call_returns_before_the_stream_completes():
    """At the Llama-3-vocabulary size a call is ~45 ms of GPU work; with the workspace reserved
    it must return after enqueueing, while the stream still has work (hipStreamQuery not ready)."""
    torch = require_gpu()
    w = WORKLOADS["llama3_vocab"]
    d = make_inputs(w.N, w.H, w.V, w.dtype, w.seed, w.targets)
    x, W, t = to_device(d)
    f = flce.FusedLinearCrossEntropy()
    f.reserve(w.N, w.H, w.V, w.chunk)
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    dx, dW = torch.empty_like(x), torch.empty_like(W)
    s = torch.cuda.current_stream()
    assert _raw_call(f, x, W, t, w.chunk, loss, dx, dW, s) == OK      # warm-up
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(s)
    t0 = time.perf_counter()
    assert _raw_call(f, x, W, t, w.chunk, loss, dx, dW, s) == OK
    host_s = time.perf_counter() - t0
    pending = not s.query()
    ev1.record(s)
    torch.cuda.synchronize()
    gpu_ms = ev0.elapsed_time(ev1)
    print(f"[async] enqueue {host_s * 1e3:.2f} ms on the host, {gpu_ms:.1f} ms on the stream, "
          f"pending after return: {pending}", flush=True)
    assert pending, "the stream had finished when the call returned: the call synchronised"
    assert host_s * 1e3 < 0.5 * gpu_ms
    assert f.check() == OK
    f.close()


def test_capture_needs_a_reserved_workspace_and_pins_it():
    torch = require_gpu()
    N, H, V, C = 512, 256, 2000, 256
    d = make_inputs(N, H, V, "bf16", seed=302)
    x, W, t = to_device(d)
    loss, dx, dW = _bufs(torch, N, H, V, torch.bfloat16)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()

    # 1. nothing reserved: the captured call cannot allocate and fails before enqueueing anything
    f = flce.FusedLinearCrossEntropy()
    marker = torch.zeros(4, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        st = _raw_call(f, x, W, t, C, loss, dx, dW, side)
        marker.add_(1.0)                       # the graph holds this kernel and nothing of the call
    assert st == UNSUPPORTED
    g.replay()
    torch.cuda.synchronize()
    assert marker[0].item() == 1.0
    assert loss.item() == 123.0 and bool((dx == 7.0).all())

    # 2. reserved: the call is captured, and the workspace is pinned from then on
    f.reserve(N, H, V, C)
    ws_bytes = f.workspace_bytes(N, H, V, C)
    with torch.cuda.stream(side):
        assert _raw_call(f, x, W, t, C, loss, dx, dW, side) == OK   # eager warm-up on the side stream
    torch.cuda.synchronize()
    want = [loss.clone(), dx.clone(), dW.clone()]
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2, stream=side):
        st = _raw_call(f, x, W, t, C, loss, dx, dW, side)
    assert st == OK
    # a call needing a larger workspace is refused (before any launch) instead of moving it
    N2 = 2 * N
    d2 = make_inputs(N2, H, V, "bf16", seed=303)
    x2, W2, t2 = to_device(d2)
    assert f.workspace_bytes(N2, H, V, 2 * C) > ws_bytes
    loss2, dx2, dW2 = _bufs(torch, N2, H, V, torch.bfloat16)
    assert _raw_call(f, x2, W2, t2, 2 * C, loss2, dx2, dW2, torch.cuda.current_stream()) == UNSUPPORTED
    assert flce.flce_reserve(f.handle, N2, H, V, 2 * C) == UNSUPPORTED
    torch.cuda.synchronize()
    assert loss2.item() == 123.0 and bool((dx2 == 7.0).all()) and bool((dW2 == -3.0).all())
    # the captured graph still replays into the same workspace and gives the eager result
    for o in (loss, dx, dW):
        o.fill_(5.0)
    g2.replay()
    torch.cuda.synchronize()
    for a, b in zip(want, (loss, dx, dW)):
        assert torch.equal(a, b)
    # calls that fit the pinned workspace still run eagerly
    assert _raw_call(f, x, W, t, C, loss, dx, dW, torch.cuda.current_stream()) == OK
    torch.cuda.synchronize()
    assert torch.equal(want[1], dx)
    assert f.check() == OK
    f.close()
