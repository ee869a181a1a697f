"""A call enqueues kernels only (no host synchronisation, no allocation once the workspace is
reserved, no memset nodes), so it can be captured in a HIP graph.  Each test captures one call,
replays the graph several times with eager work and synchronisations in between, and checks
every replay against the eager result (bitwise for the deterministic chunked path)."""
import pytest

from flce_inputs import make_inputs
from flce_testlib import require_gpu, to_device, to_f64, rel_fro

pytestmark = pytest.mark.gpu


def _capture_and_replay(fn, outs, replays=3):
    torch = require_gpu()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    results = []
    for k in range(replays):
        for o in outs:                         # scribble over the outputs between replays
            o.fill_(float(k + 7))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        results.append([o.clone() for o in outs])
        _ = (torch.randn(1024, device="cuda") * 2).sum().item()   # unrelated eager work
    return eager, results


def test_chunked_call_replays_bitwise():
    torch = require_gpu()
    from linear_cross_entropy_token_amd import FusedLinearCrossEntropy
    d = make_inputs(700, 256, 3000, "bf16", seed=131)
    x, W, t = to_device(d)
    f = FusedLinearCrossEntropy()
    f.reserve(700, 256, 3000, 256)
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    dx, dW = torch.empty_like(x), torch.empty_like(W)
    lse = torch.empty(700, dtype=torch.float32, device="cuda")
    outs = [loss, dx, dW, lse]

    def call():
        f.forward_backward(x, W, t, chunk=256, with_lse=True, out=(loss, dx, dW, lse),
                           stream=torch.cuda.current_stream())
    eager, results = _capture_and_replay(call, outs)
    assert f.check() == 0
    for k, res in enumerate(results):
        for name, e, r in zip(("loss", "dx", "dW", "lse"), eager, res):
            assert torch.equal(e, r), f"replay {k}: {name} differs from the eager call"


def test_options_call_replays_bitwise():
    """ignore_index and the device-side token count inside a graph."""
    torch = require_gpu()
    from linear_cross_entropy_token_amd import FusedLinearCrossEntropy
    d = make_inputs(520, 264, 1300, "bf16", seed=137)
    d["t"] = d["t"].copy()
    d["t"][::5] = -100
    x, W, t = to_device(d)
    f = FusedLinearCrossEntropy()
    f.reserve(520, 264, 1300, 200)
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    dx, dW = torch.empty_like(x), torch.empty_like(W)
    outs = [loss, dx, dW]

    def call():
        f.forward_backward(x, W, t, chunk=200, out=(loss, dx, dW, None), ignore_index=-100,
                           stream=torch.cuda.current_stream())
    eager, results = _capture_and_replay(call, outs)
    for k, res in enumerate(results):
        for name, e, r in zip(("loss", "dx", "dW"), eager, res):
            assert torch.equal(e, r), f"replay {k}: {name} differs from the eager call"


def test_fused_call_replays():
    """The fused variant's accumulators are cleared by fill kernels inside the graph; its fp32
    atomics make the order of additions vary, so replays are compared within a tolerance."""
    torch = require_gpu()
    from linear_cross_entropy_token_amd import FusedLinearCrossEntropy, FLCE_FUSED
    d = make_inputs(600, 256, 2100, "bf16", seed=139)
    x, W, t = to_device(d)
    f = FusedLinearCrossEntropy(dx_dtype=torch.float32, dw_dtype=torch.float32, variant=FLCE_FUSED)
    f.reserve(600, 256, 2100, 300)
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    dx = torch.empty(x.shape, dtype=torch.float32, device="cuda")
    dW = torch.empty(W.shape, dtype=torch.float32, device="cuda")
    outs = [loss, dx, dW]

    def call():
        f.forward_backward(x, W, t, chunk=300, out=(loss, dx, dW, None), stream=torch.cuda.current_stream())
    eager, results = _capture_and_replay(call, outs)
    for k, res in enumerate(results):
        assert float(res[0].item()) == float(eager[0].item()), f"replay {k}: loss"
        for name, e, r in zip(("dx", "dW"), eager[1:], res[1:]):
            err = rel_fro(to_f64(r), to_f64(e))
            assert err <= 1e-5, f"replay {k}: {name} rel err {err}"
