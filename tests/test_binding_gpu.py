"""The torch wrapper checks what the C ABI cannot see (plain pointers carry no shape, dtype or
device): outputs of the wrong size or dtype, inputs on the wrong device or with int32 targets are
rejected before any launch, and the handle keeps working afterwards."""
import pytest

from flce_inputs import make_inputs
from flce_testlib import require_gpu, to_device

pytestmark = pytest.mark.gpu


def test_wrapper_rejects_mismatched_tensors():
    torch = require_gpu()
    from linear_cross_entropy_token_amd import FusedLinearCrossEntropy
    N, H, V = 300, 128, 700
    d = make_inputs(N, H, V, "bf16", seed=161)
    x, W, t = to_device(d)
    f = FusedLinearCrossEntropy(dx_dtype=torch.float32, dw_dtype=torch.float32)
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    dx = torch.full((N, H), 7.0, dtype=torch.float32, device="cuda")
    dW = torch.full((V, H), 7.0, dtype=torch.float32, device="cuda")
    bad = {
        "dx dtype": dict(out=(loss, dx.to(torch.bfloat16), dW, None)),
        "dW shape": dict(out=(loss, dx, dW[:-1], None)),
        "lse length": dict(out=(loss, dx, dW, torch.empty(N - 1, device="cuda")), with_lse=True),
        "loss shape": dict(out=(torch.empty(1, device="cuda"), dx, dW, None)),
        "missing dW": dict(out=(loss, dx, None, None)),
    }
    for what, kw in bad.items():
        with pytest.raises(ValueError):
            f.forward_backward(x, W, t, chunk=128, **kw)
        print(f"[binding] rejected: {what}", flush=True)
    with pytest.raises(ValueError):
        f.forward_backward(x, W, t.to(torch.int32), out=(loss, dx, dW, None))
    with pytest.raises(ValueError):
        f.forward_backward(x.cpu(), W, t, out=(loss, dx, dW, None))
    with pytest.raises(ValueError):
        f.forward(x, W[:, :64].contiguous(), t)
    torch.cuda.synchronize()
    assert torch.all(dx == 7.0) and torch.all(dW == 7.0), "a rejected call wrote an output"
    f.forward_backward(x, W, t, chunk=128, out=(loss, dx, dW, None))
    torch.cuda.synchronize()
    assert f.check() == 0
    assert torch.isfinite(loss).item() and not torch.all(dx == 7.0)


def test_abi_rejects_overlapping_outputs():
    """Byte ranges are compared, not just pointers: an output that overlaps an input or another
    output by part of a row is refused with FLCE_ERR_INVALID_ARG before any launch."""
    torch = require_gpu()
    import linear_cross_entropy_token_amd as flce
    N, H, V = 64, 64, 300
    d = make_inputs(N, H, V, "bf16", seed=163)
    x, W, t = to_device(d)
    f = flce.FusedLinearCrossEntropy()
    pool = torch.zeros(4 * (N * H + V * H), dtype=torch.bfloat16, device="cuda")   # room for every layout
    base, row = pool.data_ptr(), H * 2
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    lse = torch.empty(N, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream

    Wbig = torch.zeros(2 * V * H, dtype=torch.bfloat16, device="cuda")   # W with room behind it
    Wbig[: V * H].copy_(W.view(-1))

    def call(xp, dxp, dWp, lsep=None, tp=t.data_ptr(), lossp=loss.data_ptr(), Wp=W.data_ptr()):
        return flce.flce_forward_backward_ex(f.handle, xp, Wp, tp, N, H, V, 0, lossp, dxp, dWp, lsep, s)
    xin = base                                           # x copied into the pool
    pool[: N * H].copy_(x.view(-1))
    free = base + N * H * 2                              # first byte after x
    assert call(xin, xin + row, free + 4 * N * H) == 1   # dx starts one row into x
    assert call(xin, free, free + N * H * 2 - row) == 1  # dW starts inside dx
    assert call(xin, free, free + 2 * N * H, lsep=free + 32) == 1    # lse inside dx
    assert call(xin, free, Wbig.data_ptr() + 16 * row, Wp=Wbig.data_ptr()) == 1   # dW inside W
    assert call(xin, free, free + 2 * N * H, lossp=t.data_ptr() + 8) == 1   # loss inside the targets
    torch.cuda.synchronize()
    assert torch.equal(pool[: N * H], x.view(-1)) and torch.all(pool[N * H:] == 0), "a refused call wrote"
    # adjacent, non-overlapping ranges are accepted and compute the same as separate tensors
    assert call(xin, free, free + N * H * 2, lsep=lse.data_ptr()) == 0
    torch.cuda.synchronize()
    want = f.forward_backward(x, W, t)
    torch.cuda.synchronize()
    dx_pool = pool[N * H: 2 * N * H].view(N, H)
    dW_pool = pool[2 * N * H: 2 * N * H + V * H].view(V, H)
    assert torch.equal(dx_pool, want[1]) and torch.equal(dW_pool, want[2])
