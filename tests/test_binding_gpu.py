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
