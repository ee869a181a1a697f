"""Maximum sizes.  The kernels address W, one chunk of x and the chunk's logits buffer through 32-bit
buffer offsets, so the ABI refuses any of them at 4 GiB or more (FLCE_ERR_UNSUPPORTED, before any
work); the largest weight it accepts runs correctly, its highest rows included.

Largest accepted weight: V = 262,000, H = 8,192 bf16 (4.29 GB, just under the limit), N = 256
tokens, zero except ~1,000 random rows (the last 512, whose offsets are the largest, and 512 spread
over V), so that the oracle's ``flce_sparse_weight`` (the definition with the zero rows' logits,
all 0, in closed form; pinned against ``flce``) checks it in host memory and time: the loss, every
row's lse and dx, and dW on sampled rows (every targeted row, nonzero and zero rows spread over V,
the last rows), at the bf16 tolerances (loss <= 1e-4 relative, dx and the dW sample <= 2e-2
relative Frobenius).
"""
import numpy as np
import pytest

import oracle
from flce_inputs import make_inputs
from flce_testlib import require_gpu, to_device, to_f64, rel_fro

pytestmark = pytest.mark.gpu


def test_sizes_at_the_32bit_limit_are_refused():
    torch = require_gpu()
    import linear_cross_entropy_token_amd as flce
    f = flce.FusedLinearCrossEntropy()
    assert flce.flce_reserve(f.handle, 256, 8192, 262144, 0) == 2          # W = 4 GiB
    assert flce.flce_workspace_bytes(f.handle, 256, 8192, 262144, 0) == 0
    assert flce.flce_reserve(f.handle, 20000, 4096, 128256, 20000) == 2    # chunk buffer 5.1 GB
    assert flce.flce_reserve(f.handle, 256, 8192, 262000, 0) == 0          # just under: accepted
    fu = flce.FusedLinearCrossEntropy(variant=flce.FLCE_FUSED, dw_dtype=torch.float32)
    assert flce.flce_reserve(fu.handle, 256, 8192, 131072, 0) == 2         # fp32 dW accumulator >= 4 GiB
    f.close()
    fu.close()


def test_largest_weight_under_the_limit():
    """W of 262,000 x 8,192 bf16 (4.29 GB), zero except ~1,000 random rows: the last 512 (the
    largest offsets) and 512 spread over V; half the tokens target nonzero rows, half zero rows."""
    torch = require_gpu()
    from linear_cross_entropy_token_amd import FusedLinearCrossEntropy
    N, H, V = 256, 8192, 262000
    nz = np.unique(np.concatenate([np.linspace(0, V - 600, 512).astype(np.int64), np.arange(V - 512, V)]))
    d = make_inputs(N, H, len(nz), "bf16", seed=181)
    rng = np.random.default_rng(183)
    zero_rows = np.setdiff1d(np.arange(V), nz)
    t = np.where(np.arange(N) % 2 == 0, nz[d["t"]], rng.choice(zero_rows, N))
    print(f"[max size] N={N} H={H} V={V} bf16 (W {V * H * 2 / 1e9:.2f} GB, {len(nz)} nonzero rows)", flush=True)
    x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).cuda()
    W = torch.zeros((V, H), dtype=torch.bfloat16, device="cuda")
    W[torch.from_numpy(nz).cuda()] = torch.from_numpy(d["W"].view(np.int16)).view(torch.bfloat16).cuda()
    tt = torch.from_numpy(t).cuda()
    f = FusedLinearCrossEntropy()
    loss, dx, dW, lse = f.forward_backward(x, W, tt, with_lse=True)
    torch.cuda.synchronize()
    assert f.check() == 0
    rows = np.unique(np.concatenate([t, nz[::16], zero_rows[::20000], np.arange(V - 8, V)]))
    got = {"loss": float(loss.item()), "lse": to_f64(lse), "dx": to_f64(dx),
           "dW": to_f64(dW[torch.from_numpy(rows).cuda()])}
    del x, W, dx, dW, lse
    f.close()
    torch.cuda.empty_cache()
    want = oracle.flce_sparse_weight(oracle.widen(d["x"], "bf16"), oracle.widen(d["W"], "bf16"), nz, V, t, rows)
    print(f"[max size] loss {got['loss']:.6f} vs {want['loss']:.6f}", flush=True)
    assert abs(got["loss"] - want["loss"]) / abs(want["loss"]) <= 1e-4
    assert np.max(np.abs(got["lse"] - want["lse"])) <= 1e-4 * np.max(np.abs(want["lse"]))
    assert rel_fro(got["dx"], want["dx"]) <= 2e-2
    assert rel_fro(got["dW"], want["dW_rows"]) <= 2e-2
    last = rows >= V - 8                                  # the highest offsets on their own
    assert rel_fro(got["dW"][last], want["dW_rows"][last]) <= 2e-2
    untargeted = ~np.isin(rows, t)                        # pure softmax rows
    assert rel_fro(got["dW"][untargeted], want["dW_rows"][untargeted]) <= 2e-2
