"""Every full-size bf16 workload against the whole oracle (GPU only).

The HIP path runs in the benchmark's launch configuration (chunked variant, the
workload's chunk, bf16 dx and dW); the oracle is ``oracle.flce_blocked``, the
plain fp64 definition evaluated one block of 4096 token rows at a time (pinned
against ``oracle.flce`` and the whole pin suite in tests/test_oracle_pins.py).
Nothing is sampled except where stated: the loss, every token's log-sum-exp,
every dx row and every dW row are compared.

Tolerances (the benchmark spec): loss relative error <= 1e-4; dx and dW relative
Frobenius error <= 2e-2 (bf16 inputs), and the same bound on the dW rows no
target hits (there dW is the softmax part alone, which the one-hot part would
otherwise hide); every lse within 1e-4 of the oracle's relative to max |lse|.

Every workload also runs the fused variant with fp32 gradients (its benchmark
configuration: with bf16 dW it would need an fp32 dW accumulator beyond its memory
bound) against the same oracle result; its pass-2 block shape is planned per
launch, so the workloads cover several shapes and step counts.  The
Llama-3-vocabulary workload further runs the chunked variant with fp32 gradients
and in a single chunk.  The long-context workload (N = 131,072) compares the loss,
all lse and all of dW, and dx on five whole 4096-row blocks (the first two,
two in the middle, the last), since its [N,H] fp64 dx alone would be 4.3 GB on
the host and every dx row depends on its own token only.
"""
import numpy as np
import pytest

import oracle
from flce_inputs import make_inputs, WORKLOADS
from flce_testlib import require_gpu, to_device, rel_fro

pytestmark = pytest.mark.gpu

BLOCK = 4096


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _say(capsys, msg):
    # progress reaches the terminal while the oracle runs (minutes at the largest size)
    with capsys.disabled():
        print(msg, flush=True)


def _oracle(d, capsys, name, dx_blocks=None):
    def progress(b, n):
        if b % 4 == 3 or b == n - 1:
            _say(capsys, f"  [oracle {name}] block {b + 1}/{n}")
    return oracle.flce_blocked(d["x"], d["W"], d["t"], block=BLOCK, dtype=d["dtype"], dx_blocks=dx_blocks,
                               progress=progress)


def _run(d, chunk, variant=0, grads=None, dx_rows=None):
    """One call through the C ABI on device-resident inputs; dx comes back for dx_rows only."""
    import torch
    from linear_cross_entropy_token_amd import FusedLinearCrossEntropy
    x, W, t = to_device(d)
    f = FusedLinearCrossEntropy(in_dtype=x.dtype, dx_dtype=grads, dw_dtype=grads, variant=variant)
    loss, dx, dW, lse = f.forward_backward(x, W, t, chunk=chunk, with_lse=True)
    torch.cuda.synchronize()
    status = f.check()
    f.close()
    del x, W, t
    rows = slice(None) if dx_rows is None else torch.as_tensor(dx_rows, device=dx.device)
    out = {"loss": float(loss.item()), "lse": lse.double().cpu().numpy(),
           "dx": dx[rows].double().cpu().numpy(), "dW": dW.double().cpu().numpy(), "status": status}
    del dx, dW
    torch.cuda.empty_cache()
    return out


def _check(got, want, t, V, what, capsys):
    errs = {
        "loss": abs(got["loss"] - want["loss"]) / abs(want["loss"]),
        "lse": float(np.max(np.abs(got["lse"] - want["lse"])) / np.max(np.abs(want["lse"]))),
        "dx": rel_fro(got["dx"], want["dx"]),
        "dW": rel_fro(got["dW"], want["dW"]),
    }
    untargeted = np.ones(V, dtype=bool)
    untargeted[np.asarray(t)] = False
    errs["dW_untargeted"] = rel_fro(got["dW"][untargeted], want["dW"][untargeted])
    _say(capsys, f"  [{what}] loss {got['loss']:.7f} (oracle {want['loss']:.7f}) "
                 + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    msg = f"{what}: {errs}"
    assert got["status"] == 0, msg
    assert errs["loss"] <= 1e-4, msg
    assert errs["lse"] <= 1e-4, msg
    assert errs["dx"] <= 2e-2, msg
    assert errs["dW"] <= 2e-2, msg
    assert errs["dW_untargeted"] <= 2e-2, msg
    return errs


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["llama2_vocab", "llama3_dp8_share", "llama3_tp8_share", "qwen3_vocab"])
def test_full_size_vs_oracle(name, capsys):
    import torch
    w = WORKLOADS[name]
    _say(capsys, f"\n[full-size] {name}: N={w.N} H={w.H} V={w.V} chunk={w.chunk}")
    d = make_inputs(w.N, w.H, w.V, w.dtype, w.seed, w.targets)
    runs = {"chunked bf16 grads": _run(d, w.chunk),
            "fused fp32 grads": _run(d, w.chunk, variant=1, grads=torch.float32)}
    want = _oracle(d, capsys, name)
    for what, got in runs.items():
        _check(got, want, d["t"], w.V, f"{name}, {what}", capsys)


@pytest.mark.timeout(900)
def test_llama3_full_size_both_variants_vs_oracle(capsys):
    """The benchmark workload: chunked with bf16 gradients (the benchmark's configuration, and
    again in a single chunk of all tokens), then chunked and fused with fp32 gradients and fused
    with bf16 gradients, all against one oracle result.  On fp32 outputs the
    exact invariants of the definition hold as well: dW's column sums vanish (every G row sums
    to zero) and <x,dx> = <W,dW> (z = x W^T is bilinear)."""
    import torch
    w = WORKLOADS["llama3_vocab"]
    _say(capsys, f"\n[full-size] llama3_vocab: N={w.N} H={w.H} V={w.V} chunk={w.chunk}")
    d = make_inputs(w.N, w.H, w.V, w.dtype, w.seed, w.targets)
    runs = {"chunked bf16 grads": _run(d, w.chunk),
            # all 16,384 tokens in one chunk: a 4.20 GB logits buffer, just under the kernels'
            # 32-bit offset limit, so its last rows sit at the largest offsets of every launch
            "chunked bf16 grads, one chunk": _run(d, w.N),
            "chunked fp32 grads": _run(d, w.chunk, grads=torch.float32),
            "fused fp32 grads": _run(d, w.chunk, variant=1, grads=torch.float32),
            # bf16 dx and dW, the chunked benchmark configuration: dW stored once per chunk
            "fused bf16 grads": _run(d, w.chunk, variant=1)}
    want = _oracle(d, capsys, "llama3_vocab")
    for what, got in runs.items():
        _check(got, want, d["t"], w.V, what, capsys)
    x64 = oracle.widen(d["x"], "bf16")
    W64 = oracle.widen(d["W"], "bf16")
    for what in ("chunked fp32 grads", "fused fp32 grads"):
        g = runs[what]
        colsum = np.linalg.norm(g["dW"].sum(axis=0)) / np.linalg.norm(g["dW"])
        a, b = float(np.sum(x64 * g["dx"])), float(np.sum(W64 * g["dW"]))
        _say(capsys, f"  [{what}] |colsum dW|/|dW| {colsum:.2e}  <x,dx> {a:.6e} <W,dW> {b:.6e}")
        assert colsum <= 1e-3
        assert abs(a - b) <= 1e-3 * max(abs(a), abs(b))


@pytest.mark.timeout(1200)
def test_long_context_full_size_vs_oracle(capsys):
    import torch
    w = WORKLOADS["long_context"]
    _say(capsys, f"\n[full-size] long_context: N={w.N} H={w.H} V={w.V} chunk={w.chunk}")
    d = make_inputs(w.N, w.H, w.V, w.dtype, w.seed, w.targets)
    nb = w.N // BLOCK
    blocks = [0, 1, nb // 2 - 1, nb // 2, nb - 1]
    rows = np.concatenate([np.arange(b * BLOCK, (b + 1) * BLOCK) for b in blocks])
    runs = {"chunked bf16 grads": _run(d, w.chunk, dx_rows=rows),
            "fused fp32 grads": _run(d, w.chunk, variant=1, grads=torch.float32, dx_rows=rows)}
    want = _oracle(d, capsys, "long_context", dx_blocks=blocks)
    assert np.array_equal(want["dx_rows"], rows)
    for what, got in runs.items():
        _check(got, want, d["t"], w.V, f"long_context, {what}", capsys)
