"""The C-ABI library loads and exports every entry point include/*.h declares (CPU only:
no compute call is made here)."""
import ctypes
import glob
import os
import re

import pytest

import linear_cross_entropy_token_amd as flce

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names.update(re.findall(r"\b(flce_[a-z_]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_boundary():
    names = _declared()
    for required in ("flce_create", "flce_forward_backward", "flce_destroy"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = flce.load_library()
    raw = ctypes.CDLL(flce.library_path())
    for name in _declared():
        assert hasattr(raw, name), name
        assert hasattr(flce, name), f"binding lacks {name}"
    assert lib is flce.load_library()


def test_status_strings():
    for code, name in flce.STATUS.items():
        assert flce.flce_status_string(code).startswith(name)
    assert "unknown" in flce.flce_status_string(99)


def test_effective_chunk_rule():
    # explicit chunks are clamped to [1, N]
    assert flce.flce_effective_chunk(1000, 512, 5000, 384) == 384
    assert flce.flce_effective_chunk(100, 512, 5000, 384) == 100
    # automatic: next_pow2(ceil(N / ceil(V/H))) raised to 4096, capped at 8192, at a 1.5 GB
    # logits buffer and at N
    assert flce.flce_effective_chunk(16384, 4096, 128256, 0) == 4096     # page rule gives 512
    assert flce.flce_effective_chunk(131072, 4096, 128256, 0) == 4096
    assert flce.flce_effective_chunk(1 << 20, 4096, 32000, 0) == 8192
    assert flce.flce_effective_chunk(1 << 20, 4096, 256000, 0) == 2048  # 4096 x 256000 x 2 B > 1.5 GB
    assert flce.flce_effective_chunk(256, 256, 4096, 0) == 256
    assert flce.flce_effective_chunk(0, 256, 4096, 0) == 0


def test_create_validates_before_touching_the_device():
    bad = [flce.Config(7, 0, 0, 0, 0, 0, 0), flce.Config(0, 0, 0, 9, 0, 0, 0),
           flce.Config(0, 0, 0, 0, 0, 1, 0), flce.Config(0, 0, 0, 0, -1, 0, 0)]
    for cfg in bad:
        with pytest.raises(flce.FlceError) as e:
            flce.flce_create(cfg)
        assert e.value.status == 1
    with pytest.raises(flce.FlceError) as e:       # fp32 inputs with bf16 gradients: not built
        flce.flce_create(flce.Config(1, 0, 1, 0, 0, 0, 0))
    assert e.value.status == 2


def test_null_handle_is_rejected():
    assert flce.flce_reserve(None, 10, 8, 10, 0) == 1
    assert flce.flce_check(None, None) == 1
    assert flce.flce_workspace_bytes(None, 10, 8, 10, 0) == 0
    assert flce.flce_forward_backward(None, 1, 1, 1, 1, 8, 1, 0, 1, 1, 1, None) == 1
    assert flce.flce_destroy(None) == 0


def test_wrapper_tensor_checks_on_cpu():
    """The wrapper's checks run before any library call: a CPU tensor is refused, None is skipped."""
    torch = pytest.importorskip("torch")
    from linear_cross_entropy_token_amd import _check_tensors
    _check_tensors(0, (("lse", None, (4,), torch.float32),))
    with pytest.raises(ValueError, match="must be on cuda:0"):
        _check_tensors(0, (("x", torch.zeros(2, 3), (2, 3), torch.float32),))
