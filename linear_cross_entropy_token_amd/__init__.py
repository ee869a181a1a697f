"""MI355X-native fused linear cross-entropy (FLCE).

A thin Python binding over ``libflce.so`` (hand-written HIP kernels for
gfx950 behind the C ABI declared in ``include/flce.h``).  The functions
``flce_create``, ``flce_forward_backward`` ... mirror the C entry points one
to one and only marshal arguments; every step of the computation runs in the
library's kernels.  ``FusedLinearCrossEntropy`` is a convenience wrapper that
takes torch device tensors (torch supplies device memory and the stream).

There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "FLCE_BF16", "FLCE_FP32", "FLCE_CHUNKED", "FLCE_FUSED", "STATUS", "FlceError", "Config",
    "library_path", "load_library", "flce_create", "flce_destroy", "flce_forward_backward",
    "flce_forward_backward_ex", "flce_forward_backward_opt", "flce_forward_backward_noalloc", "Options", "FLCE_MEAN", "FLCE_SUM",
    "FLCE_ACCUMULATE", "FLCE_FORWARD_ONLY", "flce_effective_chunk", "flce_workspace_bytes", "flce_workspace_bytes_opt", "flce_reserve",
    "flce_rmsnorm_forward_backward", "flce_rmsnorm_workspace_bytes",
    "flce_check", "flce_status_string", "flce_profile_enable", "flce_profile_read", "KernelStat",
    "FusedLinearCrossEntropy",
]

FLCE_BF16, FLCE_FP32 = 0, 1
FLCE_CHUNKED, FLCE_FUSED = 0, 1
FLCE_MEAN, FLCE_SUM = 0, 1
FLCE_ACCUMULATE, FLCE_FORWARD_ONLY = 1, 2
STATUS = {0: "FLCE_OK", 1: "FLCE_ERR_INVALID_ARG", 2: "FLCE_ERR_UNSUPPORTED", 3: "FLCE_ERR_OOM",
          4: "FLCE_ERR_HIP", 5: "FLCE_ERR_DATA"}


class FlceError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {flce_status_string(status)}" if what else flce_status_string(status))


class Config(ctypes.Structure):
    _fields_ = [("in_dtype", ctypes.c_int32), ("dx_dtype", ctypes.c_int32),
                ("dw_dtype", ctypes.c_int32), ("variant", ctypes.c_int32),
                ("device", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("workspace_limit", ctypes.c_int64)]


class Options(ctypes.Structure):
    _fields_ = [("reduction", ctypes.c_int32), ("flags", ctypes.c_int32), ("ignore_on", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("ignore_index", ctypes.c_int64)]


class KernelStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double),
                ("flops", ctypes.c_double), ("bytes", ctypes.c_double), ("sclk_mhz", ctypes.c_double)]


_lib: Optional[ctypes.CDLL] = None


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflce.so")


def load_library() -> ctypes.CDLL:
    """Loads libflce.so (raises OSError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise OSError(f"{path} is missing: build it with `python -m linear_cross_entropy_token_amd.build`")
    # One HIP runtime per process: torch ships its own libamdhip64, and a process that loads
    # this library first and torch afterwards ends up with two runtimes that fail each other's
    # calls.  Loading torch first makes the library bind to torch's runtime.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.flce_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(vp)]
    lib.flce_create.restype = i32
    lib.flce_destroy.argtypes = [vp]
    lib.flce_destroy.restype = i32
    lib.flce_forward_backward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, vp, vp, vp]
    lib.flce_forward_backward.restype = i32
    lib.flce_forward_backward_ex.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, vp, vp, vp, vp]
    lib.flce_forward_backward_ex.restype = i32
    lib.flce_forward_backward_opt.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, ctypes.POINTER(Options),
                                              vp, vp, vp, vp, vp]
    lib.flce_forward_backward_opt.restype = i32
    lib.flce_forward_backward_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, vp, vp, vp]
    lib.flce_forward_backward_noalloc.restype = i32
    lib.flce_effective_chunk.argtypes = [i64, i64, i64, i64]
    lib.flce_effective_chunk.restype = i64
    lib.flce_workspace_bytes.argtypes = [vp, i64, i64, i64, i64]
    lib.flce_workspace_bytes.restype = ctypes.c_size_t
    lib.flce_workspace_bytes_opt.argtypes = [vp, i64, i64, i64, i64, ctypes.POINTER(Options)]
    lib.flce_workspace_bytes_opt.restype = ctypes.c_size_t
    lib.flce_rmsnorm_forward_backward.argtypes = [vp, vp, vp, ctypes.c_float, vp, vp, i64, i64, i64, i64,
                                                  ctypes.POINTER(Options), vp, vp, vp, vp, vp, vp]
    lib.flce_rmsnorm_forward_backward.restype = i32
    lib.flce_rmsnorm_workspace_bytes.argtypes = [vp, i64, i64, i64, i64, ctypes.POINTER(Options)]
    lib.flce_rmsnorm_workspace_bytes.restype = ctypes.c_size_t
    lib.flce_reserve.argtypes = [vp, i64, i64, i64, i64]
    lib.flce_reserve.restype = i32
    lib.flce_check.argtypes = [vp, vp]
    lib.flce_check.restype = i32
    lib.flce_profile_enable.argtypes = [vp, i32]
    lib.flce_profile_enable.restype = i32
    lib.flce_profile_read.argtypes = [vp, ctypes.POINTER(KernelStat), i32, ctypes.POINTER(i32)]
    lib.flce_profile_read.restype = i32
    lib.flce_status_string.argtypes = [i32]
    lib.flce_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


# ---- one-to-one wrappers of the C entry points (plain ints/pointers) -------

def flce_status_string(status: int) -> str:
    return load_library().flce_status_string(int(status)).decode()


def flce_create(cfg: Config) -> int:
    h = ctypes.c_void_p()
    st = load_library().flce_create(ctypes.byref(cfg), ctypes.byref(h))
    if st != 0:
        raise FlceError(st, "flce_create")
    return h.value


def flce_destroy(handle: int) -> int:
    return load_library().flce_destroy(handle)


def flce_forward_backward(handle, x, W, targets, N, H, V, chunk, loss, dx, dW, stream) -> int:
    return load_library().flce_forward_backward(handle, x, W, targets, N, H, V, chunk, loss, dx, dW, stream)


def flce_forward_backward_ex(handle, x, W, targets, N, H, V, chunk, loss, dx, dW, lse, stream) -> int:
    return load_library().flce_forward_backward_ex(handle, x, W, targets, N, H, V, chunk, loss, dx, dW,
                                                   lse, stream)


def flce_forward_backward_opt(handle, x, W, targets, N, H, V, chunk, opt, loss, dx, dW, lse, stream) -> int:
    """opt: an Options instance or None (defaults)."""
    return load_library().flce_forward_backward_opt(handle, x, W, targets, N, H, V, chunk,
                                                    ctypes.byref(opt) if opt is not None else None,
                                                    loss, dx, dW, lse, stream)


def flce_forward_backward_noalloc(handle, x, W, targets, N, H, V, chunk, loss, dx, dW, stream) -> int:
    return load_library().flce_forward_backward_noalloc(handle, x, W, targets, N, H, V, chunk, loss, dx, dW,
                                                        stream)


def flce_effective_chunk(N, H, V, chunk) -> int:
    return load_library().flce_effective_chunk(N, H, V, chunk)


def flce_workspace_bytes(handle, N, H, V, chunk) -> int:
    return load_library().flce_workspace_bytes(handle, N, H, V, chunk)


def flce_workspace_bytes_opt(handle, N, H, V, chunk, opt) -> int:
    return load_library().flce_workspace_bytes_opt(handle, N, H, V, chunk,
                                                   ctypes.byref(opt) if opt is not None else None)


def flce_rmsnorm_forward_backward(handle, hidden, gamma, eps, W, targets, N, H, V, chunk, opt, loss, dhidden,
                                  dgamma, dW, lse, stream) -> int:
    return load_library().flce_rmsnorm_forward_backward(handle, hidden, gamma, float(eps), W, targets, N, H, V,
                                                        chunk, ctypes.byref(opt) if opt is not None else None,
                                                        loss, dhidden, dgamma, dW, lse, stream)


def flce_rmsnorm_workspace_bytes(handle, N, H, V, chunk, opt) -> int:
    return load_library().flce_rmsnorm_workspace_bytes(handle, N, H, V, chunk,
                                                       ctypes.byref(opt) if opt is not None else None)


def flce_reserve(handle, N, H, V, chunk) -> int:
    return load_library().flce_reserve(handle, N, H, V, chunk)


def flce_check(handle, stream) -> int:
    return load_library().flce_check(handle, stream)


def flce_profile_enable(handle, enable) -> int:
    return load_library().flce_profile_enable(handle, int(enable))


def flce_profile_read(handle):
    """Returns (status, {kernel name: dict(launches, total_ms, flops, bytes, sclk_mhz)})."""
    arr = (KernelStat * 16)()
    n = ctypes.c_int()
    st = load_library().flce_profile_read(handle, arr, 16, ctypes.byref(n))
    out = {}
    for i in range(min(n.value, 16)):
        k = arr[i]
        out[k.name.decode()] = {"launches": k.launches, "total_ms": k.total_ms, "flops": k.flops,
                                "bytes": k.bytes, "sclk_mhz": k.sclk_mhz}
    return st, out


# ---- torch convenience wrapper -----------------------------------------------

def _dt_code(dtype) -> int:
    import torch
    if dtype == torch.bfloat16:
        return FLCE_BF16
    if dtype == torch.float32:
        return FLCE_FP32
    raise ValueError(f"unsupported dtype {dtype}")


def _check_tensors(handle_device: int, specs):
    """Raises ValueError unless every given tensor is a contiguous tensor on the handle's device
    with the expected shape and dtype.  The C ABI takes plain pointers and cannot see either, so
    an output of the wrong size or dtype would otherwise be written past its end.
    specs: (name, tensor or None, shape, dtype); None tensors are skipped."""
    for name, ten, shape, dtype in specs:
        if ten is None:
            continue
        if not ten.is_cuda or ten.device.index != handle_device:
            raise ValueError(f"{name} must be on cuda:{handle_device}, not {ten.device}")
        if tuple(ten.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(ten.shape)}, expected {tuple(shape)}")
        if ten.dtype != dtype:
            raise ValueError(f"{name} has dtype {ten.dtype}, expected {dtype}")
        if not ten.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


class FusedLinearCrossEntropy:
    """Owns one library handle; takes torch device tensors.

    ``forward_backward(x, W, t)`` returns ``(loss, dx, dW)`` (and ``lse`` if
    asked): loss is a 0-d fp32 device tensor, dx/dW have the configured dtypes.
    Work is enqueued on torch's current stream of the tensors' device.
    """

    def __init__(self, in_dtype=None, dx_dtype=None, dw_dtype=None, device: int = 0,
                 variant: int = FLCE_CHUNKED, workspace_limit: int = 0):
        import torch
        in_dtype = in_dtype or torch.bfloat16
        self.in_dtype = in_dtype
        self.dx_dtype = dx_dtype or in_dtype
        self.dw_dtype = dw_dtype or in_dtype
        self.device = device
        cfg = Config(_dt_code(in_dtype), _dt_code(self.dx_dtype), _dt_code(self.dw_dtype), variant,
                     device, 0, workspace_limit)
        self.handle = flce_create(cfg)

    def close(self):
        if getattr(self, "handle", None):
            flce_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_bytes(self, N, H, V, chunk=0, forward_only: bool = False) -> int:
        if forward_only:
            return flce_workspace_bytes_opt(self.handle, N, H, V, chunk, _options("mean", None, FLCE_FORWARD_ONLY))
        return flce_workspace_bytes(self.handle, N, H, V, chunk)

    def reserve(self, N, H, V, chunk=0):
        st = flce_reserve(self.handle, N, H, V, chunk)
        if st != 0:
            raise FlceError(st, "flce_reserve")

    def profile_enable(self, enable: bool = True):
        st = flce_profile_enable(self.handle, enable)
        if st != 0:
            raise FlceError(st, "flce_profile_enable")

    def profile_read(self):
        st, out = flce_profile_read(self.handle)
        if st != 0:
            raise FlceError(st, "flce_profile_read")
        return out

    def check(self, stream=None) -> int:
        import torch
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        return flce_check(self.handle, s.cuda_stream)

    def forward_backward(self, x, W, t, chunk: int = 0, with_lse: bool = False, out=None, stream=None,
                         reduction: str = "mean", ignore_index: Optional[int] = None,
                         accumulate: bool = False):
        """Loss and both gradients.  ``reduction`` is "mean" (over tokens whose target is not
        ``ignore_index``) or "sum"; with ``accumulate`` the gradients are added into the ``dx``
        and ``dW`` of ``out`` instead of overwriting them."""
        import torch
        N, H = x.shape
        V = W.shape[0]
        if out is None:
            if accumulate:
                raise ValueError("accumulate needs the dx and dW to add into (out=...)")
            loss = torch.empty((), dtype=torch.float32, device=x.device)
            dx = torch.empty((N, H), dtype=self.dx_dtype, device=x.device)
            dW = torch.empty((V, H), dtype=self.dw_dtype, device=x.device)
            lse = torch.empty((N,), dtype=torch.float32, device=x.device) if with_lse else None
        else:
            loss, dx, dW, lse = out
        if dx is None or dW is None:
            raise ValueError("forward_backward needs dx and dW outputs (forward() computes the loss only)")
        _check_tensors(self.device, (("x", x, (N, H), self.in_dtype), ("W", W, (V, H), self.in_dtype),
                                     ("targets", t, (N,), torch.int64), ("loss", loss, (), torch.float32),
                                     ("dx", dx, (N, H), self.dx_dtype), ("dW", dW, (V, H), self.dw_dtype),
                                     ("lse", lse, (N,), torch.float32)))
        s = stream if stream is not None else torch.cuda.current_stream(x.device)
        opt = _options(reduction, ignore_index, FLCE_ACCUMULATE if accumulate else 0)
        st = flce_forward_backward_opt(self.handle, x.data_ptr(), W.data_ptr(), t.data_ptr(), N, H, V,
                                       chunk, opt, loss.data_ptr(), dx.data_ptr(), dW.data_ptr(),
                                       lse.data_ptr() if lse is not None else None, s.cuda_stream)
        if st != 0:
            raise FlceError(st, "flce_forward_backward")
        return (loss, dx, dW, lse) if with_lse else (loss, dx, dW)

    def forward(self, x, W, t, chunk: int = 0, with_lse: bool = False, stream=None,
                reduction: str = "mean", ignore_index: Optional[int] = None):
        """Loss only (and the per-token log-sum-exp if asked); no gradient is computed."""
        import torch
        N, H = x.shape
        V = W.shape[0]
        _check_tensors(self.device, (("x", x, (N, H), self.in_dtype), ("W", W, (V, H), self.in_dtype),
                                     ("targets", t, (N,), torch.int64)))
        loss = torch.empty((), dtype=torch.float32, device=x.device)
        lse = torch.empty((N,), dtype=torch.float32, device=x.device) if with_lse else None
        s = stream if stream is not None else torch.cuda.current_stream(x.device)
        opt = _options(reduction, ignore_index, FLCE_FORWARD_ONLY)
        st = flce_forward_backward_opt(self.handle, x.data_ptr(), W.data_ptr(), t.data_ptr(), N, H, V,
                                       chunk, opt, loss.data_ptr(), None, None,
                                       lse.data_ptr() if lse is not None else None, s.cuda_stream)
        if st != 0:
            raise FlceError(st, "flce_forward_backward_opt")
        return (loss, lse) if with_lse else loss


def _rmsnorm_call(self, hidden, gamma, W, t, eps, chunk, with_lse, out, stream, reduction, ignore_index,
                  flags):
    import torch
    N, H = hidden.shape
    V = W.shape[0]
    grads = not (flags & FLCE_FORWARD_ONLY)
    if out is None:
        if flags & FLCE_ACCUMULATE:
            raise ValueError("accumulate needs the dhidden, dgamma and dW to add into (out=...)")
        loss = torch.empty((), dtype=torch.float32, device=hidden.device)
        dh = torch.empty((N, H), dtype=self.dx_dtype, device=hidden.device) if grads else None
        dg = torch.empty((H,), dtype=self.dw_dtype, device=hidden.device) if grads else None
        dW = torch.empty((V, H), dtype=self.dw_dtype, device=hidden.device) if grads else None
        lse = torch.empty((N,), dtype=torch.float32, device=hidden.device) if with_lse else None
    else:
        loss, dh, dg, dW, lse = out
    if grads and (dh is None or dg is None or dW is None):
        raise ValueError("the backward needs dhidden, dgamma and dW outputs")
    _check_tensors(self.device, (("hidden", hidden, (N, H), self.in_dtype), ("gamma", gamma, (H,), self.in_dtype),
                                 ("W", W, (V, H), self.in_dtype), ("targets", t, (N,), torch.int64),
                                 ("loss", loss, (), torch.float32), ("dhidden", dh, (N, H), self.dx_dtype),
                                 ("dgamma", dg, (H,), self.dw_dtype), ("dW", dW, (V, H), self.dw_dtype),
                                 ("lse", lse, (N,), torch.float32)))
    s = stream if stream is not None else torch.cuda.current_stream(hidden.device)
    ptr = (lambda ten: ten.data_ptr() if ten is not None else None)
    st = flce_rmsnorm_forward_backward(self.handle, hidden.data_ptr(), gamma.data_ptr(), eps, W.data_ptr(),
                                       t.data_ptr(), N, H, V, chunk, _options(reduction, ignore_index, flags),
                                       loss.data_ptr(), ptr(dh), ptr(dg), ptr(dW), ptr(lse), s.cuda_stream)
    if st != 0:
        raise FlceError(st, "flce_rmsnorm_forward_backward")
    return loss, dh, dg, dW, lse


def _rmsnorm_forward_backward(self, hidden, gamma, W, t, eps: float = 1e-6, chunk: int = 0, with_lse: bool = False,
                              out=None, stream=None, reduction: str = "mean", ignore_index: Optional[int] = None,
                              accumulate: bool = False):
    """RMSNorm (x = hidden / RMS(hidden) * gamma) in front of the head, then the loss; returns
    ``(loss, dhidden, dgamma, dW)`` (and ``lse`` if asked).  ``out`` = (loss, dhidden, dgamma, dW, lse)."""
    loss, dh, dg, dW, lse = _rmsnorm_call(self, hidden, gamma, W, t, eps, chunk, with_lse, out, stream, reduction,
                                          ignore_index, FLCE_ACCUMULATE if accumulate else 0)
    return (loss, dh, dg, dW, lse) if with_lse else (loss, dh, dg, dW)


def _rmsnorm_forward(self, hidden, gamma, W, t, eps: float = 1e-6, chunk: int = 0, with_lse: bool = False,
                     stream=None, reduction: str = "mean", ignore_index: Optional[int] = None):
    """Loss only (and lse if asked) of RMSNorm + head."""
    loss, _, _, _, lse = _rmsnorm_call(self, hidden, gamma, W, t, eps, chunk, with_lse, None, stream, reduction,
                                       ignore_index, FLCE_FORWARD_ONLY)
    return (loss, lse) if with_lse else loss


FusedLinearCrossEntropy.rmsnorm_forward_backward = _rmsnorm_forward_backward
FusedLinearCrossEntropy.rmsnorm_forward = _rmsnorm_forward


def _options(reduction: str, ignore_index: Optional[int], flags: int) -> Options:
    if reduction not in ("mean", "sum"):
        raise ValueError(f"reduction must be 'mean' or 'sum', not {reduction!r}")
    return Options(FLCE_SUM if reduction == "sum" else FLCE_MEAN, flags, 0 if ignore_index is None else 1, 0,
                   0 if ignore_index is None else int(ignore_index))
