"""Python binding of libflce.so (include/flce.h): argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI; this
module checks tensor metadata, allocates outputs and workspace with torch (device
memory and the current stream are all torch supplies) and forwards raw pointers.
There is no fallback: if the library is missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflce.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "flce.h")

F32, BF16 = 0, 1
MEAN, SUM = 0, 1
_DT = {torch.float32: F32, torch.bfloat16: BF16}
_RED = {"mean": MEAN, "sum": SUM}
_ESIZE = {F32: 4, BF16: 2}

_lib = None

KERNEL_NAMES = ["fwd_partial", "fwd_combine", "fwd_loss", "bwd_dlogits", "bwd_grad_w", "bwd_grad_x", "fill",
                "bwd_gx_reduce", "bwd_atomic", "zero", "cast", "tail_fixup", "tail_pieces"]


class Timing(ctypes.Structure):
    """flce_timing: caller-created HIP events recorded between the library's kernels."""
    _fields_ = [("events", ctypes.POINTER(ctypes.c_void_p)), ("n_events", ctypes.c_int),
                ("kinds", ctypes.POINTER(ctypes.c_int)), ("n_launches", ctypes.c_int)]


_hip = None
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hip_runtime_api.h: hipEventDisableSystemFence


def _hip_runtime() -> ctypes.CDLL:
    """The HIP runtime torch has already loaded (libflce.so resolves to the same one)."""
    global _hip
    if _hip is None:
        torch.cuda.init()
        hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip = hip
    return _hip


class KernelTimer:
    """Per-kernel durations of one library call, from HIP events recorded between its
    kernels.  The events skip the system-scope fence that default events apply on
    every record (timing only; the caller's synchronize makes results visible).
    Measured on the headline step against no events: default events lengthened it by
    up to 1.3 % depending on the machine, these by at most run-to-run noise."""

    def __init__(self, n_events: int, device=None):
        hip = _hip_runtime()
        self.events = []
        for _ in range(n_events):
            ev = ctypes.c_void_p()
            code = hip.hipEventCreateWithFlags(ctypes.byref(ev), HIP_EVENT_DISABLE_SYSTEM_FENCE)
            if code != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed with HIP error {code}")
            self.events.append(ev.value)
        self._handles = (ctypes.c_void_p * n_events)(*self.events)
        self._kinds = (ctypes.c_int * max(1, n_events - 1))()
        self.t = Timing(self._handles, n_events, self._kinds, 0)

    def _elapsed(self, a, b) -> float:
        ms = ctypes.c_float()
        code = _hip_runtime().hipEventElapsedTime(ctypes.byref(ms), a, b)
        if code != 0:
            raise RuntimeError(f"hipEventElapsedTime failed with HIP error {code}")
        return ms.value

    def durations(self):
        """[(kernel name, ms)] for every launch that got an event (call after a sync)."""
        n = min(self.t.n_launches, len(self.events) - 1)
        return [(KERNEL_NAMES[self._kinds[k]], self._elapsed(self.events[k], self.events[k + 1])) for k in range(n)]

    def __del__(self):
        hip = _hip
        if hip is not None:
            for ev in getattr(self, "events", []):
                hip.hipEventDestroy(ev)


class FLCEError(RuntimeError):
    def __init__(self, code: int):
        self.code = code
        super().__init__(status_string(code))


def load() -> ctypes.CDLL:
    """Load libflce.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    i64, sz, vp, f32p = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p
    lib.flce_status_string.argtypes = [ctypes.c_int]
    lib.flce_status_string.restype = ctypes.c_char_p
    for name in ("flce_forward_workspace_bytes", "flce_backward_workspace_bytes",
                 "flce_backward_min_workspace_bytes", "flce_forward_backward_workspace_bytes"):
        fn = getattr(lib, name)
        fn.argtypes = [i64, i64, i64, ctypes.c_int]
        fn.restype = sz
    lib.flce_forward.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                 f32p, f32p, f32p, vp, sz, vp]
    lib.flce_forward.restype = ctypes.c_int
    lib.flce_backward.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                  vp, vp, vp, sz, vp]
    lib.flce_backward.restype = ctypes.c_int
    lib.flce_forward_backward.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int, vp,
                                          vp, vp, vp, vp, vp, sz, vp]
    lib.flce_forward_backward.restype = ctypes.c_int
    tp = ctypes.POINTER(Timing)
    lib.flce_forward_timed.argtypes = lib.flce_forward.argtypes + [tp]
    lib.flce_forward_timed.restype = ctypes.c_int
    lib.flce_backward_timed.argtypes = lib.flce_backward.argtypes + [tp]
    lib.flce_backward_timed.restype = ctypes.c_int
    lib.flce_backward_chunked_workspace_bytes.argtypes = [i64, i64, i64, ctypes.c_int, i64]
    lib.flce_backward_chunked_workspace_bytes.restype = sz
    lib.flce_backward_chunked.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int, i64,
                                          vp, vp, vp, sz, vp, tp]
    lib.flce_backward_chunked.restype = ctypes.c_int
    lib.flce_backward_atomic_workspace_bytes.argtypes = [i64, i64, i64, ctypes.c_int]
    lib.flce_backward_atomic_workspace_bytes.restype = sz
    lib.flce_backward_atomic.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                         vp, vp, vp, sz, vp, tp]
    lib.flce_backward_atomic.restype = ctypes.c_int
    lib.flce_forward_noalloc_max_tokens.argtypes = [i64]
    lib.flce_forward_noalloc_max_tokens.restype = i64
    lib.flce_forward_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int, f32p, f32p, f32p, vp]
    lib.flce_forward_noalloc.restype = ctypes.c_int
    _lib = lib
    return lib


def header_functions() -> list[str]:
    """Names of the functions include/flce.h declares."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(flce_\w+)\s*\(", text, re.M)))


def status_string(code: int) -> str:
    return load().flce_status_string(int(code)).decode()


def forward_workspace_bytes(N: int, H: int, V: int, dtype: torch.dtype) -> int:
    return int(load().flce_forward_workspace_bytes(N, H, V, _DT[dtype]))


def backward_workspace_bytes(N: int, H: int, V: int, dtype: torch.dtype) -> int:
    return int(load().flce_backward_workspace_bytes(N, H, V, _DT[dtype]))


def backward_min_workspace_bytes(N: int, H: int, V: int, dtype: torch.dtype) -> int:
    return int(load().flce_backward_min_workspace_bytes(N, H, V, _DT[dtype]))


def _check(x: torch.Tensor, W: torch.Tensor, target: torch.Tensor, reduction: str):
    if x.dtype not in _DT or W.dtype != x.dtype:
        raise TypeError(f"x and W must both be float32 or bfloat16, got {x.dtype}, {W.dtype}")
    if target.dtype != torch.int64:
        raise TypeError("target must be int64")
    if not (x.is_cuda and W.is_cuda and target.is_cuda) or not (x.device == W.device == target.device):
        raise ValueError("x, W and target must be on the same GPU")
    if x.dim() != 2 or W.dim() != 2 or x.shape[1] != W.shape[1] or target.shape != (x.shape[0],):
        raise ValueError(f"shapes x {tuple(x.shape)}, W {tuple(W.shape)}, target {tuple(target.shape)}")
    if not (x.is_contiguous() and W.is_contiguous() and target.is_contiguous()):
        raise ValueError("x, W and target must be contiguous")
    if reduction not in _RED:
        raise ValueError(f"reduction must be 'mean' or 'sum', got {reduction!r}")


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def flce_forward(x: torch.Tensor, W: torch.Tensor, target: torch.Tensor, reduction: str = "mean",
                 with_target_logit: bool = False, workspace: torch.Tensor | None = None,
                 timer: KernelTimer | None = None):
    """Return (loss [1] f32, lse [N] f32[, target_logit [N] f32])."""
    _check(x, W, target, reduction)
    lib = load()
    N, H = x.shape
    V = W.shape[0]
    dt = _DT[x.dtype]
    loss = torch.empty(1, dtype=torch.float32, device=x.device)
    lse = torch.empty(N, dtype=torch.float32, device=x.device)
    zt = torch.empty(N, dtype=torch.float32, device=x.device) if with_target_logit else None
    nws = lib.flce_forward_workspace_bytes(N, H, V, dt)
    ws = workspace if workspace is not None else torch.empty(nws, dtype=torch.uint8, device=x.device)
    args = (x.data_ptr(), W.data_ptr(), target.data_ptr(), N, H, V, dt, _RED[reduction],
            loss.data_ptr(), lse.data_ptr(), zt.data_ptr() if zt is not None else None,
            ws.data_ptr(), ws.numel(), _stream(x.device))
    code = lib.flce_forward(*args) if timer is None else lib.flce_forward_timed(*args, ctypes.byref(timer.t))
    if code != 0:
        raise FLCEError(code)
    return (loss, lse, zt) if with_target_logit else (loss, lse)


def flce_backward(x: torch.Tensor, W: torch.Tensor, target: torch.Tensor, lse: torch.Tensor,
                  grad_loss: torch.Tensor, reduction: str = "mean", workspace: torch.Tensor | None = None,
                  timer: KernelTimer | None = None):
    """Return (grad_x [N,H], grad_W [V,H]) in the dtype of x."""
    _check(x, W, target, reduction)
    if lse.dtype != torch.float32 or lse.shape != (x.shape[0],) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [N] tensor")
    grad_loss = grad_loss.reshape(1).to(device=x.device, dtype=torch.float32).contiguous()
    lib = load()
    N, H = x.shape
    V = W.shape[0]
    dt = _DT[x.dtype]
    gx = torch.empty_like(x)
    gW = torch.empty_like(W)
    nws = lib.flce_backward_workspace_bytes(N, H, V, dt)
    ws = workspace if workspace is not None else torch.empty(nws, dtype=torch.uint8, device=x.device)
    args = (x.data_ptr(), W.data_ptr(), target.data_ptr(), lse.data_ptr(),
            grad_loss.data_ptr(), N, H, V, dt, _RED[reduction], gx.data_ptr(),
            gW.data_ptr(), ws.data_ptr(), ws.numel(), _stream(x.device))
    code = lib.flce_backward(*args) if timer is None else lib.flce_backward_timed(*args, ctypes.byref(timer.t))
    if code != 0:
        raise FLCEError(code)
    return gx, gW


def backward_chunked_workspace_bytes(N: int, H: int, V: int, dtype: torch.dtype, chunk_tokens: int) -> int:
    return int(load().flce_backward_chunked_workspace_bytes(N, H, V, _DT[dtype], chunk_tokens))


def flce_backward_chunked(x: torch.Tensor, W: torch.Tensor, target: torch.Tensor, lse: torch.Tensor,
                          grad_loss: torch.Tensor, reduction: str = "mean", chunk_tokens: int = 1024,
                          workspace: torch.Tensor | None = None, timer: KernelTimer | None = None):
    """Token-chunked backward (each chunk's dlogits over the whole vocabulary), for
    comparison with flce_backward.  Return (grad_x [N,H], grad_W [V,H])."""
    _check(x, W, target, reduction)
    if lse.dtype != torch.float32 or lse.shape != (x.shape[0],) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [N] tensor")
    grad_loss = grad_loss.reshape(1).to(device=x.device, dtype=torch.float32).contiguous()
    lib = load()
    N, H = x.shape
    V = W.shape[0]
    dt = _DT[x.dtype]
    gx = torch.empty_like(x)
    gW = torch.empty_like(W)
    nws = lib.flce_backward_chunked_workspace_bytes(N, H, V, dt, chunk_tokens)
    ws = workspace if workspace is not None else torch.empty(max(nws, 1), dtype=torch.uint8, device=x.device)
    code = lib.flce_backward_chunked(x.data_ptr(), W.data_ptr(), target.data_ptr(), lse.data_ptr(),
                                     grad_loss.data_ptr(), N, H, V, dt, _RED[reduction], chunk_tokens,
                                     gx.data_ptr(), gW.data_ptr(), ws.data_ptr(), ws.numel(), _stream(x.device),
                                     ctypes.byref(timer.t) if timer is not None else None)
    if code != 0:
        raise FLCEError(code)
    return gx, gW


def backward_atomic_workspace_bytes(N: int, H: int, V: int, dtype: torch.dtype) -> int:
    return int(load().flce_backward_atomic_workspace_bytes(N, H, V, _DT[dtype]))


def flce_backward_atomic(x: torch.Tensor, W: torch.Tensor, target: torch.Tensor, lse: torch.Tensor,
                         grad_loss: torch.Tensor, reduction: str = "mean", workspace: torch.Tensor | None = None,
                         timer: KernelTimer | None = None):
    """Backward with float32 atomic accumulation of both gradients (one fused kernel
    per (token tile, vocabulary tile) pair), for comparison with flce_backward.
    Return (grad_x [N,H], grad_W [V,H])."""
    _check(x, W, target, reduction)
    if lse.dtype != torch.float32 or lse.shape != (x.shape[0],) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [N] tensor")
    grad_loss = grad_loss.reshape(1).to(device=x.device, dtype=torch.float32).contiguous()
    lib = load()
    N, H = x.shape
    V = W.shape[0]
    dt = _DT[x.dtype]
    gx = torch.empty_like(x)
    gW = torch.empty_like(W)
    nws = lib.flce_backward_atomic_workspace_bytes(N, H, V, dt)
    ws = workspace if workspace is not None else torch.empty(max(nws, 1), dtype=torch.uint8, device=x.device)
    code = lib.flce_backward_atomic(x.data_ptr(), W.data_ptr(), target.data_ptr(), lse.data_ptr(),
                                    grad_loss.data_ptr(), N, H, V, dt, _RED[reduction], gx.data_ptr(), gW.data_ptr(),
                                    ws.data_ptr(), ws.numel(), _stream(x.device),
                                    ctypes.byref(timer.t) if timer is not None else None)
    if code != 0:
        raise FLCEError(code)
    return gx, gW


def forward_backward_workspace_bytes(N: int, H: int, V: int, dtype: torch.dtype) -> int:
    return int(load().flce_forward_backward_workspace_bytes(N, H, V, _DT[dtype]))


def flce_forward_backward(x: torch.Tensor, W: torch.Tensor, target: torch.Tensor, reduction: str = "mean",
                          grad_loss: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Return (loss [1] f32, lse [N] f32, grad_x, grad_W) from one library call."""
    _check(x, W, target, reduction)
    lib = load()
    N, H = x.shape
    V = W.shape[0]
    dt = _DT[x.dtype]
    loss = torch.empty(1, dtype=torch.float32, device=x.device)
    lse = torch.empty(N, dtype=torch.float32, device=x.device)
    gx = torch.empty_like(x)
    gW = torch.empty_like(W)
    gl = None
    if grad_loss is not None:
        gl = grad_loss.reshape(1).to(device=x.device, dtype=torch.float32).contiguous()
    nws = lib.flce_forward_backward_workspace_bytes(N, H, V, dt)
    ws = workspace if workspace is not None else torch.empty(nws, dtype=torch.uint8, device=x.device)
    code = lib.flce_forward_backward(x.data_ptr(), W.data_ptr(), target.data_ptr(), N, H, V, dt, _RED[reduction],
                                     gl.data_ptr() if gl is not None else None, loss.data_ptr(), lse.data_ptr(),
                                     gx.data_ptr(), gW.data_ptr(), ws.data_ptr(), ws.numel(), _stream(x.device))
    if code != 0:
        raise FLCEError(code)
    return loss, lse, gx, gW


class FLCEFunction(torch.autograd.Function):
    """loss = CE(x . W^T, target) with the logits never materialised."""

    @staticmethod
    def forward(ctx, x, W, target, reduction="mean"):
        loss, lse = flce_forward(x, W, target, reduction)
        ctx.save_for_backward(x, W, target, lse)
        ctx.reduction = reduction
        return loss.reshape(())

    @staticmethod
    def backward(ctx, grad_loss):
        x, W, target, lse = ctx.saved_tensors
        gx, gW = flce_backward(x, W, target, lse, grad_loss, ctx.reduction)
        return gx, gW, None, None


def flce_loss(x: torch.Tensor, W: torch.Tensor, target: torch.Tensor, reduction: str = "mean") -> torch.Tensor:
    return FLCEFunction.apply(x, W, target, reduction)
