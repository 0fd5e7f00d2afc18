"""Work and traffic accounting for fused linear + cross-entropy (host-side arithmetic only).

* flops: the forward is one N x V x H contraction (2NHV); forward + backward is
  counted as 8NHV (forward, the backward's logit recompute, D . W and D^T . x).
* compulsory bytes: every declared tensor crosses HBM once, the accounting of the
  KernelIndex page's estimated DRAM floor ("Fused linear + cross-entropy",
  Estimated floor box): x, weight, target and loss for the forward.
"""
from __future__ import annotations

ESIZE = {"bf16": 2, "f32": 4}

# MI355X published peaks (dense, no sparsity).
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}
PEAK_HBM_GBPS = 8000.0


def fwd_flops(N: int, H: int, V: int) -> float:
    return 2.0 * N * H * V


def fwdbwd_flops(N: int, H: int, V: int) -> float:
    return 8.0 * N * H * V


def fwd_declared_bytes(N: int, H: int, V: int, dtype: str) -> int:
    """x + W + target (int64) + loss (one float32)."""
    e = ESIZE[dtype]
    return N * H * e + V * H * e + 8 * N + 4


def fwd_compulsory_bytes(N: int, H: int, V: int, dtype: str) -> int:
    """Forward HBM bytes of this library: declared tensors plus the lse [N] float32 it keeps."""
    return fwd_declared_bytes(N, H, V, dtype) + 4 * N


def fwdbwd_compulsory_bytes(N: int, H: int, V: int, dtype: str) -> int:
    """Forward bytes, then the backward reads x, W, target, lse and writes grad_x, grad_W."""
    e = ESIZE[dtype]
    bwd = N * H * e + V * H * e + 8 * N + 4 * N + N * H * e + V * H * e
    return fwd_compulsory_bytes(N, H, V, dtype) + bwd


def floor_us(nbytes: float, gbps: float) -> float:
    return nbytes / (gbps * 1e3)
