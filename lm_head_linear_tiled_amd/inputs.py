"""Seeded synthetic inputs for fused linear + cross-entropy.

This module is shared by the tests, the bench and the smoke check: it draws the
inputs that both the HIP path and the CPU oracle receive.  It holds none of the
method's arithmetic (no logits, softmax or gradients) and imports neither side.

Recipe (the workloads the pages measure, with synthetic values):

* ``x ~ N(0, 1)`` of shape [N, H], then ``W ~ N(0, std = 1/sqrt(H))`` of shape
  [V, H], then ``target ~ uniform int64 in [0, V)`` of shape [N], drawn in that
  order from one ``numpy`` PCG64 generator seeded with ``seed`` (0 by default);
* values are drawn in float32; for bfloat16 inputs each float32 is rounded to
  the nearest bfloat16 (ties to even) and the very same bits go to both sides.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "bf16_bits_from_f32", "f64_from_bf16_bits",
           "widen"]


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    H: int
    V: int
    dtype: str           # "f32" or "bf16"
    reductions: tuple    # reductions the workload is run with


# The five workloads, from the pages' shapes (see the design doc for the sources).
WORKLOADS = {
    "tiny": Workload("tiny", 64, 128, 1000, "f32", ("mean",)),
    "ragged": Workload("ragged", 3 * 423, 1000, 10000, "f32", ("sum", "mean")),
    "llama2_bf16": Workload("llama2_bf16", 2 * 1024, 4096, 32000, "bf16", ("mean",)),
    "llama2_f32": Workload("llama2_f32", 2 * 1024, 4096, 32000, "f32", ("mean",)),
    "llama2_4k": Workload("llama2_4k", 4096, 4096, 32000, "bf16", ("mean",)),
    "llama2_32k": Workload("llama2_32k", 32768, 4096, 32000, "bf16", ("mean",)),
    "llama3_4k": Workload("llama3_4k", 4096, 4096, 128256, "bf16", ("mean",)),
    "llama3_8k": Workload("llama3_8k", 8192, 4096, 128256, "bf16", ("mean",)),
    "llama3_16k": Workload("llama3_16k", 16384, 4096, 128256, "bf16", ("mean",)),
    "llama3_32k": Workload("llama3_32k", 32768, 4096, 128256, "bf16", ("mean",)),
    # the other heads the Liger-Kernel PR #928 thread benchmarks
    "qwen3_32k": Workload("qwen3_32k", 32768, 4096, 151936, "bf16", ("mean",)),
    "gemma3_8k": Workload("gemma3_8k", 8192, 2304, 262208, "bf16", ("mean",)),
}


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def f64_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits exactly to float64."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of an input array stored as ``dtype``."""
    return f64_from_bf16_bits(a) if dtype == "bf16" else np.asarray(a, dtype=np.float64)


def make_inputs(N: int, H: int, V: int, dtype: str = "f32", seed: int = 0,
                x_scale: float = 1.0, w_std: float | None = None):
    """Return (x, W, target) as host arrays in storage form.

    ``x`` and ``W`` are float32 arrays for ``dtype == "f32"`` and uint16 bfloat16
    bit arrays for ``dtype == "bf16"``; ``target`` is int64.
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError(dtype)
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal((N, H), dtype=np.float32)
    if x_scale != 1.0:
        x *= np.float32(x_scale)
    W = g.standard_normal((V, H), dtype=np.float32)
    W *= np.float32(1.0 / np.sqrt(H) if w_std is None else w_std)
    t = g.integers(0, V, size=N, dtype=np.int64)
    if dtype == "bf16":
        return bf16_bits_from_f32(x), bf16_bits_from_f32(W), t
    return x, W, t
