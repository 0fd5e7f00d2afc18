"""Plain, slow, float64 CPU oracle for fused linear + cross-entropy (FLCE).

Test infrastructure only: imported by ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg, never by the product path.  It shares no code
with the HIP library (no kernels, headers, helpers or constants).

What it computes (the plain definition; the fused GPU method reaches the same
result up to rounding order):

* "Fused linear + cross-entropy" (KernelIndex operation page), description and
  Semantics table: an LM-head projection of ``x`` float [tokens, hidden] through
  ``weight`` float [vocab, hidden], fused with cross-entropy against ``target``
  int64 [tokens], giving ``loss`` float [1].
* "[example] fused_linear_cross_entropy kernel" (pytorch/helion PR #1268), PR
  description: the forward yields the per-token log-sum-exp and the target
  logit, and keeps the log-sum-exp for the backward; the backward recomputes the
  logits and accumulates grad_input and grad_weight.
* "feat(FLCE): add helion version of fused linear cross entropy"
  (linkedin/Liger-Kernel PR #928), test log: the reductions are ``sum`` and
  ``mean``.

Readings taken where the pages are silent (each is restated in the design notes):

* mean divides by the token count N; there is no ignore_index, label smoothing,
  z-loss, soft-capping or bias (none appears on the pages);
* ``grad_loss`` is the scalar upstream gradient of ``loss``; it enters only
  through the per-token scale ``s = grad_loss / N`` (mean) or ``grad_loss``
  (sum);
* targets outside ``[0, V)`` are a caller error: the oracle raises.

All arithmetic is float64 on inputs widened exactly from their stored dtype.
The logits are materialised in token chunks (the oracle is allowed to be slow
and memory-hungry; the GPU path never materialises them).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "OracleError", "logits", "log_sum_exp", "dlogits", "scale_of", "forward",
    "backward", "forward_rows", "grad_x_rows", "grad_w_rows",
]

# Token rows per chunk: bounds the float64 logits block to CHUNK x V values.
_CHUNK_BYTES = 256 << 20


class OracleError(ValueError):
    """Raised on inputs that the definition does not cover (bad shape, target)."""


def _as_f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.float64:
        a = a.astype(np.float64)  # exact for float32 / bfloat16-widened values
    return a


def _check(x: np.ndarray, W: np.ndarray, target: np.ndarray, reduction: str):
    if x.ndim != 2 or W.ndim != 2 or x.shape[1] != W.shape[1]:
        raise OracleError(f"x {x.shape} and W {W.shape} must be [N,H] and [V,H]")
    N, V = x.shape[0], W.shape[0]
    if N == 0 or V == 0:
        raise OracleError("N and V must be positive")
    t = np.asarray(target)
    if t.shape != (N,) or not np.issubdtype(t.dtype, np.integer):
        raise OracleError(f"target must be an integer vector of length {N}")
    if t.min() < 0 or t.max() >= V:
        raise OracleError("target outside [0, V)")
    if reduction not in ("mean", "sum"):
        raise OracleError(f"reduction must be 'mean' or 'sum', got {reduction!r}")
    return t.astype(np.int64)


def _check_rows(x: np.ndarray, W: np.ndarray, target, idx, n_idx: int, what: str):
    """Shape and target checks of the per-row helpers (as ``_check``, no reduction):
    targets outside [0, V) raise instead of wrapping around in numpy indexing."""
    if x.ndim != 2 or W.ndim != 2 or x.shape[1] != W.shape[1]:
        raise OracleError(f"x {x.shape} and W {W.shape} must be [N,H] and [V,H]")
    N, V = x.shape[0], W.shape[0]
    if N == 0 or V == 0:
        raise OracleError("N and V must be positive")
    t = np.asarray(target)
    if t.shape != (N,) or not np.issubdtype(t.dtype, np.integer):
        raise OracleError(f"target must be an integer vector of length {N}")
    if t.min() < 0 or t.max() >= V:
        raise OracleError("target outside [0, V)")
    idx = np.asarray(idx)
    if idx.ndim != 1 or not np.issubdtype(idx.dtype, np.integer):
        raise OracleError(f"{what} must be an integer vector")
    if idx.size and (idx.min() < 0 or idx.max() >= n_idx):
        raise OracleError(f"{what} outside [0, {n_idx})")
    return t.astype(np.int64), idx.astype(np.int64)


def _chunk_rows(V: int) -> int:
    return max(1, _CHUNK_BYTES // (8 * max(V, 1)))


def scale_of(reduction: str, N: int, grad_loss: float = 1.0) -> float:
    """Per-token gradient scale s: d loss / d l_i times grad_loss."""
    return float(grad_loss) / N if reduction == "mean" else float(grad_loss)


def logits(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """z = x . W^T, one row per token, one column per vocabulary entry."""
    return x @ W.T


def log_sum_exp(z: np.ndarray) -> np.ndarray:
    """Row-wise log(sum_v exp(z_v)), evaluated stably about the row maximum."""
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


def dlogits(z: np.ndarray, lse: np.ndarray, target: np.ndarray, s: float) -> np.ndarray:
    """d loss / d z = s * (softmax(z) - onehot(target)), row-wise."""
    p = np.exp(z - lse[:, None])
    p[np.arange(z.shape[0]), target] -= 1.0
    return s * p


def forward(x, W, target, reduction: str = "mean"):
    """Return (loss, lse[N], target_logit[N]) in float64.

    loss_i = lse_i - z[i, t_i]; loss = sum_i loss_i, or its mean over N tokens.
    """
    x, W = _as_f64(x), _as_f64(W)
    t = _check(x, W, target, reduction)
    N = x.shape[0]
    lse = np.empty(N)
    zt = np.empty(N)
    step = _chunk_rows(W.shape[0])
    for a in range(0, N, step):
        b = min(N, a + step)
        z = logits(x[a:b], W)
        lse[a:b] = log_sum_exp(z)
        zt[a:b] = z[np.arange(b - a), t[a:b]]
    per_token = lse - zt
    loss = per_token.sum() if reduction == "sum" else per_token.sum() / N
    return float(loss), lse, zt


def backward(x, W, target, reduction: str = "mean", grad_loss: float = 1.0):
    """Return (grad_x [N,H], grad_W [V,H]) in float64.

    D = s * (softmax(z) - onehot(t)); grad_x = D . W; grad_W = D^T . x.
    """
    x, W = _as_f64(x), _as_f64(W)
    t = _check(x, W, target, reduction)
    N = x.shape[0]
    s = scale_of(reduction, N, grad_loss)
    gx = np.empty_like(x)
    gW = np.zeros_like(W)
    step = _chunk_rows(W.shape[0])
    for a in range(0, N, step):
        b = min(N, a + step)
        z = logits(x[a:b], W)
        D = dlogits(z, log_sum_exp(z), t[a:b], s)
        gx[a:b] = D @ W
        gW += D.T @ x[a:b]
    return gx, gW


def forward_rows(x, W, target, rows):
    """(lse, target_logit) for the selected token rows only."""
    x, W = _as_f64(x), _as_f64(W)
    t, rows = _check_rows(x, W, target, rows, x.shape[0], "rows")
    z = logits(x[rows], W)
    return log_sum_exp(z), z[np.arange(len(rows)), t[rows]]


def grad_x_rows(x, W, target, rows, reduction: str = "mean", grad_loss: float = 1.0):
    """grad_x for the selected token rows; each row needs only its own logits."""
    x, W = _as_f64(x), _as_f64(W)
    t, rows = _check_rows(x, W, target, rows, x.shape[0], "rows")
    if reduction not in ("mean", "sum"):
        raise OracleError(f"reduction must be 'mean' or 'sum', got {reduction!r}")
    s = scale_of(reduction, x.shape[0], grad_loss)
    z = logits(x[rows], W)
    return dlogits(z, log_sum_exp(z), t[rows], s) @ W


def grad_w_rows(x, W, target, vrows, lse, reduction: str = "mean", grad_loss: float = 1.0):
    """grad_W for the selected vocabulary rows, given the oracle's own lse[N].

    grad_W[v] = s * sum_i (exp(z_iv - lse_i) - [t_i == v]) x_i.
    """
    x, W = _as_f64(x), _as_f64(W)
    t, vrows = _check_rows(x, W, target, vrows, W.shape[0], "vrows")
    if reduction not in ("mean", "sum"):
        raise OracleError(f"reduction must be 'mean' or 'sum', got {reduction!r}")
    if np.shape(lse) != (x.shape[0],):
        raise OracleError(f"lse must have one value per token ({x.shape[0]})")
    s = scale_of(reduction, x.shape[0], grad_loss)
    zc = x @ W[vrows].T                      # [N, len(vrows)]
    P = np.exp(zc - np.asarray(lse, dtype=np.float64)[:, None])
    P -= (t[:, None] == vrows[None, :])
    return s * (P.T @ x)
