"""CPU oracle for fused linear + cross-entropy.  Test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, calls or links anything here, and this package
imports nothing from the product path.
"""
from .flce_oracle import (  # noqa: F401
    OracleError,
    logits,
    log_sum_exp,
    dlogits,
    forward,
    backward,
    forward_rows,
    grad_x_rows,
    grad_w_rows,
    scale_of,
)
