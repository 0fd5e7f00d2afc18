"""Plant plausible mistakes in the CPU oracle (on the CPU) and check that the pin
suite catches every one of them."""
import numpy as np
import pytest

import oracle.flce_oracle as fo
from tests import pins


def _wrong_sign_onehot(z, lse, target, s):
    p = np.exp(z - lse[:, None])
    p[np.arange(z.shape[0]), target] += 1.0
    return s * p


def _dropped_onehot(z, lse, target, s):
    return s * np.exp(z - lse[:, None])


def _unnormalised_softmax(z, lse, target, s):
    p = np.exp(z - z.max(axis=1)[:, None])
    p[np.arange(z.shape[0]), target] -= 1.0
    return s * p


def _lse_without_max(z):
    m = z.max(axis=1)
    return np.log(np.exp(z - m[:, None]).sum(axis=1))


def _lse_natural_overflow(z):
    with np.errstate(over="ignore"):
        return np.log(np.exp(z).sum(axis=1))


def _mean_over_vocab(reduction, N, grad_loss=1.0):
    return float(grad_loss) / (N + 1) if reduction == "mean" else float(grad_loss)


def _transposed_logits(x, W):
    # a transposed operand that still type-checks when the shapes happen to allow it
    return (x @ W.T)[:, ::-1]


def _grad_loss_ignored(reduction, N, grad_loss=1.0):
    return 1.0 / N if reduction == "mean" else 1.0


MUTANTS = {
    "onehot_sign": ("dlogits", _wrong_sign_onehot),
    "onehot_dropped": ("dlogits", _dropped_onehot),
    "softmax_unnormalised": ("dlogits", _unnormalised_softmax),
    "lse_missing_max": ("log_sum_exp", _lse_without_max),
    "lse_overflow": ("log_sum_exp", _lse_natural_overflow),
    "mean_wrong_divisor": ("scale_of", _mean_over_vocab),
    "logit_columns_permuted": ("logits", _transposed_logits),
    "grad_loss_ignored": ("scale_of", _grad_loss_ignored),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, bad = MUTANTS[name]
    monkeypatch.setattr(fo, attr, bad)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(fo)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(check.__name__)
    assert caught, f"mutant {name} passed every pin"
