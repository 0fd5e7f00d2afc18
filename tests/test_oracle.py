"""The CPU oracle against facts other than itself (closed forms, invariants,
brute force, finite differences, an independent library routine)."""
import numpy as np
import pytest

import oracle
from tests import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle)


def test_out_of_range_target_raises():
    x = np.zeros((2, 3)); W = np.zeros((4, 3))
    for bad in ([0, 4], [-1, 0]):
        with pytest.raises(oracle.OracleError):
            oracle.forward(x, W, np.array(bad), "mean")


def test_bad_reduction_and_shapes_raise():
    x = np.zeros((2, 3)); W = np.zeros((4, 3)); t = np.array([0, 1])
    with pytest.raises(oracle.OracleError):
        oracle.forward(x, W, t, "max")
    with pytest.raises(oracle.OracleError):
        oracle.forward(x, np.zeros((4, 2)), t, "mean")
    with pytest.raises(oracle.OracleError):
        oracle.forward(np.zeros((0, 3)), W, np.zeros(0, dtype=np.int64), "mean")


def test_v_equals_one():
    """V = 1: the single class has probability 1, so loss = 0 and all gradients vanish."""
    g = np.random.Generator(np.random.PCG64(11))
    x = g.standard_normal((5, 4)); W = g.standard_normal((1, 4)); t = np.zeros(5, dtype=np.int64)
    loss, lse, zt = oracle.forward(x, W, t, "sum")
    assert abs(loss) <= 1e-15 and np.array_equal(lse, zt)
    gx, gW = oracle.backward(x, W, t, "sum")
    assert np.abs(gx).max() == 0 and np.abs(gW).max() == 0


def test_chunking_is_invisible(monkeypatch):
    """Token chunking inside the oracle does not change its results."""
    import oracle.flce_oracle as fo
    g = np.random.Generator(np.random.PCG64(12))
    x = g.standard_normal((37, 6)); W = g.standard_normal((19, 6)) * 0.5
    t = g.integers(0, 19, size=37)
    ref = fo.forward(x, W, t, "sum"), fo.backward(x, W, t, "sum")
    monkeypatch.setattr(fo, "_CHUNK_BYTES", 8 * 19 * 5)  # 5 rows per chunk
    got = fo.forward(x, W, t, "sum"), fo.backward(x, W, t, "sum")
    assert abs(got[0][0] - ref[0][0]) <= 1e-12 * abs(ref[0][0])
    np.testing.assert_allclose(got[1][0], ref[1][0], rtol=1e-12)
    np.testing.assert_allclose(got[1][1], ref[1][1], rtol=1e-12, atol=1e-15)
