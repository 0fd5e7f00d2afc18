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


def test_row_helpers_validate_targets_and_indices():
    """forward_rows, grad_x_rows and grad_w_rows raise on out-of-range targets,
    row indices and reductions, as forward and backward do (a negative target must
    not wrap around to the last vocabulary column)."""
    g = np.random.Generator(np.random.PCG64(13))
    x = g.standard_normal((4, 3)); W = g.standard_normal((5, 3))
    rows = np.array([0, 2])
    lse = np.zeros(4)
    for bad_t in ([0, 1, -1, 2], [0, 5, 1, 2]):
        t = np.array(bad_t)
        with pytest.raises(oracle.OracleError):
            oracle.forward_rows(x, W, t, rows)
        with pytest.raises(oracle.OracleError):
            oracle.grad_x_rows(x, W, t, rows, "mean")
        with pytest.raises(oracle.OracleError):
            oracle.grad_w_rows(x, W, t, rows, lse, "mean")
    t = np.array([0, 1, 4, 2])
    for bad_rows in ([0, 4], [-1]):
        with pytest.raises(oracle.OracleError):
            oracle.forward_rows(x, W, t, np.array(bad_rows))
    with pytest.raises(oracle.OracleError):
        oracle.grad_w_rows(x, W, t, np.array([5]), lse, "mean")
    with pytest.raises(oracle.OracleError):
        oracle.grad_x_rows(x, W, t, rows, "max")
    # valid arguments still agree with the full oracle
    _, flse, fzt = oracle.forward(x, W, t, "sum")
    rl, rz = oracle.forward_rows(x, W, t, rows)
    np.testing.assert_allclose(rl, flse[rows], rtol=1e-14)
    np.testing.assert_array_equal(rz, fzt[rows])


def test_fp32_gradient_bar_rejects_zero_gradient():
    """The fp32 gradient bar of the GPU parity tests must be able to fail under
    mean reduction.  On the config-3-like workload (N=2048, H=4096, V=32000, fp32,
    seed 0) the oracle's grad_x entries lie below the 1e-4 absolute floor of the
    elementwise form, so an all-zero grad_x passes that form alone; the normalised
    form (max|d| / max|ref| <= 1e-4) rejects it, while a result within fp32
    rounding of the reference passes."""
    from lm_head_linear_tiled_amd.inputs import WORKLOADS, make_inputs, widen
    from tests.gpu_util import TOL, assert_grad_close
    w = WORKLOADS["llama2_f32"]
    x, W, t = make_inputs(w.N, w.H, w.V, w.dtype, seed=0)
    rows = np.arange(0, w.N, w.N // 32)
    ref = oracle.grad_x_rows(widen(x, w.dtype), widen(W, w.dtype), t, rows, "mean")
    tol = TOL["f32"]
    zero = np.zeros_like(ref)
    # the elementwise form alone cannot see the difference ...
    assert np.all(np.abs(zero - ref) <= tol["g_atol"] + tol["g_rtol"] * np.abs(ref))
    # ... the full bar does
    with pytest.raises(AssertionError):
        assert_grad_close(zero, ref, "f32", "grad_x")
    with pytest.raises(AssertionError):
        assert_grad_close(0.5 * ref, ref, "f32", "grad_x")
    g = np.random.Generator(np.random.PCG64(14))
    near = ref * (1 + 2.0 ** -22 * g.standard_normal(ref.shape))
    assert_grad_close(near, ref, "f32", "grad_x")
