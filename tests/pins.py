"""Checks that pin the CPU oracle to facts other than itself.

Each check takes the oracle module as an argument so that the mutation test can
run the same checks against deliberately broken copies of the oracle and show
that every planted mistake is caught.
"""
import math

import numpy as np

RTOL = 1e-10


def _rand(N, H, V, seed, w_std=None):
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal((N, H))
    W = g.standard_normal((V, H)) * (1.0 / math.sqrt(H) if w_std is None else w_std)
    t = g.integers(0, V, size=N)
    return x, W, t


def check_w_zero(orc):
    """W = 0: every logit is 0, so lse = ln V, loss = ln V (mean) or N ln V (sum),
    grad_x = 0 exactly, and grad_W[v] = s((1/V) sum_i x_i - sum_{i: t_i = v} x_i)."""
    N, H, V = 7, 5, 11
    x, _, t = _rand(N, H, V, 1)
    t[:3] = 4  # a repeated target
    W = np.zeros((V, H))
    for red, s in (("mean", 0.75 / N), ("sum", 0.75)):
        loss, lse, zt = orc.forward(x, W, t, red)
        np.testing.assert_allclose(lse, math.log(V), rtol=1e-14)
        np.testing.assert_array_equal(zt, 0.0)
        want = math.log(V) if red == "mean" else N * math.log(V)
        assert abs(loss - want) <= 1e-13 * want
        gx, gW = orc.backward(x, W, t, red, grad_loss=0.75)
        np.testing.assert_array_equal(gx, 0.0)
        exp_gW = np.tile(s * x.sum(axis=0) / V, (V, 1))
        for i in range(N):
            exp_gW[t[i]] -= s * x[i]
        np.testing.assert_allclose(gW, exp_gW, rtol=1e-12, atol=1e-14)


def check_all_targets_equal_w_zero(orc):
    """W = 0 and every target = c: grad_W[c] = -s (1 - 1/V) sum_i x_i, others s/V sum_i x_i."""
    N, H, V, c = 9, 4, 6, 2
    x, _, _ = _rand(N, H, V, 2)
    t = np.full(N, c)
    W = np.zeros((V, H))
    s = 1.0 / N
    _, gW = orc.backward(x, W, t, "mean")
    sx = x.sum(axis=0)
    for v in range(V):
        want = -s * (1 - 1 / V) * sx if v == c else s / V * sx
        np.testing.assert_allclose(gW[v], want, rtol=1e-12, atol=1e-15)


def check_identical_rows(orc):
    """All W rows equal: every logit of a token is the same, so l_i = ln V and grad_x = 0."""
    N, H, V = 5, 6, 13
    x, W, t = _rand(N, H, V, 3)
    W[:] = W[0]
    loss, lse, zt = orc.forward(x, W, t, "sum")
    np.testing.assert_allclose(lse - zt, math.log(V), rtol=1e-12)
    assert abs(loss - N * math.log(V)) <= 1e-12 * N * math.log(V)
    gx, _ = orc.backward(x, W, t, "sum")
    assert np.abs(gx).max() <= 1e-13


def check_invariants(orc):
    """Any input: dlogit rows sum to 0 so sum_v grad_W[v, :] = 0; sum = N * mean;
    gradients are linear in grad_loss; permuting tokens permutes grad_x rows and
    leaves loss and grad_W unchanged."""
    N, H, V = 12, 8, 30
    x, W, t = _rand(N, H, V, 4, w_std=0.7)
    lm, _, _ = orc.forward(x, W, t, "mean")
    ls, _, _ = orc.forward(x, W, t, "sum")
    assert abs(ls - N * lm) <= RTOL * abs(ls)
    gxm, gWm = orc.backward(x, W, t, "mean")
    gxs, gWs = orc.backward(x, W, t, "sum")
    np.testing.assert_allclose(gxs, N * gxm, rtol=RTOL, atol=1e-14)
    np.testing.assert_allclose(gWs, N * gWm, rtol=RTOL, atol=1e-14)
    assert np.abs(gWs.sum(axis=0)).max() <= 1e-12 * np.abs(gWs).max()
    gx3, gW3 = orc.backward(x, W, t, "sum", grad_loss=-2.5)
    np.testing.assert_allclose(gx3, -2.5 * gxs, rtol=RTOL, atol=1e-14)
    np.testing.assert_allclose(gW3, -2.5 * gWs, rtol=RTOL, atol=1e-14)
    perm = np.random.Generator(np.random.PCG64(5)).permutation(N)
    lp, _, _ = orc.forward(x[perm], W, t[perm], "sum")
    assert abs(lp - ls) <= RTOL * abs(ls)
    gxp, gWp = orc.backward(x[perm], W, t[perm], "sum")
    np.testing.assert_allclose(gxp, gxs[perm], rtol=RTOL, atol=1e-14)
    np.testing.assert_allclose(gWp, gWs, rtol=RTOL, atol=1e-14)


def brute_force(x, W, t, reduction, grad_loss=1.0):
    """Pure-Python FLCE with math.fsum: the textbook softmax cross-entropy, element by element."""
    N, H, V = len(x), len(x[0]), len(W)
    z = [[math.fsum(x[i][h] * W[v][h] for h in range(H)) for v in range(V)] for i in range(N)]
    per = []
    P = []
    for i in range(N):
        m = max(z[i])
        e = [math.exp(zv - m) for zv in z[i]]
        se = math.fsum(e)
        per.append(m + math.log(se) - z[i][t[i]])
        P.append([ev / se for ev in e])
    loss = math.fsum(per) / (N if reduction == "mean" else 1)
    s = grad_loss / N if reduction == "mean" else grad_loss
    D = [[s * (P[i][v] - (1.0 if v == t[i] else 0.0)) for v in range(V)] for i in range(N)]
    gx = [[math.fsum(D[i][v] * W[v][h] for v in range(V)) for h in range(H)] for i in range(N)]
    gW = [[math.fsum(D[i][v] * x[i][h] for i in range(N)) for h in range(H)] for v in range(V)]
    return loss, gx, gW


def check_brute_force(orc):
    """The numpy oracle equals a pure-Python fsum implementation at N=4, H=8, V=16."""
    x, W, t = _rand(4, 8, 16, 6, w_std=0.9)
    for red in ("mean", "sum"):
        loss, _, _ = orc.forward(x, W, t, red)
        gx, gW = orc.backward(x, W, t, red, grad_loss=1.3)
        bl, bgx, bgW = brute_force(x.tolist(), W.tolist(), t.tolist(), red, grad_loss=1.3)
        assert abs(loss - bl) <= 1e-13 * abs(bl)
        np.testing.assert_allclose(gx, np.array(bgx), rtol=1e-11, atol=1e-15)
        np.testing.assert_allclose(gW, np.array(bgW), rtol=1e-11, atol=1e-15)


def check_finite_differences(orc):
    """Analytic gradients equal central differences of the oracle's own loss
    (N=4, H=8, V=16, both reductions), every element of x and W."""
    x, W, t = _rand(4, 8, 16, 7, w_std=0.8)
    eps = 1e-6
    for red in ("mean", "sum"):
        gx, gW = orc.backward(x, W, t, red)
        for arr, g in ((x, gx), (W, gW)):
            num = np.empty_like(arr)
            for idx in np.ndindex(arr.shape):
                old = arr[idx]
                arr[idx] = old + eps
                lp = orc.forward(x, W, t, red)[0]
                arr[idx] = old - eps
                lm = orc.forward(x, W, t, red)[0]
                arr[idx] = old
                num[idx] = (lp - lm) / (2 * eps)
            np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def check_torch_cross_entropy(orc):
    """Special case that reduces to a library routine: torch's float64 CPU
    cross_entropy of the materialised logits, with autograd gradients."""
    import torch
    x, W, t = _rand(10, 16, 50, 8)
    for red in ("mean", "sum"):
        xt = torch.tensor(x, requires_grad=True)
        Wt = torch.tensor(W, requires_grad=True)
        ref = torch.nn.functional.cross_entropy(xt @ Wt.T, torch.tensor(t), reduction=red)
        ref.backward(torch.tensor(0.6, dtype=torch.float64))
        loss, _, _ = orc.forward(x, W, t, red)
        gx, gW = orc.backward(x, W, t, red, grad_loss=0.6)
        assert abs(loss - ref.item()) <= 1e-12 * abs(ref.item())
        np.testing.assert_allclose(gx, xt.grad.numpy(), rtol=1e-10, atol=1e-15)
        np.testing.assert_allclose(gW, Wt.grad.numpy(), rtol=1e-10, atol=1e-15)


def check_extreme_logits(orc):
    """Logits of magnitude ~1e3 stay finite (max subtraction); the softmax is then
    one-hot at the row maximum, so l_i = max_v z_iv - z_{i,t_i} to double rounding."""
    x, W, t = _rand(6, 8, 20, 9, w_std=300.0)
    loss, lse, zt = orc.forward(x, W, t, "sum")
    z = x @ W.T
    assert np.isfinite(loss) and np.all(np.isfinite(lse))
    assert np.abs(z).max() > 500
    gaps = np.sort(z, axis=1)
    assert np.all(gaps[:, -1] - gaps[:, -2] > 50)  # a clear winner per row
    np.testing.assert_allclose(lse - zt, z.max(axis=1) - z[np.arange(6), t], rtol=1e-12, atol=1e-9)
    gx, gW = orc.backward(x, W, t, "sum")
    assert np.all(np.isfinite(gx)) and np.all(np.isfinite(gW))


def check_row_helpers(orc):
    """The per-row helpers used at full size agree with the full oracle."""
    x, W, t = _rand(9, 6, 25, 10, w_std=0.9)
    _, lse, zt = orc.forward(x, W, t, "mean")
    gx, gW = orc.backward(x, W, t, "mean", grad_loss=2.0)
    rows = np.array([0, 4, 8])
    l2, z2 = orc.forward_rows(x, W, t, rows)
    np.testing.assert_allclose(l2, lse[rows], rtol=1e-14)
    np.testing.assert_allclose(z2, zt[rows], rtol=1e-14)
    np.testing.assert_allclose(orc.grad_x_rows(x, W, t, rows, "mean", 2.0), gx[rows], rtol=1e-12, atol=1e-15)
    vr = np.array([0, 3, 24, t[2]])
    np.testing.assert_allclose(orc.grad_w_rows(x, W, t, vr, lse, "mean", 2.0), gW[vr], rtol=1e-12, atol=1e-15)


ALL_CHECKS = [
    check_w_zero, check_all_targets_equal_w_zero, check_identical_rows, check_invariants,
    check_brute_force, check_finite_differences, check_torch_cross_entropy,
    check_extreme_logits, check_row_helpers,
]
