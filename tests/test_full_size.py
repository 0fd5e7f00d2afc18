"""Parity at the full benchmark sizes, in the launch configuration bench.py times
(default workspaces), against the float64 oracle:

* the oracle's full forward (lse and target logit of every token, and the loss:
  2NHV float64 flop, up to 4e13 at 32768 tokens -- tens of seconds on a
  16-core host) against the GPU's lse, target logits and loss;
* grad_x rows of sampled tokens (each needs only that token's logits);
* grad_W rows of sampled vocabulary entries, always including the targets of
  sampled tokens and the first and last entry (each needs the oracle's lse of
  every token, which the full forward gives);
* at every size, the property sum_v grad_W[v, :] = 0 (every dlogit row sums to 0).
"""
import time

import numpy as np
import pytest
import torch

import oracle
from lm_head_linear_tiled_amd.inputs import WORKLOADS, make_inputs, widen
from tests.gpu_util import TOL, note, to_dev, to_f64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["llama3_4k", "llama2_4k", "llama2_32k", "llama3_8k", "llama3_16k",
                                  "llama3_32k", "qwen3_32k", "gemma3_8k"])
def test_full_size(gpu, name):
    w = WORKLOADS[name]
    N, H, V, dt = w.N, w.H, w.V, w.dtype
    note(f"[full] {name} N={N} H={H} V={V} {dt}")
    x, W, t = make_inputs(N, H, V, dt, seed=0)
    xd, Wd, td = to_dev(x, dt), to_dev(W, dt), torch.from_numpy(t).cuda()
    loss, lse, zt = gpu.flce_forward(xd, Wd, td, "mean", with_target_logit=True)
    gx, gW = gpu.flce_backward(xd, Wd, td, lse, torch.ones(1, device="cuda"), "mean")
    torch.cuda.synchronize()
    note(f"[full] {name} GPU done")
    tol = TOL[dt]
    gbar = tol["g_norm"]

    # property at any size: every dlogit row sums to zero, so do grad_W's columns.
    # What remains is rounding: D is rounded to bf16 (|dD| <= 2^-9 |D|, and a dlogit
    # row has sum_v |D_iv| <= 2 s), then grad_W is rounded to bf16, so per column h
    # |sum_v grad_W[v,h]| <= 2^-8 s sum_i |x_ih| + 2^-9 sum_v |grad_W[v,h]| (+ fp32 sums).
    assert torch.isfinite(gx).all() and torch.isfinite(gW).all()
    colsum = gW.double().sum(dim=0).abs()
    xf_abs = torch.from_numpy(np.abs(widen(x, dt)).sum(axis=0)).cuda()
    bound = 2.0 ** -8 / N * xf_abs + 2.0 ** -9 * gW.double().abs().sum(dim=0)
    assert bool((colsum <= 1.5 * bound + 1e-12).all()), f"sum_v grad_W exceeds its rounding bound"

    xf, Wf = widen(x, dt), widen(W, dt)
    lse_h, zt_h = to_f64(lse), to_f64(zt)

    # the oracle's full forward: every token's lse and target logit, and the loss
    t0 = time.perf_counter()
    ref_loss, ref_lse, ref_zt = oracle.forward(xf, Wf, t, "mean")
    note(f"[full] {name} oracle forward {time.perf_counter() - t0:.1f} s")
    assert abs(loss.item() - ref_loss) <= tol["loss_rel"] * abs(ref_loss), (loss.item(), ref_loss)
    np.testing.assert_allclose(lse_h, ref_lse, rtol=0, atol=tol["lse_atol"] * max(1.0, np.abs(ref_lse).max()))
    np.testing.assert_allclose(zt_h, ref_zt, rtol=0, atol=tol["lse_atol"] * max(1.0, np.abs(ref_zt).max()))

    # grad_x rows of sampled tokens: normalised by the largest |grad_x| of those rows
    g = np.random.Generator(np.random.PCG64(1))
    rows = np.unique(np.concatenate([[0, N - 1], g.choice(N, 30, replace=False)]))
    r_gx = oracle.grad_x_rows(xf, Wf, t, rows, "mean")
    d = np.abs(to_f64(gx[torch.from_numpy(rows).cuda()]) - r_gx).max() / np.abs(r_gx).max()
    assert d <= gbar, f"grad_x rows: {d:.3e}"

    # grad_W rows: targets of sampled tokens (their one-hot terms), the first and
    # last entry (edge tiles) and random entries, from the oracle's own lse
    t0 = time.perf_counter()
    vrows = np.unique(np.concatenate([[0, V - 1], t[rows[:12]], g.choice(V, 20, replace=False)]))
    r_gW = oracle.grad_w_rows(xf, Wf, t, vrows, ref_lse, "mean")
    got = to_f64(gW[torch.from_numpy(vrows).cuda()])
    d = np.abs(got - r_gW).max() / np.abs(r_gW).max()
    note(f"[full] {name} grad_W rows {time.perf_counter() - t0:.1f} s, err {d:.2e}")
    assert d <= gbar, f"grad_W rows: {d:.3e}"
    # the target rows on their own, normalised by their own largest entry
    tr = np.isin(vrows, t[rows[:12]])
    d_t = np.abs(got[tr] - r_gW[tr]).max() / np.abs(r_gW[tr]).max()
    assert d_t <= gbar, f"grad_W target rows: {d_t:.3e}"
