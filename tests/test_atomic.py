"""flce_backward_atomic (float32 atomic accumulation of both gradients, one
fused kernel per token tile x vocabulary tile pair; kept for comparison with the
bounded dlogit panels) against the float64 oracle, element by element."""
import numpy as np
import pytest
import torch

import oracle
from lm_head_linear_tiled_amd.inputs import WORKLOADS, make_inputs, widen
from tests.gpu_util import assert_grad_close, note, to_dev, to_f64

pytestmark = pytest.mark.gpu


def check(gpu, N, H, V, dtype, reduction, seed, grad_loss=1.0, t=None):
    note(f"[atomic] N={N} H={H} V={V} {dtype} {reduction} seed={seed}")
    x, W, t0 = make_inputs(N, H, V, dtype, seed=seed)
    t = t0 if t is None else np.asarray(t, dtype=np.int64)
    xd, Wd, td = to_dev(x, dtype), to_dev(W, dtype), torch.from_numpy(t).cuda()
    _, lse = gpu.flce_forward(xd, Wd, td, reduction)
    gl = torch.tensor([grad_loss], dtype=torch.float32, device="cuda")
    gx, gW = gpu.flce_backward_atomic(xd, Wd, td, lse, gl, reduction)
    torch.cuda.synchronize()
    xf, Wf = widen(x, dtype), widen(W, dtype)
    rgx, rgW = oracle.backward(xf, Wf, t, reduction, grad_loss)
    assert_grad_close(to_f64(gx), rgx, dtype, "grad_x")
    assert_grad_close(to_f64(gW), rgW, dtype, "grad_W")
    return gx, gW


@pytest.mark.parametrize("name,reduction", [("tiny", "mean"), ("ragged", "sum"), ("ragged", "mean")])
def test_atomic_workloads(gpu, name, reduction):
    w = WORKLOADS[name]
    check(gpu, w.N, w.H, w.V, w.dtype, reduction, seed=0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_atomic_multi_tile_ragged(gpu, dtype, reduction):
    """Several token and vocabulary tiles, the last of each ragged, a ragged
    hidden size (edge paths of every contraction), and more pairs than one launch
    of 256 workgroups holds (V = 70000: 274 vocabulary tiles x 2 token tiles)."""
    check(gpu, 300, 264, 70000, dtype, reduction, seed=61, grad_loss=0.7)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_atomic_all_targets_equal(gpu, dtype):
    """Every token has the same target: the one-hot terms all land in one grad_W row."""
    check(gpu, 512, 128, 3000, dtype, "sum", seed=62, t=np.full(512, 1234))


def test_atomic_matches_panels(gpu):
    """Same inputs through the default backward: the two agree to the bf16 bar."""
    N, H, V = 1000, 512, 20000
    x, W, t = make_inputs(N, H, V, "bf16", seed=63)
    xd, Wd, td = to_dev(x, "bf16"), to_dev(W, "bf16"), torch.from_numpy(t).cuda()
    _, lse = gpu.flce_forward(xd, Wd, td, "mean")
    gl = torch.ones(1, device="cuda")
    a = gpu.flce_backward_atomic(xd, Wd, td, lse, gl, "mean")
    b = gpu.flce_backward(xd, Wd, td, lse, gl, "mean")
    torch.cuda.synchronize()
    for ga, gb, name in ((a[0], b[0], "grad_x"), (a[1], b[1], "grad_W")):
        assert torch.isfinite(ga).all()
        d = (ga.float() - gb.float()).abs().max().item() / gb.float().abs().max().item()
        assert d <= 1e-2, f"{name}: {d:.3e}"
