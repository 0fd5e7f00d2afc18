"""The token-chunked backward (each chunk's dlogits over the whole vocabulary)
against the CPU oracle and against the default bounded-panel backward."""
import numpy as np
import pytest
import torch

import oracle
from lm_head_linear_tiled_amd.inputs import make_inputs, widen
from tests.gpu_util import assert_grad_close, note, to_dev, to_f64

pytestmark = pytest.mark.gpu


def run(gpu, N, H, V, dtype, reduction, chunk, seed, grad_loss=1.0):
    note(f"[chunked] N={N} H={H} V={V} {dtype} {reduction} chunk={chunk} seed={seed}")
    x, W, t = make_inputs(N, H, V, dtype, seed=seed)
    xd, Wd, td = to_dev(x, dtype), to_dev(W, dtype), torch.from_numpy(t).cuda()
    loss, lse = gpu.flce_forward(xd, Wd, td, reduction)
    gl = torch.tensor([grad_loss], dtype=torch.float32, device="cuda")
    gx, gW = gpu.flce_backward_chunked(xd, Wd, td, lse, gl, reduction, chunk_tokens=chunk)
    torch.cuda.synchronize()
    return x, W, t, (xd, Wd, td, lse, gl), to_f64(gx), to_f64(gW)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("reduction", ["mean", "sum"])
@pytest.mark.parametrize("chunk", [1, 256, 300, 100000])
def test_chunked_matches_oracle(gpu, dtype, reduction, chunk):
    """Several chunks with a ragged last one (chunk 1 rounds up to 256; 300 to 512),
    and a single chunk of every token."""
    N, H, V = 700, 200, 1500
    x, W, t, _, gx, gW = run(gpu, N, H, V, dtype, reduction, chunk, seed=11, grad_loss=0.8)
    rgx, rgW = oracle.backward(widen(x, dtype), widen(W, dtype), t, reduction, 0.8)
    assert_grad_close(gx, rgx, dtype, "grad_x")
    assert_grad_close(gW, rgW, dtype, "grad_W")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunked_agrees_with_panels(gpu, dtype):
    """Same gradients, to rounding, as the default backward on a shape with several
    vocabulary panels and several token chunks."""
    N, H, V = 1100, 256, 20000
    _, _, _, dev, gx, gW = run(gpu, N, H, V, dtype, "mean", 512, seed=12)
    dx, dW = gpu.flce_backward(*dev, "mean")
    torch.cuda.synchronize()
    assert_grad_close(gx, to_f64(dx), dtype, "grad_x vs panels")
    assert_grad_close(gW, to_f64(dW), dtype, "grad_W vs panels")


def test_chunked_deterministic(gpu):
    _, _, _, dev, gx, gW = run(gpu, 600, 128, 5000, "bf16", "sum", 256, seed=13)
    gx2, gW2 = gpu.flce_backward_chunked(*dev, "sum", chunk_tokens=256)
    torch.cuda.synchronize()
    assert np.array_equal(gx, to_f64(gx2)) and np.array_equal(gW, to_f64(gW2))
